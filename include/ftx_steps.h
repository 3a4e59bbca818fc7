/*
 * ftx_steps.h -- step-level entry points of the ftx encoder forward.
 *
 * Each call enqueues ONE kernel of the forward on `stream` (a hipStream_t, NULL = the
 * default stream) and returns without waiting.  They are the same kernels ftx_forward
 * launches, exported so that each step can be checked and timed on its own.  All tensor
 * pointers are device pointers, row-major, 16-byte aligned unless noted; outputs must
 * not overlap inputs.  Shape arguments follow ftx.h: B batch, S padded sequence length
 * (multiple of 32, <= FTX_MAX_SEQ_LEN), n heads, d size per head (32 or 64), H = n d,
 * T = B S tokens.  Arguments out of range -> FTX_ERR_INVALID_ARG; valid but unsupported
 * shapes -> FTX_ERR_UNSUPPORTED; a failed launch -> FTX_ERR_DEVICE.
 *
 * Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
 * section "Faster Transformer 优化原理": per layer, matrix multiplies plus custom kernels
 * that are mostly element-wise work on the matrix-multiply results, with LayerNorm and
 * SoftMax row reductions kept in float.
 */
#ifndef FTX_STEPS_H_
#define FTX_STEPS_H_

#include "ftx.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Dense projection on matrix cores: C[M][N] = A[M][K] W + bias, where the weight is given
 * TRANSPOSED, w_t[N][K] (row n holds column n of W).  bias [N] or NULL (no bias).
 * gelu != 0 applies the tanh GELU to every output element after the bias.
 * M >= 1; N, K >= 8 and multiples of 8.  fp32 accumulation in every dtype.
 * (The attention-output projection, the first FFN projection with its GELU epilogue,
 * and the second FFN projection.)  K <= 2^20, else FTX_ERR_UNSUPPORTED. */
ftx_status ftx_step_linear(ftx_dtype dtype, int M, int N, int K, const void *a,
                           const void *w_t, const void *bias, int gelu, void *c,
                           void *stream);

/* Fused Q/K/V projection with the bias + head-split epilogue:
 *   x [T][H], w_qkv_t [3H][H] (rows 0..H-1 = Wq^T, H..2H-1 = Wk^T, 2H..3H-1 = Wv^T),
 *   b_qkv [3H] (bq | bk | bv) ->
 *   q [B][n][S][d], k [B][n][S][d], v_t [B][n][d][S] (V stored transposed per head). */
ftx_status ftx_step_qkv_projection(ftx_dtype dtype, int B, int S, int n, int d,
                                   const void *x, const void *w_qkv_t, const void *b_qkv,
                                   void *q, void *k, void *v_t, void *stream);

/* Standalone bias + head split/transpose (the projection's epilogue as its own kernel):
 *   qkv [T][3H] (projection output without bias), b_qkv [3H] -> q, k, v_t as above. */
ftx_status ftx_step_bias_qkv_split(ftx_dtype dtype, int B, int S, int n, int d,
                                   const void *qkv, const void *b_qkv, void *q, void *k,
                                   void *v_t, void *stream);

/* Fused attention: per (b, h), scores Q K^T / sqrt(d), softmax over keys
 * j < len_b (keys beyond get probability 0; row max and sum in fp32), context P V,
 * written with heads merged: ctx[T][H] with ctx[b*S+i][h*d+e].
 *   q, k [B][n][S][d], v_t [B][n][d][S]; seq_lens [B] int32 (clamped to [1, S]) or NULL. */
ftx_status ftx_step_attention(ftx_dtype dtype, int B, int S, int n, int d, const void *q,
                              const void *k, const void *v_t, const int32_t *seq_lens,
                              void *ctx, void *stream);

/* Q/K/V projection and attention in one kernel, for S = 32, 64, 128 or 256, d = 64 (or 32
 * with an even n) and a 16-bit dtype (FTX_FP16 or FTX_BF16; other shapes ->
 * FTX_ERR_UNSUPPORTED): x [B*S][H] ->
 * ctx [B*S][H] with ctx[b*S+i][h*64+e], the result of ftx_step_qkv_projection followed
 * by ftx_step_attention, except that the weight rows are ordered per head:
 *   w_qkv_t [3H][H], rows 3dh .. 3dh+d-1 = rows h*d .. h*d+d-1 of Wq^T, the next d of Wk^T,
 *   the next d of Wv^T (h = 0 .. n-1); b_qkv [3H] in the same order;
 *   seq_lens [B] int32 (clamped to [1, S]) or NULL; causal != 0: query i also ignores keys
 *   j > i (a decoder's self-attention).
 * Q, K and V stay on chip: each 256 x 192 output tile (256/S whole sequences, 64/d heads;
 * 128 x 192 tiles when the 256-row grid has at most half as many tiles as the GPU has CUs
 * and S <= 128)
 * is attended in the projection's epilogue.  ctx must not overlap x or w_qkv_t
 * (FTX_ERR_INVALID_ARG). */
ftx_status ftx_step_qkv_attention(ftx_dtype dtype, int B, int S, int n, int d, const void *x,
                                  const void *w_qkv_t, const void *b_qkv,
                                  const int32_t *seq_lens, int causal, void *ctx, void *stream);

/* The same attention with separate query and key lengths (cross-attention: queries of one
 * sequence over the keys of another) and an optional causal mask (a decoder's
 * self-attention: query i ignores keys j > i; needs Sq == Sk):
 *   q [B][n][Sq][d], k [B][n][Sk][d], v_t [B][n][d][Sk]; key_lens [B] int32 (keys
 *   j >= key_lens[b] get probability 0; clamped to [1, Sk]) or NULL; ctx [B][Sq][n*d].
 * Sq, Sk multiples of 32 in [32, 512]. */
ftx_status ftx_step_masked_attention(ftx_dtype dtype, int B, int Sq, int Sk, int n, int d,
                                     const void *q, const void *k, const void *v_t,
                                     const int32_t *key_lens, int causal, void *ctx,
                                     void *stream);

/* Bias + residual + LayerNorm (after the attention block and after the FFN), one row of
 * `cols` per token:
 *   y = LN(x + a + bias; gamma, beta) with epsilon FTX_LN_EPSILON, biased variance,
 *   statistics in fp32.  x, a, y [rows][cols]; bias, gamma, beta [cols].
 *   y may alias x or a (each row is read completely before it is written).
 *   cols a multiple of 4 and <= FTX_MAX_HIDDEN. */
ftx_status ftx_step_bias_residual_layernorm(ftx_dtype dtype, int rows, int cols,
                                            const void *x, const void *a, const void *bias,
                                            const void *gamma, const void *beta, void *y,
                                            void *stream);

/* Standalone bias + GELU (the first FFN projection's epilogue as its own kernel):
 * g = gelu(u + bias) element-wise, u, g [rows][cols] (g may alias u), bias [cols]; cols a multiple of 8. */
ftx_status ftx_step_bias_gelu(ftx_dtype dtype, int rows, int cols, const void *u,
                              const void *bias, void *g, void *stream);

/* Matrix transpose out[cols][rows] = in[rows][cols]^T (the weight repacking of
 * ftx_set_weights).  No alignment requirement. */
ftx_status ftx_step_transpose(ftx_dtype dtype, int rows, int cols, const void *in, void *out,
                              void *stream);

/* The launch plan of an M x N x K projection (ftx_step_linear and the encoder's
 * projections) on a device with `cus` compute units: the block tile tile_m x tile_n and the
 * number of ranges K is split into (1 = no split).  sums_partials != 0: the plan of a
 * projection whose split-K partials the LayerNorm after it sums (the attention-output and
 * FFN-out projections), else of one that finishes them with its own reduction.  The handles
 * and the step entry points read `cus` from the device (hipGetDeviceProperties) and plan
 * with it; the article tunes launch configurations to the shape (section "Faster
 * Transformer 优化原理").  Host arithmetic only, no HIP call: usable without a GPU.
 * M, N, K, cus >= 1 and tile_m, tile_n, splits non-NULL (host pointers), else
 * FTX_ERR_INVALID_ARG. */
ftx_status ftx_plan_linear(ftx_dtype dtype, int M, int N, int K, int cus, int sums_partials,
                           int *tile_m, int *tile_n, int *splits);

#ifdef __cplusplus
}
#endif

#endif /* FTX_STEPS_H_ */
