/* ftx decoder: a Transformer decoder forward on one MI355X (gfx950), the C ABI.
 *
 * Source: the Faster Transformer article ("有钱任性：英伟达训练80亿参数量GPT-2，1475块V100
 * 53分钟训练BERT", cloud.tencent.com/developer/article/1490359), section
 * "什么是 Faster Transformer", which lists decoder support as a later roadmap item without
 * describing it.  This library reads it as the encoder layer of the same section with a
 * causal mask on the self-attention and a cross-attention sub-layer over the encoder output
 * (the memory), each sub-layer followed by residual + LayerNorm (post-LN):
 *
 *   Y1  = LN1(X  + SelfAttn_causal(X) Wo + bo)        query i sees decoder keys j <= i
 *   Y2  = LN2(Y1 + CrossAttn(Y1, M) Wo2 + bo2)        memory keys j >= mem_lens[b] ignored
 *   out = LN3(Y2 + gelu(Y2 W1 + b1) W2 + b2)
 *
 * with everything else as the encoder of ftx.h: scores scaled by 1/sqrt(d), LayerNorm with
 * the biased variance and epsilon FTX_LN_EPSILON, tanh GELU, F = 4H, weights [in][out],
 * fp32 accumulation and statistics, and the same dtype modes (bf16 keeps the un-normalised
 * LayerNorm inputs in fp32).  Every decoder row, padded or not, is computed; by causality
 * rows past a sequence's own length never reach earlier rows.
 *
 * Conventions are those of ftx.h: device pointers, 16-byte aligned, row-major; calls
 * return an ftx_status and leave a message for ftx_last_error(); a handle is not
 * thread-safe and its forwards must not overlap in time.
 */
#ifndef FTX_DECODER_H_
#define FTX_DECODER_H_

#include "ftx.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ftx_decoder ftx_decoder;

/* One decoder layer's weights, device pointers in the run dtype, matrices [in][out]:
 * causal self-attention (w_q, w_k, w_v, w_o [H][H]; biases [H]; LayerNorm 1),
 * cross-attention (w_q2 on the decoder states, w_k2 and w_v2 on the memory, w_o2, all
 * [H][H]; biases [H]; LayerNorm 2), feed-forward (w_ffn1 [H][F], b_ffn1 [F],
 * w_ffn2 [F][H], b_ffn2 [H]; LayerNorm 3).  Copied (and repacked) by
 * ftx_decoder_set_weights; the caller keeps ownership. */
typedef struct {
  const void *w_q, *b_q, *w_k, *b_k, *w_v, *b_v, *w_o, *b_o, *ln1_gamma, *ln1_beta;
  const void *w_q2, *b_q2, *w_k2, *b_k2, *w_v2, *b_v2, *w_o2, *b_o2, *ln2_gamma, *ln2_beta;
  const void *w_ffn1, *b_ffn1, *w_ffn2, *b_ffn2, *ln3_gamma, *ln3_beta;
} ftx_decoder_layer_weights;

/* Create a decoder for batch_size sequences of tgt_len decoder positions attending to a
 * memory of mem_len positions; head_num x size_per_head (32 or 64) heads, num_layers
 * layers.  tgt_len and mem_len: any length in [1, FTX_MAX_SEQ_LEN]; a length that is not a
 * multiple of 32 is padded internally (one 2-D copy in per forward for the input and for
 * the memory, one out for the output; cross-attention keys are limited to mem_len).
 * Allocates the weights and workspace on the current device.
 * Errors: FTX_ERR_INVALID_ARG (out == NULL, values < 1, unknown dtype),
 * FTX_ERR_UNSUPPORTED (sizes outside the ranges above, not a gfx950 device),
 * FTX_ERR_OUT_OF_MEMORY, FTX_ERR_DEVICE. */
ftx_status ftx_decoder_create(int batch_size, int tgt_len, int mem_len, int head_num,
                              int size_per_head, int num_layers, ftx_dtype dtype,
                              ftx_decoder **out);

/* Copy layer `layer`'s weights (enqueued on `stream`, then synchronised).  Every pointer
 * must be non-NULL device memory.  Errors: FTX_ERR_INVALID_ARG, FTX_ERR_DEVICE. */
ftx_status ftx_decoder_set_weights(ftx_decoder *dec, int layer,
                                   const ftx_decoder_layer_weights *w, void *stream);

/* Enqueue the forward on `stream`:
 *   input    [B][tgt_len][H] decoder states, left unmodified;
 *   memory   [B][mem_len][H] encoder output, left unmodified;
 *   mem_lens [B] int32 valid memory lengths (clamped to [1, mem_len]) or NULL (all valid);
 *   output   [B][tgt_len][H], must not overlap input or memory.
 * Errors: FTX_ERR_INVALID_ARG (NULL / misaligned / overlapping / host pointers),
 * FTX_ERR_NOT_READY (a layer has no weights), FTX_ERR_DEVICE (launch failure). */
ftx_status ftx_decoder_forward(ftx_decoder *dec, const void *input, const void *memory,
                               const int32_t *mem_lens, void *output, void *stream);

/* Options a decoder takes (others -> FTX_ERR_INVALID_ARG):
 *   FTX_OPT_KERNEL_TIMING (value != 0: an event pair around every launch of the following
 *     forwards, read back by ftx_decoder_kernel_times);
 *   FTX_OPT_FUSED_ATTENTION (default 1): as for the encoder (ftx.h), for the causal
 *     self-attention: with a 16-bit dtype, size_per_head 64 (or 32 with an even head_num)
 *     and an internal decoder length of 32, 64, 128 or 256, the self Q/K/V projection
 *     attends each of its 256 x 192 (or 128 x 192) tiles in its epilogue (step class
 *     FTX_DEC_STEP_SELF_QKV_ATTENTION); 0 never; 1 when batch*len >= 256 (len: the internal
 *     decoder length) and the 256-row grid has at least 64 tiles; 2 whenever the shape
 *     fits; other
 *     values -> FTX_ERR_INVALID_ARG. */
ftx_status ftx_decoder_set_option(ftx_decoder *dec, ftx_option option, int value);

/* Step classes of the decoder's per-step timing. */
typedef enum {
  FTX_DEC_STEP_SELF_QKV_GEMM = 0,  /* Q/K/V projection with bias + head split */
  FTX_DEC_STEP_SELF_ATTENTION = 1, /* causal attention */
  FTX_DEC_STEP_SELF_OUT_GEMM = 2,  /* self-attention output projection */
  FTX_DEC_STEP_LN1 = 3,
  FTX_DEC_STEP_CROSS_Q_GEMM = 4,   /* cross-attention query projection */
  FTX_DEC_STEP_CROSS_KV_GEMM = 5,  /* cross-attention key/value projection of the memory */
  FTX_DEC_STEP_CROSS_ATTENTION = 6,
  FTX_DEC_STEP_CROSS_OUT_GEMM = 7,
  FTX_DEC_STEP_LN2 = 8,
  FTX_DEC_STEP_FFN1_GEMM = 9,      /* with bias + GELU */
  FTX_DEC_STEP_FFN2_GEMM = 10,
  FTX_DEC_STEP_LN3 = 11,
  FTX_DEC_STEP_SELF_QKV_ATTENTION = 12, /* Q/K/V projection with the causal attention inside */
  FTX_DEC_NUM_STEPS = 13
} ftx_decoder_step;

/* Synchronize the events recorded since the last call and return, per step class, the
 * summed duration in milliseconds (ms[FTX_DEC_NUM_STEPS]) and the number of launches
 * (counts[FTX_DEC_NUM_STEPS]); then reset.  Either array may be NULL. */
ftx_status ftx_decoder_kernel_times(ftx_decoder *dec, double *ms, int64_t *counts);

/* Free the handle (waits for the device first).  NULL is accepted. */
ftx_status ftx_decoder_destroy(ftx_decoder *dec);

#ifdef __cplusplus
}
#endif

#endif /* FTX_DECODER_H_ */
