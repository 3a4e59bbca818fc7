/*
 * ftx.h -- C ABI of the ftx BERT-style Transformer encoder forward for AMD MI355X (gfx950).
 *
 * What it computes.  The forward pass of a multi-layer BERT-style Transformer encoder,
 * the part the Faster Transformer article ("有钱任性：英伟达训练80亿参数量GPT-2，1475块V100
 * 53分钟训练BERT", cloud.tencent.com/developer/article/1490359) describes in its section
 * "什么是 Faster Transformer": a forward-only encoder whose network structure is fixed by
 * the attention head count and the size of each head, called with a batch size and a
 * maximum sentence length, in an FP16 or an FP32 compute mode, behind a C++ API.  Each
 * layer (section "Faster Transformer 优化原理") is matrix multiplies plus element-wise
 * work on their results: bias add, SoftMax, GELU and Layer Normalization.
 *
 * The layer, per sequence b with valid length len_b (post-LayerNorm form):
 *   Q = X Wq + bq, K = X Wk + bk, V = X Wv + bv        head h = columns h*d .. h*d+d-1
 *   P = softmax over keys j < len_b of (Q_h K_h^T / sqrt(d)); keys j >= len_b get 0
 *   C = P V (heads merged back)
 *   Y1 = LN(X + C Wo + bo; gamma1, beta1)
 *   X' = LN(Y1 + gelu(Y1 W1 + b1) W2 + b2; gamma2, beta2)
 * with LN(z) = gamma (z - mean) / sqrt(var + FTX_LN_EPSILON) + beta (biased variance),
 * gelu(u) = u/2 (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3))), and FFN width 4 * hidden.
 * Every query row, padded or not, is computed; the output covers all B x S positions.
 *
 * Precision.  FTX_FP32: fp32 storage and arithmetic.  FTX_FP16 / FTX_BF16: storage in the
 * 16-bit format, every matrix product accumulated in fp32, softmax and LayerNorm
 * statistics in fp32; activations between kernels are stored in the 16-bit format, except
 * that FTX_BF16 keeps what enters a LayerNorm un-normalised in fp32 -- the residual Y1 (the
 * first LayerNorm's output, added back before the second) and the attention-output and
 * FFN-output projections -- because bf16's rounding of those (up to 7.8e-3 at |v| in
 * [2, 4)) reaches the layer output almost unattenuated.  With the first LayerNorm folded
 * (FTX_OPT_FOLD_LAYERNORM) its un-normalised input Z1 takes Y1's place: stored in the 16-bit
 * format as the FFN-in operand (and, for FTX_BF16, in fp32 as the second LayerNorm's
 * residual), with its row statistics in fp32.
 *
 * Conventions.
 *  - All tensors are row-major.  All tensor pointers are DEVICE pointers on the device
 *    that was current at ftx_encoder_create.  Weights are [in][out] (y = x W + b).
 *  - Every function returns ftx_status; no C++ exception crosses this boundary.
 *    ftx_last_error() returns a text description of the last failure on this thread.
 *  - A handle is not thread-safe and its forwards must not overlap in time (they share
 *    the handle's workspace).  Different handles are independent.
 */
#ifndef FTX_H_
#define FTX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FTX_LN_EPSILON 1e-6f
#define FTX_MAX_SEQ_LEN 512
#define FTX_MAX_HIDDEN 4096

typedef struct ftx_encoder ftx_encoder; /* opaque; owned by the library */

typedef enum { FTX_FP32 = 0, FTX_FP16 = 1, FTX_BF16 = 2 } ftx_dtype;

typedef enum {
  FTX_OK = 0,
  FTX_ERR_INVALID_ARG = 1,   /* NULL / misaligned / aliased pointer, value out of range */
  FTX_ERR_UNSUPPORTED = 2,   /* a valid value this library does not implement */
  FTX_ERR_OUT_OF_MEMORY = 3, /* device allocation failed */
  FTX_ERR_DEVICE = 4,        /* a HIP runtime call failed (no device, launch failure...) */
  FTX_ERR_NOT_READY = 5      /* forward called before every layer's weights were set */
} ftx_status;

/* One layer's weights, every tensor in the handle's dtype, device pointers.
 * H = head_num * size_per_head, F = 4 H. */
typedef struct {
  const void *w_q, *b_q;             /* [H][H], [H] */
  const void *w_k, *b_k;             /* [H][H], [H] */
  const void *w_v, *b_v;             /* [H][H], [H] */
  const void *w_o, *b_o;             /* [H][H], [H] */
  const void *ln1_gamma, *ln1_beta;  /* [H], [H] */
  const void *w_ffn1, *b_ffn1;       /* [H][F], [F] */
  const void *w_ffn2, *b_ffn2;       /* [F][H], [H] */
  const void *ln2_gamma, *ln2_beta;  /* [H], [H] */
} ftx_layer_weights;

/* Create an encoder for a fixed shape: the four runtime parameters of the article's
 * section "什么是 Faster Transformer" (head count, size per head, batch size, maximum
 * sentence length) plus the layer count and the storage dtype.
 *   batch_size >= 1; seq_len in [1, FTX_MAX_SEQ_LEN], any value (the article fixes it at
 *   32/64/128 and names arbitrary lengths as its next feature: lengths that are not a
 *   multiple of 32 are padded to one inside the handle, with an input and an output copy
 *   per forward, and padding keys never take part in attention);
 *   size_per_head in {32, 64}; head_num >= 1 with head_num*size_per_head <= FTX_MAX_HIDDEN;
 *   num_layers >= 1; out != NULL (host pointer; receives the handle).
 * Non-positive values, an unknown dtype or out == NULL -> FTX_ERR_INVALID_ARG (no HIP call
 * is made).  Positive values outside the supported set -> FTX_ERR_UNSUPPORTED.
 * Allocates the workspace and the weight storage on the current device (hipMalloc):
 * about (10 B S H + L (12 H^2 + 13 H)) elements (plus 2 B S H fp32 values for FTX_BF16,
 * and 2 B S H elements when seq_len is not a multiple of 32; S = seq_len rounded up to 32). */
ftx_status ftx_encoder_create(int batch_size, int seq_len, int head_num, int size_per_head,
                              int num_layers, ftx_dtype dtype, ftx_encoder **out);

/* Copy one layer's weights into the handle (repacking them for the kernels: Wq|Wk|Wv
 * fused and every matrix stored transposed, [out][in]).  The copies are enqueued on
 * `stream` (a hipStream_t; NULL = the default stream), which is then synchronized, so
 * the caller may free its buffers on return.  layer in [0, num_layers); w != NULL and
 * every pointer in it non-NULL, else FTX_ERR_INVALID_ARG. */
ftx_status ftx_set_weights(ftx_encoder *enc, int layer, const ftx_layer_weights *w,
                           void *stream);

/* Run the L-layer forward on `stream` (asynchronous: returns once enqueued).
 *   input    [B][S][H] device, 16-byte aligned, left unmodified;
 *   seq_lens [B] int32 device valid lengths, or NULL for "no padding".  Values are
 *            clamped to [1, seq_len] on the device (the host cannot read them);
 *   output   [B][S][H] device, 16-byte aligned, must not overlap input.
 * The caller keeps input, seq_lens and output alive until the stream passes the call.
 * FTX_ERR_NOT_READY if some layer has no weights. */
ftx_status ftx_forward(ftx_encoder *enc, const void *input, const int32_t *seq_lens,
                       void *output, void *stream);

/* For callers that cannot allocate device memory while they run (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): ftx_forward with every
 * intermediate tensor of the forward -- Q, K, V^T, the attention context, the projection
 * outputs, the FFN hidden layer, the fp32 copies of FTX_BF16, the padded copies of a
 * seq_len that is not a multiple of 32, the split-K partial products -- in the library's
 * static scratch instead of the handle's workspace.  Same arguments, same kernels and
 * launch plans, so the same result as ftx_forward, bit for bit.
 *   The scratch is a fixed array of FTX_STATIC_SCRATCH_BYTES of device memory per GPU (the
 *   library's code object holds it; each GPU the library runs on keeps its copy until the
 *   process ends).  A handle whose workspace is larger -> FTX_ERR_UNSUPPORTED, nothing
 *   enqueued (BERT-base fp16 at seq_len 32 fits up to about 100 sequences).
 *   Allocates nothing: no hipMalloc/hipFree, no allocating library call; the padded input
 *   copy is cleared with a kernel, not hipMemsetAsync, so the call can be captured.
 *   FTX_OPT_GRAPH does not apply (the caller captures if it wishes); FTX_OPT_KERNEL_TIMING
 *   does.
 *   Every call on one GPU, from any handle or thread, uses that GPU's one scratch array and
 *   leaves its contents behind: calls that overlap in time on one GPU (other streams, other
 *   threads) race and give wrong results.  Order them on one stream or synchronize between
 *   them.  Other errors as ftx_forward. */
#define FTX_STATIC_SCRATCH_BYTES (64u << 20)
ftx_status ftx_forward_static_workspace(ftx_encoder *enc, const void *input,
                                        const int32_t *seq_lens, void *output, void *stream);

/* Free the handle and its device memory (synchronizes the device first).  NULL -> FTX_OK. */
ftx_status ftx_destroy(ftx_encoder *enc);

/* Static text for a status code. */
const char *ftx_status_string(ftx_status status);

/* Description of the most recent failure on the calling thread ("" if none). */
const char *ftx_last_error(void);

/* ---------------------------------------------------------------------------------
 * Options of a handle.
 *   FTX_OPT_FUSED_EPILOGUES (default 1): 1 = bias+QKV split and bias+GELU run inside the
 *     projection kernels' epilogues; 0 = they run as standalone element-wise kernels after
 *     plain projections (two launches per layer more: 9 instead of 7 with the attention as
 *     its own kernel and neither LayerNorm folded; the fused attention and the LayerNorm
 *     fold need 1 and take a layer down to 5).  Same result up to rounding order.
 *   FTX_OPT_KERNEL_TIMING (default 0): 1 = every forward records a HIP event pair around
 *     each launch, on the forward's stream, and accumulates per-step durations that
 *     ftx_kernel_times() returns.
 *   FTX_OPT_GRAPH (default 0): 1 = ftx_forward replays one HIP graph of the whole forward
 *     (the small-batch latency path: the article's small-batch bottleneck is kernel launch
 *     count, section "Faster Transformer 优化原理").  The graph is captured, on a stream
 *     the handle owns, at the first forward for a given (input, seq_lens, output) triple and
 *     replayed on the caller's stream (the default stream included) while those three
 *     pointers stay the same; other pointers cause a new capture.  Weights may change
 *     between forwards (they live in handle memory the graph reads).  Ignored while
 *     FTX_OPT_KERNEL_TIMING is on.
 *   FTX_OPT_FUSED_ATTENTION (default 1): for a padded length S of 32, 64, 128 or 256 (seq_len
 *     up to 256, rounded up to a multiple of 32 that is one of those), size_per_head 64 (or
 *     32 with an even head_num) and a 16-bit dtype, the Q/K/V projection and the attention
 *     run as one kernel that attends each 256 x 192 projection tile (256/S whole sequences,
 *     64/size_per_head heads; 128-row tiles when the 256-row grid has at most half as many
 *     tiles as the GPU has CUs, or more tiles than CUs with its last round at most half
 *     full) in its epilogue, so Q, K and V never reach memory
 *     (ftx_step_qkv_attention).  0 = never; 1 = when batch*S >= 256 and the 256-row grid
 *     has at least 64 tiles (ceil(batch*S/256) * 3*hidden/192), else the separate kernels;
 *     2 = whenever the shape fits.  Needs FTX_OPT_FUSED_EPILOGUES = 1.
 *     Values outside 0..2 -> FTX_ERR_INVALID_ARG.
 *   FTX_OPT_FOLD_LAYERNORM (default 1): for fp16/bf16, hidden size 768 or 1024 and a batch at
 *     which the attention-output and FFN projections do not split K, the first LayerNorm of
 *     each layer is folded into the first FFN projection (its gamma into that projection's
 *     weights, its beta into the bias; the row statistics come from the attention-output
 *     projection's epilogue), and the second LayerNorm rebuilds its residual from the same
 *     statistics: one launch per layer fewer (no FTX_STEP_LN1).  Same result up to rounding
 *     order.  0 = the LayerNorm runs as its own step.  Needs FTX_OPT_FUSED_EPILOGUES = 1.
 *     When the FFN intermediate (batch*S x 4*hidden) exceeds 160 MB the folded path runs
 *     FFN-in, FFN-out and the second LayerNorm in row chunks, one launch each per chunk.
 *   FTX_OPT_PREFETCH_WEIGHTS (default 1): on the folded path, a kernel that only reads the
 *     layer's second FFN weight matrix (FTX_STEP_PREFETCH) runs just before the second FFN
 *     projection, so that the projection finds W2 in the last-level cache instead of HBM.
 *     1 = where that projection runs on 128-row tiles, at least 1.5 tiles per CU (BERT-base
 *     from 6144 to 10240 rows, BERT-large at 8192); 2 = before every second FFN
 *     projection of the folded path; 0 = never.  One launch per layer more where it runs.
 *     Writes nothing: the result is the same bit for bit.  Values outside 0..2 ->
 *     FTX_ERR_INVALID_ARG.
 * Unknown option -> FTX_ERR_INVALID_ARG. */
typedef enum {
  FTX_OPT_FUSED_EPILOGUES = 0,
  FTX_OPT_KERNEL_TIMING = 1,
  FTX_OPT_GRAPH = 2,
  FTX_OPT_FUSED_ATTENTION = 3,
  FTX_OPT_FOLD_LAYERNORM = 4,
  FTX_OPT_PREFETCH_WEIGHTS = 5
} ftx_option;
ftx_status ftx_set_option(ftx_encoder *enc, ftx_option option, int value);

/* Step classes of the per-step timing. */
typedef enum {
  FTX_STEP_QKV_GEMM = 0,        /* Q/K/V projection (with bias + head split when fused) */
  FTX_STEP_BIAS_QKV_SPLIT = 1,  /* bias + head split as its own kernel */
  FTX_STEP_ATTENTION = 2,       /* scores, masked softmax, context: one fused kernel */
  FTX_STEP_ATTN_OUT_GEMM = 3,   /* attention-output projection (folded LN1: + bias, residual,
                                   row statistics) */
  FTX_STEP_LN1 = 4,             /* bias + residual + LayerNorm after attention */
  FTX_STEP_FFN1_GEMM = 5,       /* first FFN projection (with bias + GELU when fused; folded
                                   LN1 applied in its epilogue) */
  FTX_STEP_BIAS_GELU = 6,       /* bias + GELU as its own kernel */
  FTX_STEP_FFN2_GEMM = 7,       /* second FFN projection */
  FTX_STEP_LN2 = 8,             /* bias + residual + LayerNorm after the FFN */
  FTX_STEP_QKV_ATTENTION = 9,   /* Q/K/V projection with the attention in its epilogue */
  FTX_STEP_PREFETCH = 10,       /* read of W2 into the last-level cache (FTX_OPT_PREFETCH_WEIGHTS) */
  FTX_NUM_STEPS = 11
} ftx_step;

/* Synchronize the events recorded since the last call and return, per step class, the
 * summed duration in milliseconds (ms[FTX_NUM_STEPS]) and the number of launches
 * (counts[FTX_NUM_STEPS]); then reset.  Either array may be NULL. */
ftx_status ftx_kernel_times(ftx_encoder *enc, double *ms, int64_t *counts);

#ifdef __cplusplus
}
#endif

#endif /* FTX_H_ */
