// Host-side launchers of the ftx kernels.  Arguments are validated by the C entry points
// before these are called; each launcher enqueues one kernel and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include "ftx.h"

namespace ftx {

// Compute units and XCDs (the dies the CUs are spread over, each with its own L2) of a
// device.  The GEMM planner sizes grids and split-K from the CU count (4 SIMDs per CU) and
// the kernels map block ids to tiles per XCD.
struct DeviceInfo {
  int cus;
  int xcds;
};
// The current device's counts, read from the HIP runtime (hipGetDeviceProperties,
// hipDeviceAttributeNumberOfXccs) on the first call for that device and cached; {1, 1} if
// the runtime cannot be asked (the launch that follows then fails on its own).
DeviceInfo device_info();

// out_f32: c is written as fp32 (16-bit dtypes, without GELU; ignored in fp32 mode).
// ws / ws_elems: fp32 workspace for split-K; a GEMM whose plan splits K runs unsplit when
// the workspace is missing or smaller than gemm_splitk_workspace() says.
hipError_t launch_linear(ftx_dtype dt, int M, int N, int K, const void* a, const void* w_t,
                         const void* bias, bool gelu, void* c, hipStream_t s,
                         bool out_f32 = false, float* ws = nullptr, size_t ws_elems = 0);

hipError_t launch_qkv_projection(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                 const void* w_qkv_t, const void* b_qkv, void* q, void* k,
                                 void* vt, hipStream_t s, float* ws = nullptr,
                                 size_t ws_elems = 0);

// Projection of x [B*S][H] onto `count` blocks of H columns (w_t [count*H][H], bias
// [count*H]) written head-split: block c goes to slot first + c of (q [B][n][S][d],
// k [B][n][S][d], vt [B][n][d][S]); first + count <= 3.  Slots not written may be NULL.
hipError_t launch_head_projection(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                  const void* w_t, const void* bias, int first, int count,
                                  void* q, void* k, void* vt, hipStream_t s,
                                  float* ws = nullptr, size_t ws_elems = 0);

// Whether the fused projection + attention below takes this shape: a 16-bit dtype, S (the
// padded length) 32, 64, 128 or 256, d = 64, or d = 32 with an even head count (a 192-column
// tile holds Q, K and V of 64 / d whole heads).
bool qkv_attention_fits(ftx_dtype dt, int S, int nh, int d);

// Tiles of the fused projection + attention for T rows of hidden size H: 256 rows by 192
// columns.
inline long fused_attention_tiles(long T, long H) { return (T + 255) / 256 * (3 * H / 192); }

// Whether the automatic mode runs the projection + attention as one kernel: from 256 rows,
// with at least a quarter as many 256-row tiles as the device has CUs (64 on 256 CUs).
// Below that the tiles are mostly padding rows or the long epilogue runs on few CUs, while
// the separate kernels spread the same work.
inline bool fused_attention_pays(long T, long H, int cus) {
  return T >= 256 && 4 * fused_attention_tiles(T, H) >= cus;
}

// Q/K/V projection of x [B*S][H] with the attention of every (sequence, head) in the same
// kernel: w_qkv_t [3H][H] and b_qkv [3H] ordered per head ([Q_h | K_h | V_h], 3d rows each),
// ctx [B*S][H] as launch_attention writes it.  Keys at or past min(lens[b], s_valid) are
// masked (s_valid 1..S, default S; lens NULL: s_valid); causal: query i also ignores keys
// j > i.  hipErrorInvalidValue when the shape does not fit.
hipError_t launch_qkv_attention(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                const void* w_qkv_t, const void* b_qkv, const int32_t* lens,
                                int s_valid, void* ctx, hipStream_t s, bool causal = false);

// fp32 elements of split-K workspace the GEMM of this shape uses (0: it does not split).
size_t gemm_splitk_workspace(ftx_dtype dt, int M, int N, int K);

// The launch plan of an M x N x K projection on a device with `cus` CUs: block tile
// tile_m x tile_n and K ranges (1: no split).  sums_partials as for linear_splits.
void plan_linear(ftx_dtype dt, int M, int N, int K, int cus, bool sums_partials, int* tile_m,
                 int* tile_n, int* splits);

// K ranges a projection of this shape is split into with ws_elems fp32 of workspace (1:
// none).  sums_partials: the partials go to the kernel after it (launch_linear_partials,
// then the split-K LayerNorm), which splits more shapes than a projection that finishes
// its partials with a reduction launch of its own (launch_linear and the other GEMMs).
int linear_splits(ftx_dtype dt, int M, int N, int K, size_t ws_elems, bool sums_partials);

// The split-K partial products of the projection c = a w alone: ws[z][M][N] fp32 for the
// linear_splits(...) ranges z, summed by nobody yet (launch_splitk_bias_residual_layernorm
// consumes them).  hipErrorInvalidValue when the shape does not split.
hipError_t launch_linear_partials(ftx_dtype dt, int M, int N, int K, const void* a,
                                  const void* w_t, float* ws, size_t ws_elems, hipStream_t s);

hipError_t launch_bias_qkv_split(ftx_dtype dt, int B, int S, int nh, int d, const void* qkv,
                                 const void* b_qkv, void* q, void* k, void* vt, hipStream_t s);

// Sq, Sk: the (padded) query and key lengths of the Q [B][n][Sq][d] and K [B][n][Sk][d],
// V^T [B][n][d][Sk] layouts, multiples of 32; ctx [B*Sq][n*d].  s_valid (1..Sk, default
// Sk): the length keys are limited to when lens is NULL, and the bound lens are clamped to.
// causal (Sq == Sk): query i also ignores keys j > i.
hipError_t launch_attention(ftx_dtype dt, int B, int Sq, int Sk, int nh, int d, const void* q,
                            const void* k, const void* vt, const int32_t* lens, void* ctx,
                            hipStream_t s, int s_valid = 0, bool causal = false);

// The S = 32 attention of every (sequence, head) with that head's share of the
// attention-output projection: p[h][b*32 + i][n] = sum over d < D of C_h[b*32 + i][d] *
// wo_t[n][h*D + d] (fp32; C_h rounded to the storage type first), the split-K partials of the
// projection split by head, for the split-K LayerNorm (nh splits).  16-bit data, S = 32,
// hidden size a multiple of 32 and at most 1024 (attention_out_partials_fit); q, k, vt as for
// launch_attention; keys at or past min(lens[b], s_valid) masked.
bool attention_out_partials_fit(ftx_dtype dt, int S, int nh, int d);
hipError_t launch_attention_out_partials(ftx_dtype dt, int B, int nh, int d, const void* q,
                                         const void* k, const void* vt, const int32_t* lens,
                                         int s_valid, const void* wo_t, float* p, hipStream_t s);

hipError_t launch_bias_residual_layernorm(ftx_dtype dt, int rows, int cols, const void* x,
                                          const void* a, const void* bias, const void* gamma,
                                          const void* beta, void* y, hipStream_t s);

// The same LayerNorm with an fp32 residual stream: the branch `a` is fp32, x is read as
// fp32 when x_f32 (else in the storage type), and yf (non-null) receives y in fp32 as well
// as y in the storage type.  16-bit dtypes only.
hipError_t launch_bias_residual_layernorm_f32res(ftx_dtype dt, int rows, int cols,
                                                 const void* x, bool x_f32, const float* a,
                                                 const void* bias, const void* gamma,
                                                 const void* beta, void* y, float* yf,
                                                 hipStream_t s);

// Projection a w_t (N = 128: one 64 x 128 tile holds whole rows) with the bias + residual +
// LayerNorm of launch_bias_residual_layernorm in its epilogue: y = LN(x + a w_t + bias).
// a_f32: the projection's output counts unrounded (the fp32 residual stream of the 16-bit
// modes); x_f32: x is fp32; yf (non-null) also receives y in fp32.
// hipErrorInvalidValue when N != 128.
hipError_t launch_linear_layernorm(ftx_dtype dt, int M, int N, int K, const void* a,
                                   const void* w_t, const void* x, bool x_f32, bool a_f32,
                                   const void* bias, const void* gamma, const void* beta,
                                   void* y, float* yf, hipStream_t s);

// The LayerNorm above after a projection split over K: a = the sum of the fp32 partials
// p[0..splits-1][rows][cols] in split order (what the split-K reduction computes), rounded to
// the storage type unless a_f32 (the projection's output would have been fp32); x is read
// as fp32 when x_f32; yf (non-null) also receives y in fp32.  One workgroup per row.
hipError_t launch_splitk_bias_residual_layernorm(ftx_dtype dt, int rows, int cols,
                                                 const void* x, bool x_f32, const float* p,
                                                 int splits, bool a_f32, const void* bias,
                                                 const void* gamma, const void* beta, void* y,
                                                 float* yf, hipStream_t s);

// LayerNorm folded into the projection after it (16-bit data).  The projection before it
// stores z = x + a w_t + bias (rounded to the storage type; zf non-null: also in fp32) and,
// per row and per tile of the planner's tile width tn, the mean and centred sum of squares
// of the fp32 z over the tile's columns: stats[row][tile] as float2 pairs, ntn =
// ceil(N / tn) tiles.  hipErrorInvalidValue when the planner would split K, ntn does not
// match or N is not a multiple of 8.
hipError_t launch_linear_residual_stats(ftx_dtype dt, int M, int N, int K, const void* a,
                                        const void* w_t, const void* bias, const void* x,
                                        void* z, float* zf, float* stats, int ntn, hipStream_t s);

// The projection of LN(z) through the folded weights w_t = (gamma o W)^T [N][K]:
// c = act(r (z w_t) + s csum + bias) per row, with r, s from the row's ntn stats pairs
// (tiles of bn columns of the K-wide rows), csum and bias fp32 (launch_fold_layernorm_weights).
hipError_t launch_linear_norm_in(ftx_dtype dt, int M, int N, int K, const void* z,
                                 const void* w_t, const float* bias, const float* csum,
                                 const float* stats, int ntn, int bn, bool gelu, void* c,
                                 hipStream_t s);

// y = LN(x + a + bias) with x = LN_x(zx) rebuilt from zx and its stats (the folded
// LayerNorm's gamma xgamma and beta xbeta): the layer's second LayerNorm after a folded
// first.  zx and a both in the storage type, or both fp32 (zx_f32 = a_f32 = true).  cols
// 768 or 1024, every pointer 16-byte aligned; else hipErrorInvalidValue.
hipError_t launch_bias_residual_layernorm_xnorm(ftx_dtype dt, int rows, int cols, const void* zx,
                                                bool zx_f32, const float* xstats, int ntn, int bn,
                                                const void* xgamma, const void* xbeta,
                                                const void* a, bool a_f32, const void* bias,
                                                const void* gamma, const void* beta, void* y,
                                                hipStream_t s);

// Folded weights of a LayerNorm (gamma, beta) followed by the projection w_t [N][K], bias b:
// wf_t[n][k] = w_t[n][k] gamma[k] rounded, csum[n] = sum_k wf_t[n][k] (fp32), bias_f[n] =
// b[n] + sum_k beta[k] w_t[n][k] (fp32).  16-bit data.
hipError_t launch_fold_layernorm_weights(ftx_dtype dt, int N, int K, const void* w_t,
                                         const void* gamma, const void* beta, const void* b,
                                         void* wf_t, float* csum, float* bias_f, hipStream_t s);

hipError_t launch_bias_gelu(ftx_dtype dt, int rows, int cols, const void* u, const void* bias,
                            void* g, hipStream_t s);

hipError_t launch_transpose(ftx_dtype dt, int rows, int cols, const void* in, void* out,
                            hipStream_t s);

// Zero `bytes` bytes at p (16-byte aligned, a multiple of 16) with a kernel.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Read `bytes` bytes at p (16-byte aligned, a multiple of 16) and discard them: a prefetch
// into the last-level cache ahead of a kernel that reads them.  Writes nothing.
hipError_t launch_prefetch(const void* p, size_t bytes, hipStream_t s);

// Largest LayerNorm row the library handles (4-element vectors, <= 16 per lane of a wave).
constexpr int kMaxLayerNormCols = 4096;
// largest inner dimension K of a projection: a 256-row panel of K elements stays below 2^31
// bytes, the range of the buffer resources the GEMM loads through
constexpr int kMaxInnerDim = 1 << 20;

}  // namespace ftx
