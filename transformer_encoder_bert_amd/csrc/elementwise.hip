// Element-wise and row-reduction kernels of the encoder layer: bias + residual + LayerNorm,
// bias + GELU, bias + Q/K/V head split, and the weight transpose used when weights are set.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "Faster Transformer 优化原理": everything except the matrix multiplies is fused
// into a few custom kernels that work element-wise on the matrix-multiply results; 16-bit
// data are moved as packed pairs and promoted to float for the SoftMax / LayerNorm sums;
// row sums use register shuffles; 1/sqrt becomes rsqrt and pow(x, 3) becomes x*x*x.
// Here: 64-lane wavefronts, 8- or 16-byte vector accesses, fp32 statistics, and a
// two-pass (mean, then centred sum of squares) variance held entirely in registers.

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace ftx {

// the most split partials the split-K LayerNorm loads all at once (the planner splits K at
// most 16 ways; the attention-output partials split by head, up to 16 heads here)
constexpr int kMaxSplitsAll = 16;

// ------------------------------------------------------------------------------------
// bias + residual + LayerNorm: y = gamma * (z - mean) * rsqrt(var + eps) + beta,
// z = x + a + bias.  LPR lanes own one row; each lane holds MAXV vectors of EV elements,
// vector v of a lane sits at column EV * (v * LPR + sub) so that a wave's loads of one v
// are contiguous.  EXACT: every lane owns exactly MAXV vectors (cols == EV * LPR * MAXV).
// EV = 8 for 16-bit data (16-byte vectors) when rows allow it, else 4.
// TX and TA are the types of the residual x and the branch a (T, or float when the
// residual stream is kept in fp32); yf, when non-null, receives an fp32 copy of y.
// The residual given un-normalised (a LayerNorm folded into its consumers): x = LN(zx) with
// per-tile row statistics of zx (merge_row_stats) and the first LayerNorm's gamma and beta.
template <typename T> struct ResidualNorm {
  const float2* stats = nullptr;  // [rows][ntn]
  int ntn = 0, bn = 0;
  const T* gamma = nullptr;
  const T* beta = nullptr;
};

template <typename T, typename TX, typename TA, int EV, int LPR, int MAXV, bool EXACT, bool XN = false>
__global__ __launch_bounds__(256) void layernorm_kernel(const TX* __restrict__ x,
                                                        const TA* __restrict__ a,
                                                        const T* __restrict__ bias,
                                                        const T* __restrict__ gamma,
                                                        const T* __restrict__ beta,
                                                        T* y, float* yf, int rows, int cols,
                                                        ResidualNorm<T> xn) {
  typedef typename VecT<T, EV>::type tv;
  typedef typename VecT<TX, EV>::type xv_t;
  typedef typename VecT<TA, EV>::type av_t;
  typedef typename VecT<float, EV>::type fv;
  constexpr int RPW = kWave / LPR;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int row = (blockIdx.x * (blockDim.x / kWave) + wave) * RPW + lane / LPR;
  const int sub = lane % LPR;
  if (row >= rows) return;  // whole LPR-lane groups leave together
  const int nvec = cols / EV;
  const size_t base = (size_t)row * cols;

  float z[MAXV][EV];
  float sum = 0.f;
  if constexpr (XN) {
    // every load of the row first (the stats pairs with the vectors), then the merge
    static_assert(EXACT, "the rebuilt residual takes the exact tilings");
    float2 st[kMaxStatTiles];
#pragma unroll
    for (int t = 0; t < kMaxStatTiles; ++t)
      st[t] = t < xn.ntn ? xn.stats[(size_t)row * xn.ntn + t] : make_float2(0.f, 0.f);
    xv_t xv[MAXV];
    av_t av[MAXV];
    tv bv[MAXV], xg[MAXV], xb[MAXV];
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int vi = v * LPR + sub;
      xv[v] = *(const xv_t*)(x + base + EV * vi);
      av[v] = *(const av_t*)(a + base + EV * vi);
      bv[v] = *(const tv*)(bias + EV * vi);
      xg[v] = *(const tv*)(xn.gamma + EV * vi);
      xb[v] = *(const tv*)(xn.beta + EV * vi);
    }
    const float2 xrs = merge_row_stats<kMaxStatTiles>(st, xn.ntn, xn.bn, cols, FTX_LN_EPSILON);
#pragma unroll
    for (int v = 0; v < MAXV; ++v)
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        const float xe = fmaf(to_f32(xg[v][e]), fmaf(to_f32(xv[v][e]), xrs.x, xrs.y), to_f32(xb[v][e]));
        z[v][e] = xe + to_f32(av[v][e]) + to_f32(bv[v][e]);
        sum += z[v][e];
      }
  } else {
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const int vi = v * LPR + sub;
      if (EXACT || vi < nvec) {
        const xv_t xv = *(const xv_t*)(x + base + EV * vi);
        const av_t av = *(const av_t*)(a + base + EV * vi);
        const tv bv = *(const tv*)(bias + EV * vi);
#pragma unroll
        for (int e = 0; e < EV; ++e) {
          z[v][e] = to_f32(xv[e]) + to_f32(av[e]) + to_f32(bv[e]);
          sum += z[v][e];
        }
      }
    }
  }
  const float inv_n = 1.0f / (float)cols;
  const float mean = group_sum<LPR>(sum) * inv_n;
  float sq = 0.f;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int vi = v * LPR + sub;
    if (EXACT || vi < nvec) {
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        const float c = z[v][e] - mean;
        sq += c * c;
      }
    }
  }
  const float var = group_sum<LPR>(sq) * inv_n;
  const float rs = rsqrtf(var + FTX_LN_EPSILON);
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int vi = v * LPR + sub;
    if (EXACT || vi < nvec) {
      const tv gv = *(const tv*)(gamma + EV * vi);
      const tv btv = *(const tv*)(beta + EV * vi);
      fv of;
      tv o;
#pragma unroll
      for (int e = 0; e < EV; ++e) {
        of[e] = to_f32(gv[e]) * ((z[v][e] - mean) * rs) + to_f32(btv[e]);
        o[e] = from_f32<T>(of[e]);
      }
      *(tv*)(y + base + EV * vi) = o;
      if (yf) *(fv*)(yf + base + EV * vi) = of;
    }
  }
}

template <typename T, typename TX, typename TA, int EV, int LPR, int MAXV, bool EXACT, bool XN = false>
static hipError_t ln_launch(int rows, int cols, const void* x, const void* a, const void* bias,
                            const void* gamma, const void* beta, void* y, float* yf,
                            hipStream_t s, ResidualNorm<T> xn = {}) {
  constexpr int rows_per_block = (256 / kWave) * (kWave / LPR);
  const int grid = (rows + rows_per_block - 1) / rows_per_block;
  layernorm_kernel<T, TX, TA, EV, LPR, MAXV, EXACT, XN><<<grid, 256, 0, s>>>(
      (const TX*)x, (const TA*)a, (const T*)bias, (const T*)gamma, (const T*)beta, (T*)y, yf,
      rows, cols, xn);
  return hipGetLastError();
}

// The folded-LayerNorm residual (16-bit, the exact tilings of the common hidden sizes only;
// TX, TA: T or float)
template <typename T, typename TX, typename TA>
static hipError_t ln_xnorm_dispatch(int rows, int cols, const void* x, const void* a,
                                    const void* bias, const void* gamma, const void* beta,
                                    void* y, ResidualNorm<T> xn, hipStream_t s) {
  for (const void* p : {x, a, bias, gamma, beta, (const void*)y, (const void*)xn.gamma, (const void*)xn.beta})
    if (!p || ((uintptr_t)p & 15)) return hipErrorInvalidValue;
  switch (cols) {
    case 768: return ln_launch<T, TX, TA, 8, 32, 3, true, true>(rows, cols, x, a, bias, gamma, beta, y, nullptr, s, xn);
    case 1024: return ln_launch<T, TX, TA, 8, 32, 4, true, true>(rows, cols, x, a, bias, gamma, beta, y, nullptr, s, xn);
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t ln_xnorm_types(bool x_f32, bool a_f32, int rows, int cols, const void* x,
                                 const void* a, const void* bias, const void* gamma,
                                 const void* beta, void* y, ResidualNorm<T> xn, hipStream_t s) {
  if (x_f32 && a_f32) return ln_xnorm_dispatch<T, float, float>(rows, cols, x, a, bias, gamma, beta, y, xn, s);
  if (!x_f32 && !a_f32) return ln_xnorm_dispatch<T, T, T>(rows, cols, x, a, bias, gamma, beta, y, xn, s);
  return hipErrorInvalidValue;
}

template <typename T, typename TX, typename TA>
static hipError_t ln_dispatch(int rows, int cols, const void* x, const void* a, const void* bias,
                              const void* gamma, const void* beta, void* y, float* yf,
                              hipStream_t s) {
  // 16-byte vectors of 16-bit data when every row start and parameter vector is 16-byte
  // aligned (rows a multiple of 8 elements)
  bool wide = sizeof(T) == 2 && cols % 8 == 0;
  for (const void* p : {x, a, bias, gamma, beta, (const void*)y, (const void*)yf})
    if (p && ((uintptr_t)p & 15)) wide = false;
  if constexpr (sizeof(T) == 2) {
    if (wide) {
      switch (cols) {  // exact register tilings for the common hidden sizes
        case 128: return ln_launch<T, TX, TA, 8, 16, 1, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        case 256: return ln_launch<T, TX, TA, 8, 32, 1, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        case 384: return ln_launch<T, TX, TA, 8, 16, 3, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        case 512: return ln_launch<T, TX, TA, 8, 32, 2, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        case 768: return ln_launch<T, TX, TA, 8, 32, 3, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        case 1024: return ln_launch<T, TX, TA, 8, 32, 4, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
        default: break;
      }
      if (cols <= 8 * 16 * 4)  // small rows: a quarter wave per row
        return ln_launch<T, TX, TA, 8, 16, 4, false>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
      return ln_launch<T, TX, TA, 8, 64, 8, false>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    }
  }
  switch (cols) {
    case 128: return ln_launch<T, TX, TA, 4, 32, 1, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case 256: return ln_launch<T, TX, TA, 4, 64, 1, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case 384: return ln_launch<T, TX, TA, 4, 32, 3, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case 512: return ln_launch<T, TX, TA, 4, 64, 2, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case 768: return ln_launch<T, TX, TA, 4, 64, 3, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case 1024: return ln_launch<T, TX, TA, 4, 64, 4, true>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    default: break;
  }
  if (cols <= 4 * 16 * 4)  // small rows: a quarter wave per row
    return ln_launch<T, TX, TA, 4, 16, 4, false>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
  return ln_launch<T, TX, TA, 4, 64, 16, false>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
}

hipError_t launch_bias_residual_layernorm(ftx_dtype dt, int rows, int cols, const void* x,
                                          const void* a, const void* bias, const void* gamma,
                                          const void* beta, void* y, hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return ln_dispatch<float, float, float>(rows, cols, x, a, bias, gamma, beta, y, nullptr, s);
    case FTX_FP16: return ln_dispatch<f16, f16, f16>(rows, cols, x, a, bias, gamma, beta, y, nullptr, s);
    case FTX_BF16: return ln_dispatch<bf16, bf16, bf16>(rows, cols, x, a, bias, gamma, beta, y, nullptr, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bias_residual_layernorm_xnorm(ftx_dtype dt, int rows, int cols, const void* zx,
                                                bool zx_f32, const float* xstats, int ntn, int bn,
                                                const void* xgamma, const void* xbeta,
                                                const void* a, bool a_f32, const void* bias,
                                                const void* gamma, const void* beta, void* y,
                                                hipStream_t s) {
  if (ntn < 1 || ntn > kMaxStatTiles || bn < 1 || (cols + bn - 1) / bn != ntn) return hipErrorInvalidValue;
  switch (dt) {
    case FTX_FP16: {
      const ResidualNorm<f16> xn{(const float2*)xstats, ntn, bn, (const f16*)xgamma, (const f16*)xbeta};
      return ln_xnorm_types<f16>(zx_f32, a_f32, rows, cols, zx, a, bias, gamma, beta, y, xn, s);
    }
    case FTX_BF16: {
      const ResidualNorm<bf16> xn{(const float2*)xstats, ntn, bn, (const bf16*)xgamma, (const bf16*)xbeta};
      return ln_xnorm_types<bf16>(zx_f32, a_f32, rows, cols, zx, a, bias, gamma, beta, y, xn, s);
    }
    default: break;
  }
  return hipErrorInvalidValue;
}

// A LayerNorm (gamma, beta over the K index) folded into the projection after it, W^T [N][K]:
// w'[n][k] = w[n][k] gamma[k] rounded to T, csum[n] = the fp32 sum over k of the rounded
// w'[n][k], bias'[n] = b[n] + sum_k beta[k] w[n][k] in fp32, so that LN(z) W + b =
// r (z W') + s csum + bias' for the row's r, s.  One wave per row n, sums in a fixed order.
// Weight preparation only (set_weights), not on the forward's path.
template <typename T>
__global__ __launch_bounds__(256) void fold_ln_weights_kernel(const T* __restrict__ w,
                                                              const T* __restrict__ gamma,
                                                              const T* __restrict__ beta,
                                                              const T* __restrict__ b, T* wf,
                                                              float* csum, float* bf, int N,
                                                              int K) {
  const int n = blockIdx.x * (256 / kWave) + threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (n >= N) return;
  float cs = 0.f, bs = 0.f;
  for (int k = lane; k < K; k += kWave) {
    const float wv = to_f32(w[(size_t)n * K + k]);
    const T wr = from_f32<T>(wv * to_f32(gamma[k]));
    wf[(size_t)n * K + k] = wr;
    cs += to_f32(wr);
    bs += to_f32(beta[k]) * wv;
  }
  cs = group_sum<kWave>(cs);
  bs = group_sum<kWave>(bs);
  if (lane == 0) {
    csum[n] = cs;
    bf[n] = to_f32(b[n]) + bs;
  }
}

hipError_t launch_fold_layernorm_weights(ftx_dtype dt, int N, int K, const void* w_t,
                                         const void* gamma, const void* beta, const void* b,
                                         void* wf_t, float* csum, float* bias_f, hipStream_t s) {
  const int blocks = (N + 3) / 4;
  switch (dt) {
    case FTX_FP16:
      fold_ln_weights_kernel<f16><<<blocks, 256, 0, s>>>((const f16*)w_t, (const f16*)gamma, (const f16*)beta,
                                                          (const f16*)b, (f16*)wf_t, csum, bias_f, N, K);
      return hipGetLastError();
    case FTX_BF16:
      fold_ln_weights_kernel<bf16><<<blocks, 256, 0, s>>>((const bf16*)w_t, (const bf16*)gamma, (const bf16*)beta,
                                                           (const bf16*)b, (bf16*)wf_t, csum, bias_f, N, K);
      return hipGetLastError();
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bias_residual_layernorm_f32res(ftx_dtype dt, int rows, int cols,
                                                 const void* x, bool x_f32, const float* a,
                                                 const void* bias, const void* gamma,
                                                 const void* beta, void* y, float* yf,
                                                 hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return hipErrorInvalidValue;  // fp32 mode has no separate residual copy
    case FTX_FP16:
      return x_f32 ? ln_dispatch<f16, float, float>(rows, cols, x, a, bias, gamma, beta, y, yf, s)
                   : ln_dispatch<f16, f16, float>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
    case FTX_BF16:
      return x_f32 ? ln_dispatch<bf16, float, float>(rows, cols, x, a, bias, gamma, beta, y, yf, s)
                   : ln_dispatch<bf16, bf16, float>(rows, cols, x, a, bias, gamma, beta, y, yf, s);
  }
  return hipErrorInvalidValue;
}

// Sum over the 256 threads of a workgroup in a fixed order (deterministic); `red` holds
// four floats of LDS.
__device__ __forceinline__ float block_sum256(float v, float* red) {
  v = group_sum<kWave>(v);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();  // every thread has read red before it is written again
  return t;
}

// bias + residual + LayerNorm of a projection that was split over K (the small-batch path):
// the branch a is the sum of the fp32 partials in split order -- the split-K reduction's
// sum -- rounded to TA as the projection would have stored it, so one launch replaces the
// reduction and the LayerNorm.  One workgroup of 256 threads per row, 4 columns per thread
// and group (cols <= 4096, a multiple of 4): the partial reads of a row spread over a
// whole CU.  ALL (5 to kMaxSplitsAll splits): a thread issues the loads of all the splits of
// its columns before adding them (one memory round trip; at batch 1 the FFN-out projection
// is cut in 16), a variant of its own so that fewer splits keep the smaller kernel.  Statistics
// as in layernorm_kernel (fp32, mean, then centred sum of squares).
template <typename T, typename TX, typename TA, bool ALL>
__global__ __launch_bounds__(256) void splitk_layernorm_kernel(const TX* __restrict__ x,
                                                               const float* __restrict__ p,
                                                               int splits,
                                                               const T* __restrict__ bias,
                                                               const T* __restrict__ gamma,
                                                               const T* __restrict__ beta,
                                                               T* y, float* yf, int rows,
                                                               int cols) {
  constexpr int G = kMaxLayerNormCols / (4 * 256);
  typedef typename VecT<T, 4>::type t4;
  typedef typename VecT<TX, 4>::type x4;
  __shared__ float red[4];
  const int row = blockIdx.x;
  const size_t base = (size_t)row * cols, mn = (size_t)rows * cols;
  float z[G][4];
  float sum = 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int c = 4 * (threadIdx.x + 256 * gi);
    if (c < cols) {
      const f32x4 acc = ALL ? sum_partials_all<kMaxSplitsAll>(p + base + c, mn, splits)
                            : sum_partials4(p + base + c, mn, splits);
      const x4 xv = *(const x4*)(x + base + c);
      const t4 bv = *(const t4*)(bias + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the reduction's store: no projection bias (the LayerNorm adds it), rounded to TA
        const float a = to_f32(from_f32<TA>(acc[e] + 0.0f));
        z[gi][e] = to_f32(xv[e]) + a + to_f32(bv[e]);
        sum += z[gi][e];
      }
    }
  }
  const float inv_n = 1.0f / (float)cols;
  const float mean = block_sum256(sum, red) * inv_n;
  float sq = 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
    if (4 * (threadIdx.x + 256 * gi) < cols)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = z[gi][e] - mean;
        sq += d * d;
      }
  const float rs = rsqrtf(block_sum256(sq, red) * inv_n + FTX_LN_EPSILON);
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int c = 4 * (threadIdx.x + 256 * gi);
    if (c < cols) {
      const t4 gv = *(const t4*)(gamma + c), btv = *(const t4*)(beta + c);
      f32x4 of;
      t4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        of[e] = to_f32(gv[e]) * ((z[gi][e] - mean) * rs) + to_f32(btv[e]);
        o[e] = from_f32<T>(of[e]);
      }
      *(t4*)(y + base + c) = o;
      if (yf) *(f32x4*)(yf + base + c) = of;
    }
  }
}

template <typename T, typename TX, typename TA>
static hipError_t splitk_ln_launch(int rows, int cols, const void* x, const float* p, int splits,
                                   const void* bias, const void* gamma, const void* beta,
                                   void* y, float* yf, hipStream_t s) {
  if (splits > 4 && splits <= kMaxSplitsAll)
    splitk_layernorm_kernel<T, TX, TA, true><<<rows, 256, 0, s>>>(
        (const TX*)x, p, splits, (const T*)bias, (const T*)gamma, (const T*)beta, (T*)y, yf, rows,
        cols);
  else
    splitk_layernorm_kernel<T, TX, TA, false><<<rows, 256, 0, s>>>(
        (const TX*)x, p, splits, (const T*)bias, (const T*)gamma, (const T*)beta, (T*)y, yf, rows,
        cols);
  return hipGetLastError();
}

hipError_t launch_splitk_bias_residual_layernorm(ftx_dtype dt, int rows, int cols,
                                                 const void* x, bool x_f32, const float* p,
                                                 int splits, bool a_f32, const void* bias,
                                                 const void* gamma, const void* beta, void* y,
                                                 float* yf, hipStream_t s) {
  if (rows < 1 || cols < 4 || cols % 4 || cols > kMaxLayerNormCols || splits < 1)
    return hipErrorInvalidValue;
  if (x_f32 && !a_f32) return hipErrorInvalidValue;  // an fp32 residual comes with an fp32 branch
  switch (dt) {
    case FTX_FP32:
      return splitk_ln_launch<float, float, float>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
    case FTX_FP16:
      if (x_f32) return splitk_ln_launch<f16, float, float>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
      if (a_f32) return splitk_ln_launch<f16, f16, float>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
      return splitk_ln_launch<f16, f16, f16>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
    case FTX_BF16:
      if (x_f32) return splitk_ln_launch<bf16, float, float>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
      if (a_f32) return splitk_ln_launch<bf16, bf16, float>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
      return splitk_ln_launch<bf16, bf16, bf16>(rows, cols, x, p, splits, bias, gamma, beta, y, yf, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------
// bias + GELU over [rows][cols], 16-byte vectors, grid-stride.
template <typename T>
__global__ __launch_bounds__(256) void bias_gelu_kernel(const T* u, const T* __restrict__ bias,
                                                        T* g, int64_t nvec, int cols) {
  typedef typename Vec16<T>::type vec;
  constexpr int N = Vec16<T>::N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int col = (int)((i * N) % cols);
    const vec uv = *(const vec*)(u + i * N);
    const vec bv = *(const vec*)(bias + col);
    vec o;
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = from_f32<T>(gelu_tanh(to_f32(uv[e]) + to_f32(bv[e])));
    *(vec*)(g + i * N) = o;
  }
}

template <typename T>
static hipError_t gelu_launch(int rows, int cols, const void* u, const void* bias, void* g,
                              hipStream_t s) {
  const int64_t nvec = (int64_t)rows * cols / Vec16<T>::N;
  int64_t blocks = (nvec + 255) / 256;
  const int64_t cap = 256 * 16;  // 16 waves' worth of blocks per CU is plenty
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  bias_gelu_kernel<T><<<(int)blocks, 256, 0, s>>>((const T*)u, (const T*)bias, (T*)g, nvec, cols);
  return hipGetLastError();
}

hipError_t launch_bias_gelu(ftx_dtype dt, int rows, int cols, const void* u, const void* bias,
                            void* g, hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return gelu_launch<float>(rows, cols, u, bias, g, s);
    case FTX_FP16: return gelu_launch<f16>(rows, cols, u, bias, g, s);
    case FTX_BF16: return gelu_launch<bf16>(rows, cols, u, bias, g, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------
// bias + head split: qkv [T][3H] -> q, k [B][n][S][D], vt [B][n][D][S].
// Block = 32 tokens of one (which, head); V goes through LDS to be written along tokens.
template <typename T, int D>
__global__ __launch_bounds__(256) void bias_qkv_split_kernel(const T* __restrict__ qkv,
                                                             const T* __restrict__ bias,
                                                             T* __restrict__ q, T* __restrict__ k,
                                                             T* __restrict__ vt, int S, int nh) {
  typedef typename Vec16<T>::type vec;
  constexpr int N = Vec16<T>::N;
  constexpr int CPR = D / N;  // 16-byte chunks per head row
  __shared__ T tile[32][D + N];
  const int H = nh * D;
  const int which = blockIdx.y / nh, h = blockIdx.y % nh;
  const int t0 = blockIdx.x * 32;
  const int b = t0 / S, s0 = t0 % S;
  const size_t head = (size_t)b * nh + h;
  for (int c = threadIdx.x; c < 32 * CPR; c += blockDim.x) {
    const int r = c / CPR, cc = (c % CPR) * N;
    const int col = which * H + h * D + cc;
    const vec iv = *(const vec*)(qkv + (size_t)(t0 + r) * 3 * H + col);
    const vec bv = *(const vec*)(bias + col);
    vec o;
#pragma unroll
    for (int e = 0; e < N; ++e) o[e] = from_f32<T>(to_f32(iv[e]) + to_f32(bv[e]));
    if (which < 2) {
      T* dst = (which == 0 ? q : k) + (head * S + s0 + r) * D + cc;
      *(vec*)dst = o;
    } else {
      *(vec*)&tile[r][cc] = o;
    }
  }
  if (which == 2) {  // uniform across the block
    __syncthreads();
    constexpr int TCH = 32 / N;  // chunks along the 32 tokens
    for (int c = threadIdx.x; c < D * TCH; c += blockDim.x) {
      const int dd = c / TCH, sc = (c % TCH) * N;
      vec o;
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = tile[sc + e][dd];
      *(vec*)(vt + (head * D + dd) * S + s0 + sc) = o;
    }
  }
}

template <typename T>
static hipError_t split_launch(int B, int S, int nh, int d, const void* qkv, const void* b_qkv,
                               void* q, void* k, void* vt, hipStream_t s) {
  dim3 grid((unsigned)(B * S / 32), (unsigned)(3 * nh));
  if (d == 64)
    bias_qkv_split_kernel<T, 64><<<grid, 256, 0, s>>>((const T*)qkv, (const T*)b_qkv, (T*)q, (T*)k, (T*)vt, S, nh);
  else if (d == 32)
    bias_qkv_split_kernel<T, 32><<<grid, 256, 0, s>>>((const T*)qkv, (const T*)b_qkv, (T*)q, (T*)k, (T*)vt, S, nh);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bias_qkv_split(ftx_dtype dt, int B, int S, int nh, int d, const void* qkv,
                                 const void* b_qkv, void* q, void* k, void* vt, hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return split_launch<float>(B, S, nh, d, qkv, b_qkv, q, k, vt, s);
    case FTX_FP16: return split_launch<f16>(B, S, nh, d, qkv, b_qkv, q, k, vt, s);
    case FTX_BF16: return split_launch<bf16>(B, S, nh, d, qkv, b_qkv, q, k, vt, s);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------
// Transpose out[cols][rows] = in[rows][cols], 32x32 tiles through LDS, element accesses
// (no alignment assumption).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, T* __restrict__ out,
                                                        int rows, int cols) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
  for (int i = ty; i < 32; i += 8) {
    const int r = r0 + i, c = c0 + tx;
    if (r < rows && c < cols) tile[i][tx] = in[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int i = ty; i < 32; i += 8) {
    const int c = c0 + i, r = r0 + tx;
    if (r < rows && c < cols) out[(size_t)c * rows + r] = tile[tx][i];
  }
}

template <typename T>
static hipError_t transpose_launch(int rows, int cols, const void* in, void* out, hipStream_t s) {
  dim3 grid((unsigned)((cols + 31) / 32), (unsigned)((rows + 31) / 32));
  transpose_kernel<T><<<grid, 256, 0, s>>>((const T*)in, (T*)out, rows, cols);
  return hipGetLastError();
}

hipError_t launch_transpose(ftx_dtype dt, int rows, int cols, const void* in, void* out,
                            hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return transpose_launch<float>(rows, cols, in, out, s);
    case FTX_FP16: return transpose_launch<f16>(rows, cols, in, out, s);
    case FTX_BF16: return transpose_launch<bf16>(rows, cols, in, out, s);
  }
  return hipErrorInvalidValue;
}

// Zero n16 16-byte vectors at p (grid-stride; the pointer is 16-byte aligned).  A kernel
// rather than hipMemsetAsync, so a caller's HIP graph capture records a kernel node.
__global__ __launch_bounds__(256) void zero16_kernel(uint4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = uint4{0u, 0u, 0u, 0u};
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  if (((uintptr_t)p & 15u) || (bytes & 15u)) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 4096);
  zero16_kernel<<<(unsigned)blocks, 256, 0, s>>>((uint4*)p, n16);
  return hipGetLastError();
}

// Read n16 16-byte vectors at p and discard them, so that the lines sit in the last-level
// cache (and the reading XCD's L2) when the next kernel reads them.  Four independent loads
// per thread per iteration; the XOR of everything read goes to an empty asm statement, which
// keeps the loads without any store.
__global__ __launch_bounds__(256) void prefetch16_kernel(const uint4* __restrict__ p, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  unsigned acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  asm volatile("" ::"v"(acc));
}

hipError_t launch_prefetch(const void* p, size_t bytes, hipStream_t s) {
  if (((uintptr_t)p & 15u) || (bytes & 15u)) return hipErrorInvalidValue;
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const size_t blocks = std::min<size_t>((n16 + 255) / 256, 512);
  prefetch16_kernel<<<(unsigned)blocks, 256, 0, s>>>((const uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace ftx
