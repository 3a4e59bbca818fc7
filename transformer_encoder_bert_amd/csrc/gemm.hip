// Dense projections of the encoder layer on CDNA4 matrix cores (MFMA), LDS-tiled.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "Faster Transformer 优化原理": the per-layer matrix multiplies (there: cuBLAS with
// the fastest algorithm chosen per shape, on Tensor Cores in FP16) with everything
// element-wise fused around them.  Here the projections are hand-written for gfx950:
//   C[M][N] = A[M][K] * W[K][N], W held transposed (Wt[N][K], K contiguous) so both
//   operands are read along K with 16-byte loads;
//   v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate) or v_mfma_f32_32x32x2f32 for fp32;
//   a block tile BM x BN staged through double-buffered, padded LDS, waves WM x WN each
//   owning a (BM/WM) x (BN/WN) sub-tile of 32x32 accumulators;
//   the bias, the tanh GELU and the Q/K/V head split are applied in the epilogue on the
//   fp32 accumulators, so U never makes a round trip through memory before its GELU.
//
// MFMA operand layout used (32x32 output tile, 64 lanes, g = lane / 32):
//   A fragment: lane holds row (lane % 32), VEC consecutive K values at K-offset g * VEC;
//   B fragment: lane holds column (lane % 32), the same K offsets;
//   accumulator register r of a lane holds row 8*(r/4) + 4*g + (r%4), column lane % 32.
// The K order inside a fragment only has to agree between A and B, which it does by
// construction (both load K-contiguous runs at the same offsets).

#include "device_common.h"
#include "launch.h"

namespace ftx {

template <typename T> struct Mfma;

template <> struct Mfma<f16> {
  static constexpr int VEC = 8;  // elements per lane per fragment (16 bytes)
  static constexpr int KF = 16;  // K consumed per fragment
  typedef f16x8 frag;
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<bf16> {
  static constexpr int VEC = 8;
  static constexpr int KF = 16;
  typedef bf16x8 frag;
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int VEC = 4;
  static constexpr int KF = 8;   // four 32x32x2 steps per 16-byte fragment
  typedef f32x4 frag;
  __device__ static __forceinline__ void mma(const frag& a, const frag& b, f32x16& c) {
#pragma unroll
    for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
  }
};

// ------------------------------------------------------------------------------- epilogues
// apply(row0, col, g, acc, M, N): acc is the 32x32 accumulator tile whose first row is
// row0 and whose column for this lane is col.

template <typename T, bool GELU> struct EpiLinear {
  T* c;
  const T* bias;  // may be null
  __device__ __forceinline__ void apply(int row0, int col, int g, const f32x16& acc, int M,
                                        int N) const {
    if (col >= N) return;
    const float bv = bias ? to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + 8 * (r / 4) + 4 * g + (r % 4);
      if (row < M) {
        float v = acc[r] + bv;
        if (GELU) v = gelu_tanh(v);
        c[(size_t)row * N + col] = from_f32<T>(v);
      }
    }
  }
};

// bias + head split: column col of [Q|K|V] -> (which, head, dd); rows of one 32-row tile
// belong to one sequence because S is a multiple of 32.
template <typename T> struct EpiQKV {
  T* q;
  T* k;
  T* vt;
  const T* bias;
  int S, nh, d;
  __device__ __forceinline__ void apply(int row0, int col, int g, const f32x16& acc, int M,
                                        int N) const {
    if (col >= N || row0 >= M) return;
    const int H = nh * d;
    const int which = col / H;
    const int rem = col - which * H;
    const int h = rem / d;
    const int dd = rem - h * d;
    const int b = row0 / S;
    const int s0 = row0 - b * S;
    const size_t head = (size_t)b * nh + h;
    const float bv = to_f32(bias[col]);
    if (which < 2) {
      T* dst = (which == 0 ? q : k) + (head * S + s0) * d + dd;
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[(size_t)(8 * (r / 4) + 4 * g + (r % 4)) * d] = from_f32<T>(acc[r] + bv);
    } else {
      typedef typename VecT<T, 4>::type v4;
      T* dst = vt + (head * d + dd) * S + s0;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        v4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(acc[4 * rr + e] + bv);
        *(v4*)(dst + 8 * rr + 4 * g) = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------------- kernel

template <typename T, int BM, int BN, int WM, int WN> struct GemmCfg {
  typedef Mfma<T> MF;
  static constexpr int VEC = MF::VEC;
  static constexpr int BK = 128 / sizeof(T);        // 128 bytes of K per tile row
  static constexpr int LDS_STRIDE = BK + VEC;       // +16 bytes: conflict-free 16-byte reads
  static constexpr int NT = WM * WN * kWave;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int CPR = BK / VEC;              // 16-byte chunks per tile row
  static constexpr int A_CH = BM * CPR / NT;
  static constexpr int B_CH = BN * CPR / NT;
  static constexpr int STAGE = (BM + BN) * LDS_STRIDE;  // elements per LDS buffer
  static_assert(TM >= 1 && TN >= 1, "wave tile below 32x32");
  static_assert(A_CH * NT == BM * CPR && B_CH * NT == BN * CPR, "tile not divisible");
};

// Map the linear block id to a (tile_m, tile_n): blocks are handed to the 8 XCDs round
// robin, so first give every XCD a contiguous range of tiles, then walk each range in
// groups of GROUP_M tile rows so the blocks resident on one XCD share A and W panels in
// that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int XCDS = 8, GROUP_M = 8;
  const int nt = tiles_m * tiles_n;
  int L = bid;
  if (nt % XCDS == 0) L = (bid % XCDS) * (nt / XCDS) + bid / XCDS;
  const int per_group = GROUP_M * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = L - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

template <typename T, int BM, int BN, int WM, int WN, typename Epi>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_kernel(const T* __restrict__ A,
                                                               const T* __restrict__ Bt, int M,
                                                               int N, int K, Epi epi) {
  typedef GemmCfg<T, BM, BN, WM, WN> C;
  typedef typename C::MF MF;
  typedef typename MF::frag frag;
  __shared__ __attribute__((aligned(16))) T smem[2 * C::STAGE];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, g = lane / 32;

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  frag ra[C::A_CH], rb[C::B_CH];
  const frag zero = {};

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / C::CPR, kc = (c % C::CPR) * C::VEC;
      const int gr = m0 + r, gk = k0 + kc;
      ra[i] = (gr < M && gk < K) ? *(const frag*)(A + (size_t)gr * K + gk) : zero;
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / C::CPR, kc = (c % C::CPR) * C::VEC;
      const int gr = n0 + r, gk = k0 + kc;
      rb[i] = (gr < N && gk < K) ? *(const frag*)(Bt + (size_t)gr * K + gk) : zero;
    }
  };
  auto sstore = [&](int buf) {
    T* As = smem + buf * C::STAGE;
    T* Bs = As + BM * C::LDS_STRIDE;
#pragma unroll
    for (int i = 0; i < C::A_CH; ++i) {
      const int c = tid + i * C::NT;
      *(frag*)(As + (c / C::CPR) * C::LDS_STRIDE + (c % C::CPR) * C::VEC) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < C::B_CH; ++i) {
      const int c = tid + i * C::NT;
      *(frag*)(Bs + (c / C::CPR) * C::LDS_STRIDE + (c % C::CPR) * C::VEC) = rb[i];
    }
  };

  const int nk = (K + C::BK - 1) / C::BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * C::BK);
    const T* As = smem + cur * C::STAGE + (wm * C::TM * 32 + lr) * C::LDS_STRIDE + g * C::VEC;
    const T* Bs = smem + cur * C::STAGE + (BM + wn * C::TN * 32 + lr) * C::LDS_STRIDE + g * C::VEC;
#pragma unroll
    for (int kk = 0; kk < C::BK; kk += MF::KF) {
      frag a[C::TM], b[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) a[i] = *(const frag*)(As + i * 32 * C::LDS_STRIDE + kk);
#pragma unroll
      for (int j = 0; j < C::TN; ++j) b[j] = *(const frag*)(Bs + j * 32 * C::LDS_STRIDE + kk);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) MF::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      epi.apply(m0 + (wm * C::TM + i) * 32, n0 + (wn * C::TN + j) * 32 + lr, g, acc[i][j], M, N);
}

// --------------------------------------------------------------------------- tile choice

enum TileCfg { TILE_128x128 = 0, TILE_64x64 = 1, TILE_32x32 = 2 };

static TileCfg choose_tile(int M, int N) {
  const long t128 = (long)((M + 127) / 128) * ((N + 127) / 128);
  if (t128 >= 512) return TILE_128x128;
  const long t64 = (long)((M + 63) / 64) * ((N + 63) / 64);
  if (t64 >= 256) return TILE_64x64;
  return TILE_32x32;
}

template <typename T, int BM, int BN, int WM, int WN, typename Epi>
static hipError_t gemm_launch_cfg(int M, int N, int K, const void* a, const void* w_t, Epi epi,
                                  hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  gemm_kernel<T, BM, BN, WM, WN, Epi><<<tiles, WM * WN * kWave, 0, s>>>(
      (const T*)a, (const T*)w_t, M, N, K, epi);
  return hipGetLastError();
}

template <typename T, typename Epi>
static hipError_t gemm_launch(int M, int N, int K, const void* a, const void* w_t, Epi epi,
                              hipStream_t s) {
  switch (choose_tile(M, N)) {
    case TILE_128x128: return gemm_launch_cfg<T, 128, 128, 2, 2>(M, N, K, a, w_t, epi, s);
    case TILE_64x64: return gemm_launch_cfg<T, 64, 64, 2, 2>(M, N, K, a, w_t, epi, s);
    case TILE_32x32: return gemm_launch_cfg<T, 32, 32, 1, 1>(M, N, K, a, w_t, epi, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t linear_t(int M, int N, int K, const void* a, const void* w_t, const void* bias,
                           bool gelu, void* c, hipStream_t s) {
  if (gelu) return gemm_launch<T>(M, N, K, a, w_t, EpiLinear<T, true>{(T*)c, (const T*)bias}, s);
  return gemm_launch<T>(M, N, K, a, w_t, EpiLinear<T, false>{(T*)c, (const T*)bias}, s);
}

hipError_t launch_linear(ftx_dtype dt, int M, int N, int K, const void* a, const void* w_t,
                         const void* bias, bool gelu, void* c, hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return linear_t<float>(M, N, K, a, w_t, bias, gelu, c, s);
    case FTX_FP16: return linear_t<f16>(M, N, K, a, w_t, bias, gelu, c, s);
    case FTX_BF16: return linear_t<bf16>(M, N, K, a, w_t, bias, gelu, c, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t qkv_t(int B, int S, int nh, int d, const void* x, const void* w, const void* b,
                        void* q, void* k, void* vt, hipStream_t s) {
  const int M = B * S, H = nh * d;
  EpiQKV<T> epi{(T*)q, (T*)k, (T*)vt, (const T*)b, S, nh, d};
  return gemm_launch<T>(M, 3 * H, H, x, w, epi, s);
}

hipError_t launch_qkv_projection(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                 const void* w_qkv_t, const void* b_qkv, void* q, void* k,
                                 void* vt, hipStream_t s) {
  switch (dt) {
    case FTX_FP32: return qkv_t<float>(B, S, nh, d, x, w_qkv_t, b_qkv, q, k, vt, s);
    case FTX_FP16: return qkv_t<f16>(B, S, nh, d, x, w_qkv_t, b_qkv, q, k, vt, s);
    case FTX_BF16: return qkv_t<bf16>(B, S, nh, d, x, w_qkv_t, b_qkv, q, k, vt, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace ftx
