// Dense projections of the encoder layer on CDNA4 matrix cores (MFMA), LDS-tiled.
//
// Source: the Faster Transformer article (cloud.tencent.com/developer/article/1490359),
// section "Faster Transformer 优化原理": the per-layer matrix multiplies (there: cuBLAS with
// the fastest algorithm chosen per shape, on Tensor Cores in FP16) with everything
// element-wise fused around them.  Here the projections are hand-written for gfx950:
//   C[M][N] = A[M][K] * W[K][N], W held transposed (Wt[N][K], K contiguous) so both
//   operands are read along K with 16-byte loads;
//   v_mfma_f32_32x32x16_{f16,bf16} (fp32 accumulate) or v_mfma_f32_32x32x2f32 for fp32;
//   a block tile BM x BN staged through two LDS buffers that the buffer loads fill
//   directly (global memory to LDS, no register hop), 128 bytes of K per row and slab,
//   XOR-swizzled so the fragment reads are free of bank conflicts; the next slab loads
//   while the current one is multiplied; waves WM x WN each own a (BM/WM) x (BN/WN)
//   sub-tile of 32x32 accumulators;
//   the bias, the tanh GELU and the Q/K/V head split are applied in the epilogue on the
//   fp32 accumulators, so U never makes a round trip through memory before its GELU; for
//   sequences of up to 256 tokens the Q/K/V projection can also run the attention of its
//   tile in the epilogue (EpiQKVAttn), so Q, K and V never reach memory at all.
//
// MFMA operand layout used (32x32 output tile, 64 lanes, g = lane / 32):
//   first operand: lane holds row (lane % 32), VEC consecutive K values at K-offset g * VEC;
//   second operand: lane holds column (lane % 32), the same K offsets;
//   accumulator register r of a lane holds row 8*(r/4) + 4*g + (r%4), column lane % 32.
// The K order inside a fragment only has to agree between the operands, which it does by
// construction (both load K-contiguous runs at the same offsets).  The waves compute C^T
// tiles -- the weight fragment is the first operand, the activation fragment the second --
// so the four consecutive accumulator rows a lane holds are four consecutive columns n of
// one output row m; the epilogue regroups them through LDS into 16-byte row vectors.

#include <math.h>

#include <algorithm>
#include <mutex>
#include <vector>

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
// After the K loop every wave holds C^T tiles of 32x32 fp32 accumulators: register r of a
// lane holds column nt + 8 (r / 4) + 4 g + r % 4 of output row m = mt + lane % 32.  The
// epilogue object supplies
//   bias4(n)             the bias of columns n .. n+3 (read before the K loop, so its
//                        latency hides behind the matrix multiply; zeros if there is none);
//   act(v)               the element-wise work after the bias (GELU or nothing);
//   tile(mt, nt)         where the 32x32 tile at rows mt.., columns nt.. goes: its base
//                        pointer, the pointer step per staged row, and whether it is stored
//                        column-major (staged transposed) -- computed once per tile, so the
//                        divisions behind it are not repeated per element;
//   valid(mt, nt, r, c)  whether staged row r, column c (16-byte vector) is inside C;
// and the kernel stages each tile through LDS (converted to the output type) so that every
// store is 16 bytes per lane, 64 contiguous bytes per row.  N is a multiple of 8, M of the
// QKV projection a multiple of 32, so no vector straddles the end of a row.
template <typename TO> struct TileDst {
  TO* base;    // element (staged row 0, column 0)
  long step;   // elements between consecutive staged rows
  bool tr;     // staged transposed: staged rows run along n, columns along m
};

template <typename T, bool GELU, typename TO = T> struct EpiLinear {
  static constexpr bool kBlock = false;  // per-32x32-tile epilogue
  typedef TO out_t;
  typedef typename Vec16<TO>::type vec;
  typedef typename VecT<T, 4>::type b4;
  TO* c;
  const T* bias;  // may be null
  int M, N;
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (bias && n < N) v = *(const b4*)(bias + n);
    return v;
  }
  __device__ __forceinline__ float act(float v) const { return GELU ? gelu_tanh(v) : v; }
  __device__ __forceinline__ TileDst<TO> tile(int mt, int nt) const {
    return {c + (size_t)mt * N + nt, N, false};
  }
  __device__ __forceinline__ bool valid(int mt, int nt, int r, int col) const {
    return mt + r < M && nt + col < N;
  }
  // four finished columns n..n+3 of row m (the split-K reduction's store)
  __device__ __forceinline__ void store4(int m, int n, const float (&v)[4]) const {
    typename VecT<TO, 4>::type o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = from_f32<TO>(v[e]);
    *(typename VecT<TO, 4>::type*)(c + (size_t)m * N + n) = o;
  }
};

// bias + head split: a 32-column tile lies inside one of Q, K, V and inside one head (d is
// 32 or 64 and H a multiple of 32), and its 32 rows are consecutive tokens of one sequence
// (S is a multiple of 32).  Q and K are written [B][n][S][d]; V transposed per head,
// [B][n][d][S], from tiles staged column-major.  Column block c of the projection (H
// columns each) goes to slot first + c of (Q, K, V): the fused Q/K/V projection has
// first = 0 and three blocks; a cross-attention's query projection first = 0 and one, its
// key/value projection over the memory first = 1 and two.
template <typename T> struct EpiQKV {
  static constexpr bool kBlock = false;
  typedef T out_t;
  typedef typename Vec16<T>::type vec;
  typedef typename VecT<T, 4>::type b4;
  T* q;
  T* k;
  T* vt;
  const T* bias;
  int S, nh, d, M, N, first;
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (n < N) v = *(const b4*)(bias + n);
    return v;
  }
  __device__ __forceinline__ float act(float v) const { return v; }
  __device__ __forceinline__ TileDst<T> tile(int mt, int nt) const {
    const int H = nh * d;
    const int blk = nt / H, rem = nt - blk * H, which = first + blk;
    const int h = rem / d, dd0 = rem - h * d;
    const int b = mt / S, s0 = mt - b * S;
    const size_t head = (size_t)b * nh + h;
    if (which < 2) return {(which == 0 ? q : k) + (head * S + s0) * d + dd0, d, false};
    return {vt + (head * d + dd0) * S + s0, S, true};
  }
  __device__ __forceinline__ bool valid(int mt, int nt, int, int) const {
    return mt < M && nt < N;
  }
  // four finished columns n..n+3 of row m (the split-K reduction's store): they lie in one
  // head of one of Q, K, V (d is a multiple of 4)
  __device__ __forceinline__ void store4(int m, int n, const float (&v)[4]) const {
    const int H = nh * d;
    const int blk = n / H, rem = n - blk * H, which = first + blk;
    const int h = rem / d, dd = rem - h * d;
    const int b = m / S, s = m - b * S;
    const size_t head = (size_t)b * nh + h;
    if (which < 2) {
      b4 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(v[e]);
      *(b4*)((which == 0 ? q : k) + (head * S + s) * d + dd) = o;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[(head * d + dd + e) * S + s] = from_f32<T>(v[e]);
    }
  }
};

// Projection + bias + residual + LayerNorm for a hidden size of 128, where a 64 x 128 tile
// (4 waves, 2 x 2, each 32 rows x 64 columns) holds whole rows: y = LN(x + a + bias; gamma,
// beta) with a the projection (rounded to the storage type as a separate projection's
// store would be, unless A_F32: the fp32 residual stream of the 16-bit modes), the
// statistics in fp32 -- mean, then the centred sum of squares -- with the two wave columns
// of a row meeting in LDS.  TX: type of the residual x; yf (non-null): y in fp32 as well.
template <typename T, typename TX, bool A_F32> struct EpiLinearLN {
  static constexpr bool kBlock = true;
  typedef T out_t;
  typedef typename VecT<T, 4>::type b4;
  typedef typename VecT<TX, 4>::type x4;
  const TX* x;
  const T* bias;
  const T* gamma;
  const T* beta;
  T* y;
  float* yf;
  int M, N;
  static constexpr size_t kLdsBytes = 2 * 64 * 2 * sizeof(float);  // row partials of 2 passes
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (n < N) v = *(const b4*)(bias + n);
    return v;
  }
  template <int TM, int TN, int WN>
  __device__ __forceinline__ void block(char* smem, int m0, int n0, int wave, int lane,
                                        const f32x16 (&acc)[TN][TM],
                                        const b4 (&bq)[TN][4]) const {
    static_assert(TM == 1 && TN == 2 && WN == 2, "64 x 128 tile of 2 x 2 waves");
    const int wm = wave / WN, wn = wave % WN, lr = lane % 32, g = lane / 32;
    const int rl = wm * 32 + lr, row = m0 + rl;
    const bool ok = row < M;
    float* red = (float*)smem;  // [pass][64 rows][2 wave columns]
    float z[TN][16];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * g;
        x4 xv = {};
        if (ok) xv = *(const x4*)(x + (size_t)row * N + n);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float av = acc[j][0][4 * q + e] + 0.0f;
          const float a = A_F32 ? av : to_f32(from_f32<T>(av));
          z[j][4 * q + e] = to_f32(xv[e]) + a + to_f32(bq[j][q][e]);
          sum += z[j][4 * q + e];
        }
      }
    sum += __shfl_xor(sum, 32);
    if (g == 0) red[rl * 2 + wn] = sum;
    __syncthreads();
    const float inv_n = 1.0f / (float)N;
    const float mean = (red[rl * 2] + red[rl * 2 + 1]) * inv_n;
    float sq = 0.f;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float d = z[j][r] - mean;
        sq += d * d;
      }
    sq += __shfl_xor(sq, 32);
    if (g == 0) red[128 + rl * 2 + wn] = sq;
    __syncthreads();
    const float rs = rsqrtf((red[128 + rl * 2] + red[128 + rl * 2 + 1]) * inv_n + FTX_LN_EPSILON);
    if (!ok) return;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * g;
        const b4 gv = *(const b4*)(gamma + n), btv = *(const b4*)(beta + n);
        f32x4 of;
        b4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          of[e] = to_f32(gv[e]) * ((z[j][4 * q + e] - mean) * rs) + to_f32(btv[e]);
          o[e] = from_f32<T>(of[e]);
        }
        *(b4*)(y + (size_t)row * N + n) = o;
        if (yf) *(f32x4*)(yf + (size_t)row * N + n) = of;
      }
  }
};

// Projection + bias + residual, with the statistics the LayerNorm after it needs, for a
// LayerNorm folded into the next projection: z = x + a + bias is stored (rounded to the
// storage type, and in fp32 as well when zf is set) and, for each row, the mean and the
// centred sum of squares of the fp32 z over this tile's columns go to stats[row][tile
// column] -- the LayerNorm's own two-pass statistics, taken per tile; a consumer merges the
// tiles' pairs (equal-count groups: mean of means, sum of M2 plus the spread of the means).
// Whole-tile epilogue.  The residual tile comes into LDS by DMA (16-byte chunks,
// row-contiguous; chunk c of tile row R at position c ^ (R & SW) of the row, SW = 7 for rows of
// a multiple of 8 chunks, 3 for 96-column tiles, 12 chunks) while the
// accumulators take the bias; each lane adds its elements of x from LDS in the accumulator
// layout and writes z back over them in place (no other lane touches those bytes), and the
// block then stores z from LDS as 16-byte row-contiguous chunks.  The wave columns of a row
// meet in `red`, an LDS area of 2 x BM x 2 floats past the slab buffers (pre_bytes).  The
// fp32 copy goes out through a per-wave LDS scratch, 32 x 32 tiles at a time.  16-bit data,
// two wave columns at most.
template <typename T> struct EpiLinearResStats {
  static constexpr bool kBlock = true;
  typedef T out_t;
  typedef typename VecT<T, 4>::type b4;
  const T* x;       // residual [M][N]
  const T* bias;    // [N]
  T* z;             // [M][N]
  float* zf;        // [M][N] fp32 copy of z, or null
  float2* stats;    // [M][ntn]
  int M, N, ntn;
  static constexpr size_t kLdsBytes = 0;  // the tile uses the slab buffers, `red` its own area
  template <int BM, int BN> static constexpr int pre_bytes() { return 2 * BM * 2 * 4; }
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (n < N) v = *(const b4*)(bias + n);
    return v;
  }
  template <int TM, int TN, int WN, int BM>
  __device__ __forceinline__ void block(char* smem, float* red, int m0, int n0, int wave, int lane,
                                        const f32x16 (&acc)[TN][TM],
                                        const b4 (&bq)[TN][4]) const {
    static_assert(sizeof(T) == 2 && WN <= 2, "16-bit tiles, two wave columns at most");
    constexpr int BN = TN * 32 * WN;
    constexpr int CPR = BN / 8;         // 16-byte chunks per tile row
    constexpr int NCH = BM * CPR;       // chunks in the tile
    static_assert(NCH % kWave == 0, "whole wave loads");
    constexpr int ROWB = BN * 2;        // LDS bytes per tile row
    constexpr int SW = CPR % 8 == 0 ? 7 : 3;  // the chunk swizzle stays inside the row
    static_assert(CPR % 4 == 0, "rows of a multiple of 4 chunks");
    static_assert(BM * ROWB <= 2 * (BM + BN) * 128, "the tile fits the two slab buffers");
    const int nth = blockDim.x;
    const int wm = wave / WN, wn = wave % WN, lr = lane % 32, g = lane / 32;
    const int cnt = min(BN, N - n0);
    const float inv = 1.0f / (float)cnt;
    // x rows m0 .. m0 + BM - 1 (rows past M and columns past N read as zero)
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + (size_t)m0 * N), (short)0, min(BM, M - m0) * N * (int)sizeof(T), 0x00020000);
    for (int c0 = wave * kWave; c0 < NCH; c0 += nth) {
      const int c = c0 + lane, R = c / CPR, pos = c % CPR;
      const int col = n0 + ((pos ^ (R & SW)) * 8);
      const int voff = col < N ? (R * N + col) * (int)sizeof(T) : 0x7ffffff0;
      lds_dma16(rx, voff, smem + c0 * 16);
    }
    float zv[TM][TN][16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) zv[i][j][4 * q + e] = acc[j][i][4 * q + e] + to_f32(bq[j][q][e]);
    wait_vmcnt<0>();   // this wave's share of x is in LDS
    workgroup_barrier();
    // LDS byte address of this lane's 4 elements (row rl, columns 8 q + 4 g of column tile j)
    auto lds_at = [&](int rl, int j, int q) {
      const int chunk = (wn * TN + j) * 4 + q;
      return rl * ROWB + ((chunk ^ (rl & SW)) * 16) + g * 8;
    };
    float mean[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = (wm * TM + i) * 32 + lr, row = m0 + rl;
      float sum = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * g;
          const bool ok = row < M && n < N;
          const b4 xv = *(const b4*)(smem + lds_at(rl, j, q));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = ok ? zv[i][j][4 * q + e] + to_f32(xv[e]) : 0.f;
            zv[i][j][4 * q + e] = v;
            sum += v;
          }
        }
      sum += __shfl_xor(sum, 32);
      if (g == 0) red[rl * 2 + wn] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = (wm * TM + i) * 32 + lr;
      mean[i] = (WN == 2 ? red[rl * 2] + red[rl * 2 + 1] : red[rl * 2]) * inv;
      float sq = 0.f;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + (wn * TN + j) * 32 + 8 * q + 4 * g;
          b4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            o[e] = from_f32<T>(zv[i][j][4 * q + e]);
            if (n < N) {
              const float d = zv[i][j][4 * q + e] - mean[i];
              sq += d * d;
            }
          }
          *(b4*)(smem + lds_at(rl, j, q)) = o;  // z over this lane's own x
        }
      sq += __shfl_xor(sq, 32);
      if (g == 0) red[2 * BM + rl * 2 + wn] = sq;
    }
    __syncthreads();  // LDS writes (not only the barrier) complete first
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rl = (wm * TM + i) * 32 + lr, row = m0 + rl;
      if (row < M && wn == 0 && g == 0) {
        const float m2 = WN == 2 ? red[2 * BM + rl * 2] + red[2 * BM + rl * 2 + 1] : red[2 * BM + rl * 2];
        stats[(size_t)row * ntn + n0 / BN] = make_float2(mean[i], m2);
      }
    }
    typedef typename Vec16<T>::type vec;
    for (int c = threadIdx.x; c < NCH; c += nth) {
      const int R = c / CPR, ch = c % CPR, col = n0 + ch * 8;
      if (m0 + R < M && col < N)
        *(vec*)(z + (size_t)(m0 + R) * N + col) = *(const vec*)(smem + R * ROWB + ((ch ^ (R & SW)) * 16));
    }
    if (!zf) return;
    // fp32 copy: each 32 x 32 tile of the wave through its own LDS scratch (32 rows of 36
    // floats), then 8 lanes per 128-byte row segment
    __syncthreads();  // every wave's reads of the tile above are done
    float* ws = (float*)smem + wave * 32 * 36;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int mt = m0 + (wm * TM + i) * 32, nt = n0 + (wn * TN + j) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = zv[i][j][4 * q + e];
          *(f32x4*)(ws + lr * 36 + 8 * q + 4 * g) = v;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int r = p * 8 + lane / 8, cc = (lane % 8) * 4;
          const f32x4 v = *(const f32x4*)(ws + r * 36 + cc);
          if (mt + r < M && nt + cc < N) *(f32x4*)(zf + (size_t)(mt + r) * N + nt + cc) = v;
        }
      }
  }
};

// Projection of un-normalised rows z whose LayerNorm is folded in: with W' = gamma o W
// (gamma scaling the rows of W, i.e. the K index), LN(z) W + b = r (z W') + s colsum(W') +
// (b + beta W) for each row's r, s (merge_row_stats).  The weights arrive folded; csum holds
// colsum(W') of the folded, rounded weights, bias the fp32 b + beta W.  Then the activation.
template <typename T, bool GELU> struct EpiLinearNormIn {
  static constexpr bool kBlock = false;
  typedef T out_t;
  typedef typename Vec16<T>::type vec;
  typedef f32x4 b4;
  T* c;
  const float* bias;   // [N]: b + beta W
  const float* csum;   // [N]: colsum(gamma o W)
  const float2* stats; // [M][ntn]
  int ntn, bn, h;      // the producer's tile width and the normalised width (K)
  int M, N;
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (n < N) v = *(const f32x4*)(bias + n);
    return v;
  }
  __device__ __forceinline__ float act(float v) const { return GELU ? gelu_tanh(v) : v; }
  // The block's row factors (r, s) and column sums, staged in LDS after the slab buffers:
  // thread t < BM loads the stats pairs of row m0 + t, thread BM + c the column sum of
  // column n0 + c (pre_load, issued before the first slab loads), and after the prologue's
  // wait it merges and stores them (pre_store); the LDS wait and barrier every wave passes
  // before the epilogue publish them, and the epilogue reads LDS only.  Needs BM + BN <= the
  // block's threads.
  template <int BM, int BN> static constexpr int pre_bytes() { return BM * 8 + BN * 4; }
  struct PreRegs {
    float2 st[kMaxStatTiles];
    float c;
  };
  template <int BM, int BN>
  __device__ __forceinline__ PreRegs pre_load(int m0, int n0, int tid) const {
    PreRegs p;
    p.c = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxStatTiles; ++u) p.st[u] = make_float2(0.f, 0.f);
    if (tid < BM) {
      const int m = m0 + tid;
      if (m < M) {
        const float2* st = stats + (size_t)m * ntn;
#pragma unroll
        for (int u = 0; u < kMaxStatTiles; ++u)
          if (u < ntn) p.st[u] = st[u];
      }
    } else if (tid < BM + BN) {
      const int n = n0 + tid - BM;
      if (n < N) p.c = csum[n];
    }
    return p;
  }
  template <int BM, int BN>
  __device__ __forceinline__ void pre_store(const PreRegs& p, char* lds, int m0, int tid) const {
    if (tid < BM) {
      ((float2*)lds)[tid] = m0 + tid < M ? merge_row_stats<kMaxStatTiles>(p.st, ntn, bn, h, FTX_LN_EPSILON)
                                         : make_float2(0.f, 0.f);
    } else if (tid < BM + BN) {
      ((float*)(lds + BM * 8))[tid - BM] = p.c;
    }
  }
  __device__ __forceinline__ TileDst<T> tile(int mt, int nt) const {
    return {c + (size_t)mt * N + nt, N, false};
  }
  __device__ __forceinline__ bool valid(int mt, int nt, int r, int col) const {
    return mt + r < M && nt + col < N;
  }
};
template <typename E> struct is_res_stats { static constexpr bool value = false; };
template <typename T> struct is_res_stats<EpiLinearResStats<T>> { static constexpr bool value = true; };
template <typename E> struct is_norm_in { static constexpr bool value = false; };
template <typename T, bool G> struct is_norm_in<EpiLinearNormIn<T, G>> { static constexpr bool value = true; };
// LDS bytes an epilogue stages at the start of a BM x BN block (after the slab buffers), and
// the registers that carry its loads across the prologue
template <typename Epi, int BM, int BN> constexpr int epi_pre_bytes() {
  if constexpr (is_norm_in<Epi>::value || is_res_stats<Epi>::value)
    return Epi::template pre_bytes<BM, BN>();
  else return 0;
}
struct NoPre {};
template <typename Epi, bool = is_norm_in<Epi>::value> struct PreOf { typedef NoPre type; };
template <typename Epi> struct PreOf<Epi, true> { typedef typename Epi::PreRegs type; };

// Split-K partial products: the tile of K range blockIdx.y is written, unscaled and in fp32,
// to P[blockIdx.y][M][N]; splitk_reduce_kernel then sums the ranges in order and applies
// the real epilogue.
struct EpiPartial {
  static constexpr bool kBlock = false;
  typedef float out_t;
  typedef f32x4 vec;
  typedef f32x4 b4;
  float* p;
  int M, N;
  __device__ __forceinline__ b4 bias4(int) const { return b4{}; }
  __device__ __forceinline__ float act(float v) const { return v; }
  __device__ __forceinline__ TileDst<float> tile(int mt, int nt) const {
    return {p + (size_t)blockIdx.y * M * N + (size_t)mt * N + nt, N, false};
  }
  __device__ __forceinline__ bool valid(int mt, int nt, int r, int col) const {
    return mt + r < M && nt + col < N;
  }
};

// Sum of the split-K partials in split order (deterministic), then bias, activation and the
// store of the epilogue `epi`; one thread per four consecutive columns of a row.
template <typename Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P,
                                                            int splits, int M, int N, Epi epi) {
  const int64_t idx = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int q4 = N / 4;
  if (idx >= (int64_t)M * q4) return;
  const int m = (int)(idx / q4), n = (int)(idx % q4) * 4;
  const size_t mn = (size_t)M * N;
  const f32x4 acc = sum_partials4(P + (size_t)m * N + n, mn, splits);
  const auto bv = epi.bias4(n);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = epi.act(acc[e] + to_f32(bv[e]));
  epi.store4(m, n, v);
}

// Stage one C^T tile (columns nt.., rows mt..) through this wave's LDS scratch `ws`
// (32 x (32 + pad) elements of the output type) and store it as 16-byte vectors.
// Wave-private: LDS accesses of one wave complete in order.
// A normalising epilogue (is_norm_in) also takes this lane's row factors rs and the column
// sums cs of its columns 8 q + 4 g.
template <typename Epi>
__device__ __forceinline__ void epilogue_tile(const Epi& epi, typename Epi::out_t* ws, int mt,
                                              int nt, int lane, const f32x16& acc,
                                              const typename Epi::b4 (&bq)[4],
                                              float2 rs = make_float2(1.f, 0.f),
                                              const f32x4* cs = nullptr) {
  typedef typename Epi::out_t TO;
  typedef typename Epi::vec vec;
  constexpr int EV = 16 / sizeof(TO);       // elements per 16-byte vector
  constexpr int LDW = 32 + EV;              // padded LDS row
  constexpr int CPR = 32 / EV;              // vectors per 32-element row
  constexpr int RPP = kWave / CPR;          // rows per pass
  const int lr = lane % 32, g = lane / 32;
  const TileDst<TO> dst = epi.tile(mt, nt);
  typedef typename VecT<TO, 4>::type t4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int nl = 8 * q + 4 * g;           // local column of register 4q
    t4 o;
    if constexpr (is_norm_in<Epi>::value) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = from_f32<TO>(epi.act(fmaf(rs.x, acc[4 * q + e], fmaf(rs.y, cs[q][e], to_f32(bq[q][e])))));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = from_f32<TO>(epi.act(acc[4 * q + e] + to_f32(bq[q][e])));
    }
    if (dst.tr) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ws[(nl + e) * LDW + lr] = o[e];  // LDS rows run along n
    } else {
      *(t4*)(ws + lr * LDW + nl) = o;
    }
  }
#pragma unroll
  for (int p = 0; p < 32 / RPP; ++p) {
    const int row = p * RPP + lane / CPR, c = (lane % CPR) * EV;
    const vec v = *(const vec*)(ws + row * LDW + c);
    const bool ok = dst.tr ? epi.valid(mt + c, nt + row, 0, 0) : epi.valid(mt, nt, row, c);
    if (ok) *(vec*)(dst.base + (size_t)row * dst.step + c) = v;
  }
}

// ---------------------------------------------------------------------------------- kernel

// LDS row of a slab: 128 bytes of K (8 chunks of 16 bytes).  Chunk c of tile row R sits at
// position c ^ swz(R).  A wave's fragment read takes one 16-byte chunk from each of 32
// consecutive rows; with this swizzle any 8 consecutive rows hit 8 different positions and
// any 16 consecutive rows cover each (row parity, position) pair once, so the reads are free
// of bank conflicts whether the LDS serves 8 or 16 lanes per pass.  swz depends on R mod 32
// only, so the 32-row tiles of a wave differ by a constant offset.
__device__ __forceinline__ int swz(int R) { return (R & 7) ^ ((R >> 3) & 3); }

// Q/K/V projection of SEQ-token sequences (SEQ = 32, 64, 128 or 256) with head size D (64,
// or 32 with an even head count), and the attention of each (sequence, head) in the epilogue
// (the layer's first steps, section "Faster Transformer 优化原理" of the Faster Transformer
// article).  The weight rows (output columns) are ordered per head, [Q_h | K_h | V_h] for
// h = 0 .. nh-1, so the 192 columns of a tile column are exactly Q, K and V of 64 / D heads,
// and the R rows of a tile (256 with 8 waves, or 128 with 4 when the 256-row grid would
// leave half the CUs idle) are R / SEQ whole sequences.  After the K loop the tile is
// biased, rounded to the storage type (as Q, K and V are when they go through memory) and
// split in LDS into Q and K (rows of the tile's 64 head columns) and V^T (one row per head
// column, R tokens); then each of the R / 32 waves takes one block of 32 queries (wave w: sequence
// w / (SEQ/32), query block w % (SEQ/32)) and, for each head of the tile in turn, runs the
// chain of the attention kernel over all keys of its sequence: S^T = K Q^T per 32-key tile
// (D/16 MFMAs), the key mask at the sequence's valid length and the exp2 softmax on the fp32
// scores (key tiles wholly past it are skipped: their probabilities are 0), C^T = V^T P^T
// with the probabilities rounded to the storage type, and the division by the row sum; with
// the causal flag (a decoder's self-attention) query i also ignores keys j > i and key tiles
// past its own block are skipped.  Each head's context is staged in the wave's own Q rows
// and columns of that head and stored as rows of ctx[b*SEQ + i][h*D + e].  Q, K and V never
// reach global memory.
template <typename T, int SEQ, int D, int R = 256> struct EpiQKVAttn {
  static_assert(SEQ == 32 || SEQ == 64 || SEQ == 128 || SEQ == 256, "sequence length");
  static_assert((R == 128 || R == 256) && R % SEQ == 0, "whole sequences per tile");
  static_assert(D == 32 || D == 64, "head size");
  static constexpr bool kBlock = true;
  static constexpr int NKT = SEQ / 32;  // key tiles (and query blocks) per sequence
  static constexpr int HPT = 64 / D;    // heads per 192-column tile
  static constexpr int NQF = D / 16;    // 16-wide fragments along d
  static constexpr int DT = D / 32;     // 32-row tiles of the transposed context along d
  static constexpr int VPR = D / 8;     // 16-byte vectors per context row of one head
  typedef T out_t;
  typedef typename VecT<T, 4>::type b4;
  typedef typename Vec16<T>::type vec;
  T* ctx;               // [M][N / 3]
  const T* bias;        // [N], ordered like the weight rows
  const int32_t* lens;  // [M / SEQ] valid lengths, or null
  int M, N;             // M = SEQ * sequences, N = 3 * D * heads
  int s_valid;          // keys at or past it are masked in every sequence
  float scale_log2e;    // log2(e) / sqrt(D)
  int causal;           // non-zero: query i also ignores keys j > i
  // LDS: Q and K rows (the tile's 64 head columns) padded to 72 elements, V^T rows (one per
  // head column) to R + 4 tokens, so the fragment reads of 32 consecutive rows fall in
  // distinct banks
  static constexpr int QLD = 72, VLD = R + 4;
  static constexpr int KOFF = R * QLD, VOFF = 2 * R * QLD;
  static constexpr size_t kLdsBytes = (size_t)(VOFF + 64 * VLD) * sizeof(T);
  __device__ __forceinline__ b4 bias4(int n) const {
    b4 v = {};
    if (n < N) v = *(const b4*)(bias + n);
    return v;
  }
  template <int TM, int TN, int WN>
  __device__ __forceinline__ void block(char* smem, int m0, int n0, int wave, int lane,
                                        const f32x16 (&acc)[TN][TM],
                                        const b4 (&bq)[TN][4]) const {
    static_assert(TM == 2 && TN == 3 && WN == 2, "R x 192 tile of (R / 64) x 2 waves");
    typedef typename Mfma<T>::frag frag;
    T* lds = (T*)smem;
    const int wm = wave / WN, wn = wave % WN, lr = lane % 32, g = lane / 32;
    // 1. register r of accumulator (j, i): tile column c0 + 8 (r / 4) + 4 g + r % 4 of row
    //    (wm TM + i) 32 + lr; a 32-column tile lies inside one of Q, K, V of one head hh, at
    //    head column hh D + (c0 mod D) of the 64 the tile holds
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int c0 = (wn * TN + j) * 32;
      const int blk = c0 / D, hh = blk / 3, part = blk % 3, dd0 = hh * D + c0 % D;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = (wm * TM + i) * 32 + lr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int dd = dd0 + 8 * q + 4 * g;
          b4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(acc[j][i][4 * q + e] + to_f32(bq[j][q][e]));
          if (part < 2) {
            *(b4*)(lds + part * KOFF + row * QLD + dd) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) lds[VOFF + (dd + e) * VLD + row] = o[e];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
    workgroup_barrier();

    // 2. this wave's queries: tile rows r0 .. r0 + 31 of the sequence at tile row k0; no
    //    barrier follows
    const int qb = wave % NKT, k0 = (wave / NKT) * SEQ, r0 = k0 + qb * 32;
    if (m0 + k0 >= M) return;
    const int b = (m0 + k0) / SEQ;
    int len = lens ? lens[b] : s_valid;
    len = min(max(len, 1), s_valid);
    int nkt = (len + 31) / 32;
    if (causal) nkt = min(nkt, qb + 1);  // later key tiles are entirely in the future
    const int query = qb * 32 + lr;
    const int H = N / 3;
#pragma unroll
    for (int hh = 0; hh < HPT; ++hh) {
      const int hc = hh * D;  // this head's first column in the tile's Q, K and V^T
      // query lr of Q: d = 16 f + 8 g .. + 7 of fragment f
      frag qf[NQF];
#pragma unroll
      for (int f = 0; f < NQF; ++f) qf[f] = *(const frag*)(lds + (r0 + lr) * QLD + hc + 8 * g + 16 * f);
      // S^T = K Q^T per key tile: register r of sc[t] holds key 32 t + 8 (r / 4) + 4 g + r % 4
      // of query lr
      f32x16 sc[NKT];
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[t][r] = -INFINITY;
        if (t < nkt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[t][r] = 0.f;
          const T* krow = lds + KOFF + (k0 + 32 * t + lr) * QLD + hc + 8 * g;
#pragma unroll
          for (int f = 0; f < NQF; ++f) Mfma<T>::mma(*(const frag*)(krow + 16 * f), qf[f], sc[t]);
          // the per-key mask, only on a tile that reaches the valid length or (causal) the
          // query block's diagonal
          if (32 * t + 32 > len || (causal && 32 * t + 31 > qb * 32)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = 32 * t + 8 * (r / 4) + 4 * g + (r % 4);
              if (key >= len || (causal && key > query)) sc[t][r] = -INFINITY;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[t][r]);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));  // finite: key 0 is always valid
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
        if (t < nkt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            sc[t][r] = exp2_flush((sc[t][r] - mx) * scale_log2e);
            sum += sc[t][r];
          }
        }
      sum += __shfl_xor(sum, 32);
      // C^T = V^T P^T; MFMA (t, u) takes P registers 8u .. 8u+7 of key tile t = keys
      // 32 t + 16 u + {0..3, 8..11} + 4 g, against V^T rows hc + 32 dt + lr at those keys
      f32x16 o[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
#pragma unroll
      for (int t = 0; t < NKT; ++t)
        if (t < nkt) {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            frag pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = from_f32<T>(sc[t][8 * u + e]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const T* vp = lds + VOFF + (hc + 32 * dt + lr) * VLD + k0 + 32 * t + 16 * u + 4 * g;
              const b4 lo = *(const b4*)vp, hi = *(const b4*)(vp + 8);
              frag vf;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                vf[e] = lo[e];
                vf[e + 4] = hi[e];
              }
              Mfma<T>::mma(vf, pf, o[dt]);
            }
          }
        }
      // register r of o[dt]: d = 32 dt + 8 (r / 4) + 4 g + r % 4 of query lr; staged in this
      // wave's own Q rows, this head's columns (no other wave reads them, this wave reads
      // them no more; a wave's LDS accesses complete in order)
      const float inv = 1.0f / sum;
      T* st = lds + r0 * QLD + hc;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          b4 vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) vv[e] = from_f32<T>(o[dt][4 * s4 + e] * inv);
          *(b4*)(st + lr * QLD + 32 * dt + 8 * s4 + 4 * g) = vv;
        }
      T* out = ctx + (size_t)(m0 + r0) * H + ((n0 / 192) * HPT + hh) * D;
#pragma unroll
      for (int p = 0; p < 32 * VPR / kWave; ++p) {
        const int row = p * (kWave / VPR) + lane / VPR, c = (lane % VPR) * 8;
        *(vec*)(out + (size_t)row * H + c) = *(const vec*)(st + row * QLD + c);
      }
    }
  }
};

template <typename T, int BM_, int BN_, int WM, int WN> struct GemmCfg {
  static constexpr int BM = BM_, BN = BN_;
  typedef Mfma<T> MF;
  static constexpr int VEC = MF::VEC;               // elements per 16-byte chunk
  static constexpr int ROWB = 128;                  // bytes of K per tile row and slab
  static constexpr int BK = ROWB / sizeof(T);       // K per slab
  static constexpr int NS = BK / MF::KF;            // MFMA sub-steps per slab
  static constexpr int NW = WM * WN;
  static constexpr int kWN = WN;
  static constexpr int TM = BM / WM / 32;
  static constexpr int TN = BN / WN / 32;
  static constexpr int AQ = BM / 8 / NW;            // 1 KB (8-row) loads per wave and slab
  static constexpr int BQ = BN / 8 / NW;
  static constexpr int STAGE = (BM + BN) * ROWB;    // bytes per LDS buffer
  static_assert(NS == 4, "a slab holds four fragment sub-steps");
  static_assert(TM >= 1 && TN >= 1 && TM * WM * 32 == BM && TN * WN * 32 == BN, "wave tiling");
  static_assert(AQ * 8 * NW == BM && BQ * 8 * NW == BN, "slab loads not divisible");
};

// Map the linear block id to a (tile_m, tile_n): blocks are handed to the device's xcds
// XCDs round robin, so first give every XCD a contiguous range of tiles, then walk each
// range in groups of GROUP_M tile rows so the blocks resident on one XCD share A and W
// panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int xcds, int& tm,
                                            int& tn) {
  constexpr int GROUP_M = 8;
  const int nt = tiles_m * tiles_n;
  int L = bid;
  if (xcds > 1 && nt % xcds == 0) L = (bid % xcds) * (nt / xcds) + bid / xcds;
  const int per_group = GROUP_M * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = L - group * per_group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// After the K loop, with both LDS buffers free: the block epilogue, or each 32x32 tile of
// the wave staged through the wave's own share of the LDS.
template <typename C, typename Epi>
__device__ __forceinline__ void gemm_epilogue(const Epi& epi, char* smem, int m0, int n0,
                                              int wave, int lane,
                                              const f32x16 (&acc)[C::TN][C::TM],
                                              const typename Epi::b4 (&bq)[C::TN][4],
                                              const char* pre = nullptr) {
  constexpr int TM = C::TM, TN = C::TN, WN = C::kWN;
  if constexpr (Epi::kBlock) {
    static_assert(Epi::kLdsBytes <= 2 * C::STAGE, "block epilogue LDS");
    if constexpr (is_res_stats<Epi>::value)
      epi.template block<TM, TN, WN, C::BM>(smem, (float*)pre, m0, n0, wave, lane, acc, bq);
    else
      epi.template block<TM, TN, WN>(smem, m0, n0, wave, lane, acc, bq);
  } else {
    typedef typename Epi::out_t TO;
    constexpr int SCRATCH = 32 * (32 + 16 / sizeof(TO));  // elements of TO per wave
    static_assert(SCRATCH * sizeof(TO) * C::NW <= 2 * C::STAGE, "epilogue scratch");
    const int wm = wave / WN, wn = wave % WN;
    TO* ws = (TO*)smem + wave * SCRATCH;
    // the normalising epilogue's row factors and column sums, read from LDS once per row
    // tile and column tile of the wave
    const int lr = lane % 32, g = lane / 32;
    float2 rsv[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      rsv[i] = make_float2(1.f, 0.f);
      if constexpr (is_norm_in<Epi>::value) rsv[i] = ((const float2*)pre)[(wm * TM + i) * 32 + lr];
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      f32x4 csv[4] = {};
      if constexpr (is_norm_in<Epi>::value) {
        const float* csl = (const float*)(pre + C::BM * 8) + (wn * TN + j) * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) csv[q] = *(const f32x4*)(csl + 8 * q + 4 * g);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
        epilogue_tile(epi, ws, m0 + (wm * TM + i) * 32, n0 + (wn * TN + j) * 32, lane, acc[j][i],
                      bq[j], rsv[i], csv);
    }
  }
}

// K range of this block: [blockIdx.y * kchunk, min(K, (blockIdx.y + 1) * kchunk)); kchunk is
// K (one range) or, under split-K, a multiple of the slab depth.  K * BM * sizeof(T) and
// K * BN * sizeof(T) stay below 2^31 (callers bound K).
// NST LDS buffers (slab stages): slab kt + NST - 1 is loaded while slab kt is multiplied, so
// NST - 1 slabs are in flight; small tiles with a long K chain take more than two.
template <typename T, int BM, int BN, int WM, int WN, typename Epi, int NST = 2>
__global__ __launch_bounds__(WM * WN * kWave) void gemm_kernel(const T* __restrict__ A,
                                                               const T* __restrict__ Bt, int M,
                                                               int N, int K, int kchunk, int xcds,
                                                               Epi epi) {
  typedef GemmCfg<T, BM, BN, WM, WN> C;
  typedef typename C::MF MF;
  typedef typename MF::frag frag;
  constexpr int TM = C::TM, TN = C::TN, AQ = C::AQ, BQ = C::BQ, ROWB = C::ROWB;
  static_assert(NST >= 2 && NST <= 8, "slab stages");
  constexpr int PRE = epi_pre_bytes<Epi, BM, BN>();
  static_assert(BM + BN <= C::NW * kWave || !is_norm_in<Epi>::value, "one staged row or column per thread");
  __shared__ __attribute__((aligned(1024))) char smem[NST * C::STAGE + PRE];

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, xcds, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, g = lane / 32;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // this lane's bias vectors for its columns nt + 8 q + 4 g of each of its column tiles
  typename Epi::b4 bq[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[j][q] = epi.bias4(n0 + (wn * TN + j) * 32 + 8 * q + 4 * g);
  char* const pre = smem + NST * C::STAGE;
  [[maybe_unused]] typename PreOf<Epi>::type pre_regs;
  if constexpr (is_norm_in<Epi>::value) pre_regs = epi.template pre_load<BM, BN>(m0, n0, threadIdx.x);

  const int kb = blockIdx.y * kchunk;
  const int kn = min(K - kb, kchunk);
  const int nk = (kn + C::BK - 1) / C::BK;

  // Slabs go from global memory straight into LDS (no register staging).  The buffer
  // resources cover this block's row panels of A and W^T, so rows past M (N) read as zero.
  // Load q of this wave fills tile rows 8 grp .. 8 grp + 7 (grp = wave * AQ + q): lane l
  // lands at position l % 8 of row 8 grp + l / 8 and so fetches chunk (l % 8) ^ swz(row).
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (size_t)m0 * K), (short)0, min(BM, M - m0) * K * (int)sizeof(T), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)n0 * K), (short)0, min(BN, N - n0) * K * (int)sizeof(T), 0x00020000);
  int avo[AQ], bvo[BQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int R = (wave * AQ + q) * 8 + lane / 8;
    avo[q] = (R * K + kb + ((lane & 7) ^ swz(R)) * C::VEC) * (int)sizeof(T);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int R = (wave * BQ + q) * 8 + lane / 8;
    bvo[q] = (R * K + kb + ((lane & 7) ^ swz(R)) * C::VEC) * (int)sizeof(T);
  }
  auto load_slab = [&](int kt, int buf) {
    char* base = smem + buf * C::STAGE;
    const int kbytes = kt * ROWB;
#pragma unroll
    for (int q = 0; q < AQ; ++q) lds_dma16(ra, avo[q] + kbytes, base + (wave * AQ + q) * 1024);
#pragma unroll
    for (int q = 0; q < BQ; ++q)
      lds_dma16(rb, bvo[q] + kbytes, base + BM * ROWB + (wave * BQ + q) * 1024);
  };
  // A slab that runs past the block's K range (the last one, when kn is not a multiple of
  // BK) holds the next columns of each row there: zero them in both operands.
  auto zero_k_tail = [&](int buf, int kv) {
    char* base = smem + buf * C::STAGE;
    for (int it = threadIdx.x; it < (BM + BN) * 8; it += C::NW * kWave) {
      const int R = it / 8, p = it % 8;
      if ((p ^ swz(R)) * C::VEC >= kv) *(frag*)(base + R * ROWB + p * 16) = frag{};
    }
  };

  // fragment reads: row (32-row tile base + lr), chunk 2 s + g of sub-step s
  const int hl = swz(lr);
  const int a_row = (wm * TM * 32 + lr) * ROWB, b_row = BM * ROWB + (wn * TN * 32 + lr) * ROWB;
  frag fa[2][TM], fb[2][TN];
  auto read_frags = [&](int buf, int s, int set) {
    const int pos = ((2 * s + g) ^ hl) * 16;
    const char* As = smem + buf * C::STAGE + a_row + pos;
    const char* Bs = smem + buf * C::STAGE + b_row + pos;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[set][i] = *(const frag*)(As + i * 32 * ROWB);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[set][j] = *(const frag*)(Bs + j * 32 * ROWB);
  };

  // Slab kt sits in buffer kt % NST.  At the top of step kt every wave waits for its own
  // loads of slab kt (the loads of the NST - 2 later slabs may stay in flight: every wave
  // issues exactly AQ + BQ loads per slab, and loads complete in order), and the barrier
  // makes all of them visible and tells that every wave is done with buffer (kt - 1) % NST,
  // which then receives slab kt + NST - 1 while slab kt is multiplied.  Inside a slab the
  // fragments of sub-step s + 1 are read before the MFMAs of sub-step s; the scheduling
  // barriers keep the compiler from regrouping them, so LDS latency hides behind the MFMAs.
#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nk) load_slab(p, p);
  if constexpr (is_norm_in<Epi>::value) epi.template pre_store<BM, BN>(pre_regs, pre, m0, threadIdx.x);
  for (int k0 = 0; k0 < nk; k0 += NST) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int kt = k0 + u;
      if (kt < nk) {
        if (kt + NST - 2 < nk)
          wait_vmcnt<(NST - 2) * (AQ + BQ)>();
        else
          wait_vmcnt<0>();
        workgroup_barrier();
        if (kt == nk - 1 && kn - kt * C::BK < C::BK) {
          zero_k_tail(u, kn - kt * C::BK);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's zero stores done
          workgroup_barrier();
        }
        if (kt + NST - 1 < nk) load_slab(kt + NST - 1, (u + NST - 1) % NST);
        read_frags(u, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
          if (s + 1 < C::NS) read_frags(u, s + 1, (s + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int i = 0; i < TM; ++i) MF::mma(fb[s & 1][j], fa[s & 1][i], acc[j][i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  }

  // every wave is done with both buffers before the LDS is reused as epilogue scratch
  __builtin_amdgcn_s_waitcnt(0xC07F);
  workgroup_barrier();
  gemm_epilogue<C, Epi>(epi, smem, m0, n0, wave, lane, acc, bq, pre);
}

// Ping-pong K loop for the 8-wave tiles in 16-bit types (BM = 256, waves 4 x 2).  Waves w
// and w + 4 run on the same SIMD; the two groups of four waves alternate between a memory
// phase (read every fragment of a slab from LDS into registers, issue global-to-LDS loads)
// and a compute phase (the slab's 4 x TM x TN MFMAs back to back, at raised wave priority),
// half a slab apart, with a workgroup barrier between phases.  So while one wave of a SIMD
// waits on LDS and memory latency, the other keeps the matrix core busy, and no barrier
// finds both waves of a SIMD with empty MFMA queues.  Slab k sits in buffer k % 2; group 0
// reads it in phase 2k and computes it in phase 2k + 1, group 1 one phase later.  Group 0
// loads its share of slab k + 1 at the start of phase 2k (the buffer's previous slab was
// read by both groups by then) and waits for it at the end of phase 2k + 1; group 1 loads
// its share of slab k + 2 in phase 2k + 1, into the buffer of slab k, and waits for it one
// slab later.  Group 0 read slab k before the barrier that opens phase 2k + 1, but the
// other waves of group 1 read it during that phase (a wave's fragment reads span rows that
// the other waves of its group load), so each group-1 wave, its reads done, adds one to an
// LDS counter and issues its loads only once all four have (a wait inside group 1 alone;
// bounded, so that it cannot hang).  Every wave passes 2 nk + 3 barriers.  The sums are those
// of gemm_kernel, in the same order.  Needs the block's K range to be whole slabs.
template <typename T, int BM, int BN, typename Epi>
__global__ __launch_bounds__(8 * kWave) void gemm_pp_kernel(const T* __restrict__ A,
                                                            const T* __restrict__ Bt, int M,
                                                            int N, int K, int kchunk, int xcds,
                                                            Epi epi) {
  constexpr int WM = 4, WN = 2;
  typedef GemmCfg<T, BM, BN, WM, WN> C;
  typedef typename C::MF MF;
  typedef typename MF::frag frag;
  constexpr int TM = C::TM, TN = C::TN, AQ = C::AQ, BQ = C::BQ, ROWB = C::ROWB, NS = C::NS;
  constexpr int LQ = AQ + BQ;  // loads per wave and slab
  static_assert(sizeof(T) == 2 && BM == 256, "16-bit, 8-wave tiles");
  // the two slab buffers, then a counter of the group-1 waves done reading their current slab
  // (one LDS object: a second one gives the compiler alias scopes under which it waits for
  // every slab load in flight before any LDS read)
  constexpr int PRE = epi_pre_bytes<Epi, BM, BN>();
  static_assert(BM + BN <= 8 * kWave || !is_norm_in<Epi>::value, "one staged row or column per thread");
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE + 16 + PRE];
  unsigned* const g1_reads_done = (unsigned*)(smem + 2 * C::STAGE);
  char* const pre = smem + 2 * C::STAGE + 16;
  if (threadIdx.x == 0) *g1_reads_done = 0;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the store lands before the prologue's barrier

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, xcds, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  // wave-uniform, so the group's branches around barriers are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % 32, g = lane / 32;
  const int grp = wave / 4;

  f32x16 acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  const int kb = blockIdx.y * kchunk;
  const int nk = min(K - kb, kchunk) / C::BK;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (size_t)m0 * K), (short)0, min(BM, M - m0) * K * (int)sizeof(T), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)n0 * K), (short)0, min(BN, N - n0) * K * (int)sizeof(T), 0x00020000);
  int avo[AQ], bvo[BQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int R = (wave * AQ + q) * 8 + lane / 8;
    avo[q] = (R * K + kb + ((lane & 7) ^ swz(R)) * C::VEC) * (int)sizeof(T);
  }
#pragma unroll
  for (int q = 0; q < BQ; ++q) {
    const int R = (wave * BQ + q) * 8 + lane / 8;
    bvo[q] = (R * K + kb + ((lane & 7) ^ swz(R)) * C::VEC) * (int)sizeof(T);
  }
  auto load_slab = [&](int kt, int buf) {
    char* base = smem + buf * C::STAGE;
    const int kbytes = kt * ROWB;
#pragma unroll
    for (int q = 0; q < AQ; ++q) lds_dma16(ra, avo[q] + kbytes, base + (wave * AQ + q) * 1024);
#pragma unroll
    for (int q = 0; q < BQ; ++q)
      lds_dma16(rb, bvo[q] + kbytes, base + BM * ROWB + (wave * BQ + q) * 1024);
  };
  const int hl = swz(lr);
  const int a_row = (wm * TM * 32 + lr) * ROWB, b_row = BM * ROWB + (wn * TN * 32 + lr) * ROWB;
  frag fa[NS][TM], fb[NS][TN];
  auto read_slab = [&](int buf) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int pos = ((2 * s + g) ^ hl) * 16;
      const char* As = smem + buf * C::STAGE + a_row + pos;
      const char* Bs = smem + buf * C::STAGE + b_row + pos;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[s][i] = *(const frag*)(As + i * 32 * ROWB);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[s][j] = *(const frag*)(Bs + j * 32 * ROWB);
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    workgroup_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: slab 0 from every wave, group 1's share of slab 1 as well (after the epilogue's
  // staged loads, which the waits below then cover)
  [[maybe_unused]] typename PreOf<Epi>::type pre_regs;
  if constexpr (is_norm_in<Epi>::value) pre_regs = epi.template pre_load<BM, BN>(m0, n0, threadIdx.x);
  if (nk > 0) load_slab(0, 0);
  if (grp == 1 && nk > 1) {
    load_slab(1, 1);
    wait_vmcnt<LQ>();
  } else {
    wait_vmcnt<0>();
  }
  if constexpr (is_norm_in<Epi>::value) epi.template pre_store<BM, BN>(pre_regs, pre, m0, threadIdx.x);
  barrier();
  if (grp == 1) barrier();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    // memory phase
    if (grp == 0) {
      if (kt + 1 < nk) load_slab(kt + 1, buf ^ 1);
      read_slab(buf);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the fragments are in registers
    } else {
      read_slab(buf);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's reads of the buffer are done
      if (kt + 2 < nk) {
        // every group-1 wave's reads of slab kt are done before any of them loads into its
        // buffer (the counter only grows: 4 (kt + 1) arrivals by now).  Relaxed LDS atomics:
        // this wave's reads completed (lgkmcnt(0) above) before its add, and its loads issue
        // only after the count it waits for has been read; release/acquire would also wait
        // for its loads in flight (vmcnt(0)), the very loads the early issue is for.
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (lane == 0)
          __hip_atomic_fetch_add(g1_reads_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const unsigned target = 4u * (unsigned)(kt + 1);
        for (int spin = 0; spin < (1 << 16); ++spin) {
          if (__hip_atomic_load(g1_reads_done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= target)
            break;
          __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_slab(kt + 2, buf);
        wait_vmcnt<LQ>();  // its share of slab kt + 1 has landed
      } else {
        wait_vmcnt<0>();
      }
    }
    barrier();
    // compute phase
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) MF::mma(fb[s][j], fa[s][i], acc[j][i]);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (grp == 0) wait_vmcnt<0>();  // its share of slab kt + 1 has landed
    barrier();
  }

  typename Epi::b4 bq[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) bq[j][q] = epi.bias4(n0 + (wn * TN + j) * 32 + 8 * q + 4 * g);
  if (grp == 0) barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  barrier();
  gemm_epilogue<C, Epi>(epi, smem, m0, n0, wave, lane, acc, bq, pre);
}

// Small-M projection (the rows of a few short sequences): one workgroup of kSmallWaves
// waves per (32 TM) x 32 output tile, the waves splitting K.  Each wave issues the
// global-to-LDS loads of its whole K range at once (at most small_max_slabs(TM) slabs, so one
// round trip of memory latency instead of a chain of slab steps), multiplies its slabs (TM
// row tiles against one weight fragment), and the waves' fp32 partial tiles are summed in
// wave order through LDS (deterministic) and finished by the projection's own epilogue.  One
// launch where the split-K path takes a partial-product launch and a reduction launch.  K is
// a whole number of slabs.  TM = 2 (64-row tiles) where 32-row tiles would outnumber the CUs.
constexpr int kSmallWaves = 4;
// slabs a wave holds: four of 8 KB for 32-row tiles, three of 12 KB for 64-row tiles
constexpr int small_max_slabs(int tm) { return tm == 1 ? 4 : 3; }

template <typename T, typename Epi, int TM>
__global__ __launch_bounds__(kSmallWaves * kWave) void gemm_small_kernel(const T* __restrict__ A,
                                                                         const T* __restrict__ Bt,
                                                                         int M, int N, int K,
                                                                         Epi epi) {
  typedef GemmCfg<T, 32 * TM, 32, 1, 1> Cg;  // one slab: 32 TM rows of A and 32 rows of W^T
  typedef typename Cg::MF MF;
  typedef typename MF::frag frag;
  constexpr int BM = 32 * TM, ROWB = Cg::ROWB, SLAB = Cg::STAGE;
  constexpr int REGION = small_max_slabs(TM) * SLAB;
  static_assert(16 * kWave * sizeof(float) * TM + 32 * 40 * 4 <= REGION, "reduction and epilogue scratch");
  __shared__ __attribute__((aligned(1024))) char smem[kSmallWaves * REGION];
  const int tiles_n = (N + 31) / 32;
  const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * 32;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave, lr = lane % 32, g = lane / 32;
  const int nk = K / Cg::BK;
  const int spw = (nk + kSmallWaves - 1) / kSmallWaves;  // slabs per wave (<= small_max_slabs)
  const int k0 = wave * spw, k1 = min(nk, k0 + spw);
  char* const mine = smem + wave * REGION;

  typename Epi::b4 bq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bq[q] = epi.bias4(n0 + 8 * q + 4 * g);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + (size_t)m0 * K), (short)0, min(BM, M - m0) * K * (int)sizeof(T), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(Bt + (size_t)n0 * K), (short)0, min(32, N - n0) * K * (int)sizeof(T), 0x00020000);
  // load q of a slab fills rows 8 q .. 8 q + 7 (of A, then of W^T): lane l lands at position
  // l % 8 of row 8 q + l / 8 and so fetches chunk (l % 8) ^ swz(row)
  for (int kt = k0; kt < k1; ++kt) {
    char* base = mine + (kt - k0) * SLAB;
#pragma unroll
    for (int q = 0; q < 4 * TM; ++q) {
      const int R = q * 8 + lane / 8;
      lds_dma16(ra, (R * K + kt * Cg::BK + ((lane & 7) ^ swz(R)) * Cg::VEC) * (int)sizeof(T),
                base + q * 1024);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int R = q * 8 + lane / 8;
      lds_dma16(rb, (R * K + kt * Cg::BK + ((lane & 7) ^ swz(R)) * Cg::VEC) * (int)sizeof(T),
                base + BM * ROWB + q * 1024);
    }
  }
  wait_vmcnt<0>();  // this wave's slabs are in LDS (no other wave reads them)

  f32x16 acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const int hl = swz(lr);
  for (int kt = k0; kt < k1; ++kt) {
    const char* base = mine + (kt - k0) * SLAB;
#pragma unroll
    for (int st = 0; st < Cg::NS; ++st) {
      const int pos = ((2 * st + g) ^ hl) * 16;
      const frag fb = *(const frag*)(base + BM * ROWB + lr * ROWB + pos);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const frag fa = *(const frag*)(base + (32 * i + lr) * ROWB + pos);
        MF::mma(fb, fa, acc[i]);
      }
    }
  }
  // partial tiles through LDS: register r of row tile i of lane l at float (16 i + r) * 64 + l
  // of the wave's region (after its own reads, in order), summed by wave 0 in wave order
  float* red = (float*)mine;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(16 * i + r) * kWave + lane] = acc[i][r];
  __syncthreads();
  if (wave != 0) return;
  // epilogue scratch past wave 0's partials, inside its own region
  typedef typename Epi::out_t TO;
  TO* scratch = (TO*)(smem + 16 * kWave * sizeof(float) * TM);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    f32x16 sum;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum[r] = 0.f;
    for (int w = 0; w < kSmallWaves; ++w) {
      const float* pw = (const float*)(smem + w * REGION);
#pragma unroll
      for (int r = 0; r < 16; ++r) sum[r] += pw[(16 * i + r) * kWave + lane];
    }
    if (m0 + 32 * i < M) epilogue_tile(epi, scratch, m0 + 32 * i, n0, lane, sum, bq);
  }
}

// Row tiles of 32 (TM) rows per small-M workgroup for this shape, 0 where the small kernel
// does not take it: K a whole number of slabs within the waves' reach, and the workgroups no
// more than the CUs (32-row tiles first, then 64-row tiles).
template <typename T>
static int small_gemm_tm(int M, int N, int K, int cus) {
  constexpr int BK = GemmCfg<T, 32, 32, 1, 1>::BK;
  if (K % BK != 0) return 0;
  const long tn = (N + 31) / 32;
  if ((long)((M + 31) / 32) * tn <= cus && K / BK <= kSmallWaves * small_max_slabs(1)) return 1;
  if ((long)((M + 63) / 64) * tn <= cus && K / BK <= kSmallWaves * small_max_slabs(2)) return 2;
  return 0;
}

// --------------------------------------------------------------------------- tile choice
// The launch configuration is chosen per shape (the article tunes grid and block sizes to
// the number of input rows, which ranges from tens at batch 1 to thousands at batch in the
// hundreds).  Candidates, with the fraction of MFMA peak a full CU reaches in each
// (measured on the BERT-base and BERT-large projections at 16384 rows; 64x64 and 32x32 at
// 2048 to 4096 rows), and how many blocks share a CU:
//   256x256, 8 waves (4 x 2), 128 KB LDS: 0.37, 1 block per CU
//   256x192, 8 waves (4 x 2), 112 KB LDS: 0.36, 1 block per CU
//   256x128, 8 waves (4 x 2),  96 KB LDS: 0.34, 1 block per CU
//   128x128, 4 waves (2 x 2),  64 KB LDS: 0.36, 2 blocks per CU
//    64x64,  4 waves (2 x 2),  32 KB LDS: 0.25, 4 blocks per CU
//    32x32,  1 wave,           16 KB LDS: 0.18, 8 blocks per CU
// The modelled time of a launch is (rounds of blocks over the device's CUs) x (one block's
// time, longer when several blocks share a CU); the candidate with the least modelled time
// wins, so small batches get small tiles that still spread over every CU.  fp32 (twice the
// register footprint per element) uses the table without its two largest tiles.

// TILE_128x96 (4 waves of 32 x 96) is not a candidate of the cost model: plan_gemm takes it in
// place of 128x128 where its grid fits two blocks per CU (below).
enum TileCfg { TILE_256x256, TILE_256x192, TILE_256x128, TILE_128x128, TILE_64x64, TILE_32x32,
               TILE_128x96, TILE_COUNT };
static const int kTileM[TILE_COUNT] = {256, 256, 256, 128, 64, 32, 128};
static const int kTileN[TILE_COUNT] = {256, 192, 128, 128, 64, 32, 96};

static TileCfg choose_tile(int M, int N, bool wide, int cus) {
  struct Cand { int bm, bn, per_cu; double eff; };
  static const Cand cand[TILE_32x32 + 1] = {{256, 256, 1, 0.37}, {256, 192, 1, 0.36}, {256, 128, 1, 0.34},
                                            {128, 128, 2, 0.36}, {64, 64, 4, 0.25},   {32, 32, 8, 0.18}};
  const long kCUs = std::max(cus, 1);
  int best = TILE_32x32;
  double best_t = 1e300;
  for (int c = wide ? 0 : TILE_256x128; c <= TILE_32x32; ++c) {
    const Cand& x = cand[c];
    const long tiles = (long)((M + x.bm - 1) / x.bm) * ((N + x.bn - 1) / x.bn);
    const long rounds = (tiles + (long)kCUs * x.per_cu - 1) / ((long)kCUs * x.per_cu);
    // blocks that share a CU in a round: up to per_cu, but no more than the grid puts there
    const long share = std::min<long>(x.per_cu, (tiles + kCUs - 1) / kCUs);
    // a block's time: its tile's work (MFMAs run on the whole tile, also on rows past M) at
    // its efficiency, shared with the other blocks on its CU
    const double t = (double)rounds * x.bm * x.bn * share / x.eff;
    if (t < best_t * 0.999) {
      best_t = t;
      best = c;
    }
  }
  return (TileCfg)best;
}

// Split-K (the small-batch path): when the chosen configuration has fewer tiles than there
// are CUs, K is cut into up to 16 ranges of at least two slabs each, so that about twice as
// many blocks as CUs run (512 on 256 CUs).  When it has more tiles than CUs but fewer waves than SIMDs (only 32x32
// tiles, one wave each, reach this), K is cut so that about one wave per SIMD runs -- but
// only where the LayerNorm after the projection sums the partials (no reduction launch)
// and its rows are at least 256 wide.  Measured in whole forwards against splitting below
// 256 tiles only (same box): BERT-base B12 0.683 -> 0.529 ms, B16 0.653 -> 0.518, BERT-large
// S512 B1 2.346 -> 1.796, S128 B2 2.264 -> 1.436, the decoder B16 1.205 -> 1.029.  Losses
// that set the conditions: the same split with a reduction launch (Q/K/V and FFN-in at 128
// rows, S128 B1 0.500 -> 0.551), hidden size 128 (the 4x32 model B64 0.297 -> 0.317, B128
// 0.328 -> 0.372), 384 four-wave 64x64 tiles at B64 cut in two (0.813 -> 0.845), and
// filling the SIMDs below 256 tiles too (B8: 6 splits of two slabs, not 3 of four, 0.548 ->
// 0.561).
// The partial products go to an fp32 workspace [splits][M][N] and a reduction kernel (or
// the LayerNorm that follows) finishes them.  The partials are capped at 16 MiB, at 4 MiB
// where a reduction launch finishes them (fewer splits, or none): their round trip through memory must stay small
// against what the split saves -- at 4096 rows a 6-way split of the 768-wide projections
// would move 75 MB and lose.  Without a workspace of the planned size the GEMM is not
// split.  Even a short K chain gains: the split spreads the reads of weights that arrive
// cold from memory over six times the blocks (BERT-base batch 1, K = 768 unsplit: 0.481
// against 0.463 ms per forward), although the same projection repeated on weights already
// in L2 runs faster unsplit (4.6 against 7.5 us).
struct GemmPlan {
  TileCfg cfg;
  int splits;  // 1 = no split
  int kchunk;  // K elements per split (K when splits == 1)
};

constexpr size_t kMaxPartialBytes = 16u << 20;
constexpr int kSmallTileDeepSlabsPlan = 12;  // = kSmallTileDeepSlabs
// A split finished by a reduction launch also pays that launch and the second read of the
// partials: above 4 MiB of partials it lost in whole forwards (BERT-base B8, FFN-in at 256
// rows cut in three, 9 MiB: 0.551 against 0.511 ms unsplit; S64 B4 0.563 against 0.523;
// the decoder B8 0.987 against 0.911).
constexpr size_t kMaxReducedPartialBytes = 4u << 20;

// sums_partials: the kernel after this projection sums its partials itself (the split-K
// LayerNorm), so a split costs no reduction launch.
static GemmPlan plan_gemm(int M, int N, int K, int elem_bytes, bool sums_partials, int cus) {
  const long kCUs = std::max(cus, 1), kSIMDs = 4 * kCUs;
  GemmPlan p{choose_tile(M, N, elem_bytes == 2, cus), 1, K};
  const int bk = 128 / elem_bytes;
  const long tiles = (long)((M + kTileM[p.cfg] - 1) / kTileM[p.cfg]) * ((N + kTileN[p.cfg] - 1) / kTileN[p.cfg]);
  const int nk = (K + bk - 1) / bk;
  static const int waves[TILE_COUNT] = {8, 8, 8, 4, 4, 1, 4};
  const bool fill_simds = sums_partials && N >= 256 && tiles * waves[p.cfg] < kSIMDs;
  if ((tiles < kCUs || fill_simds) && nk >= 4) {
    const size_t max_partial_bytes = sums_partials ? kMaxPartialBytes : kMaxReducedPartialBytes;
    const long by_bytes = (long)(max_partial_bytes / ((size_t)M * N * sizeof(float)));
    const long wv = tiles * waves[p.cfg];
    const long fill = tiles < kCUs ? (2 * kCUs + tiles - 1) / tiles : (kSIMDs + wv - 1) / wv;
    int sp = (int)std::min<long>(std::min<long>(fill, nk / 2),
                                 std::min<long>(16, by_bytes));
    if (sp > 1) {
      p.kchunk = (nk + sp - 1) / sp * bk;
      p.splits = (K + p.kchunk - 1) / p.kchunk;
    }
    // one-wave 32x32 blocks left with a K chain of 32 slabs or more: 64x64 blocks (4 waves
    // sharing each slab), split again for their own grid (BERT-large S512 B1, FFN-out 512 x
    // 1024 x 4096: 2 splits of 32 slabs -> 4 of 16; with the three-stage 32x32 rule, whole
    // forwards 1.675 -> 1.476 ms on one box)
    if (p.cfg == TILE_32x32 && fill_simds && p.kchunk / bk >= 32) {
      const long t64 = (long)((M + 63) / 64) * ((N + 63) / 64);
      const long f64 = t64 < kCUs ? (2 * kCUs + t64 - 1) / t64 : (kSIMDs + 4 * t64 - 1) / (4 * t64);
      const int sp64 = (int)std::min<long>(std::min<long>(f64, nk / 2), std::min<long>(16, by_bytes));
      p.cfg = TILE_64x64;
      p.splits = 1;
      p.kchunk = K;
      if (sp64 > 1) {
        p.kchunk = (nk + sp64 - 1) / sp64 * bk;
        p.splits = (K + p.kchunk - 1) / p.kchunk;
      }
    }
  }
  // An unsplit 16-bit 128x128 grid, N a multiple of 96, whose 128x96 grid still fits two
  // blocks per CU: 128x96 tiles cover the same rows with more blocks -- one per CU on three
  // LDS stages from 12 slabs, or two per CU on two.  BERT-base 4096 x 768 x 3072 alone: 27.9
  // -> 25.7 us (192 -> 256 tiles); 4096 x 768 x 768: 9.8 -> 8.9 us; 8192 x 768 x 3072: 44.5
  // -> 41.8 us (384 -> 512); 6144 x 768 x 3072 39.5 -> 37.2, x 768 13.5 -> 12.2.
  if (p.cfg == TILE_128x128 && p.splits == 1 && elem_bytes == 2 && N % 96 == 0 &&
      nk >= kSmallTileDeepSlabsPlan && (long)((M + 127) / 128) * (N / 96) <= 2 * kCUs)
    p.cfg = TILE_128x96;
  return p;
}

DeviceInfo device_info() {
  static std::mutex mu;
  static std::vector<DeviceInfo> cache;  // per device id; cus == 0: not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return {1, 1};
  }
  std::lock_guard<std::mutex> lock(mu);
  if ((size_t)dev < cache.size() && cache[dev].cus > 0) return cache[dev];
  hipDeviceProp_t prop;
  int xcds = 1;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess || prop.multiProcessorCount < 1) {
    (void)hipGetLastError();
    return {1, 1};
  }
  if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) {
    (void)hipGetLastError();
    xcds = 1;
  }
  if ((size_t)dev >= cache.size()) cache.resize(dev + 1, DeviceInfo{0, 0});
  cache[dev] = {prop.multiProcessorCount, xcds};
  return cache[dev];
}

size_t gemm_splitk_workspace(ftx_dtype dt, int M, int N, int K) {
  const int cus = device_info().cus;
  size_t need = 0;
  for (bool sums : {false, true}) {
    const GemmPlan p = plan_gemm(M, N, K, dt == FTX_FP32 ? 4 : 2, sums, cus);
    if (p.splits > 1) need = std::max(need, (size_t)p.splits * M * N);
  }
  return need;
}

void plan_linear(ftx_dtype dt, int M, int N, int K, int cus, bool sums_partials, int* tile_m,
                 int* tile_n, int* splits) {
  const GemmPlan p = plan_gemm(M, N, K, dt == FTX_FP32 ? 4 : 2, sums_partials, cus);
  *tile_m = kTileM[p.cfg];
  *tile_n = kTileN[p.cfg];
  *splits = p.splits;
}

// The ping-pong K loop from 12 slabs (K >= 768 in 16-bit).  Measured in whole forwards,
// against the two-buffer loop on the same box: BERT-base S32 B512 3.242 -> 3.215 ms (FFN-in
// alone 94.0 -> 91.2 us), S128 B64 2.165 -> 2.128, S64 B64 1.222 -> 1.210, the decoder B512
// 4.875 -> 4.777; BERT-large (K = 1024) Q/K/V 202 -> 195 us, FFN-out at K = 3072-4096 7-15%
// faster.  (A 256x192 projection repeated alone on weights already in L2 runs 0-4% slower
// at 12 slabs; in the forward it gains.)
constexpr int kPingPongMinSlabs = 12;

// A 64x64 tile multiplies 64 x 64 x 64 per slab, far less than the latency of the slab's
// loads: with 12 slabs or more per block it keeps two slabs in flight (three LDS stages,
// 48 KB).  Measured on whole forwards against two stages (same box): BERT-base B64 0.814 ->
// 0.805 ms, B16 0.670 -> 0.653, the decoder B64 1.516 -> 1.455; the FFN-out projection at
// batch 64 (2048 x 768 x 3072) alone 24.8 -> 20.6 us.
constexpr int kSmallTileDeepSlabs = 12;

// A 128x128 grid with no more blocks than the GPU has CUs runs one block per CU whatever its
// LDS, so from 12 slabs it takes three stages (96 KB) instead of two (64 KB, which would let
// two blocks share a CU).  Measured on whole forwards against two stages (same box):
// BERT-base S32 B128 1.203 -> 1.129 ms and S64 B64 1.232 -> 1.147 (4096 rows: the
// attention-output and FFN-out projections on 192 tiles).  With more tiles than CUs three
// stages lose (6144 rows 1.82 -> 2.03 ms, 8192 rows 2.19 -> 2.33): a second round of blocks
// replaces the second block per CU.

template <typename T, int BM, int BN, int WM, int WN, typename Epi>
static void gemm_kernel_launch(dim3 grid, int kchunk, int M, int N, int K, const void* a,
                               const void* w_t, Epi epi, int xcds, hipStream_t s) {
  constexpr int BK = GemmCfg<T, BM, BN, WM, WN>::BK;
  if constexpr (BM == 64 && BN == 64) {
    if ((kchunk + BK - 1) / BK >= kSmallTileDeepSlabs) {
      gemm_kernel<T, BM, BN, WM, WN, Epi, 3><<<grid, WM * WN * kWave, 0, s>>>(
          (const T*)a, (const T*)w_t, M, N, K, kchunk, xcds, epi);
      return;
    }
  }
  if constexpr (BM == 128 && (BN == 128 || BN == 96)) {
    if ((kchunk + BK - 1) / BK >= kSmallTileDeepSlabs &&
        (int64_t)grid.x * grid.y <= device_info().cus) {
      gemm_kernel<T, BM, BN, WM, WN, Epi, 3><<<grid, WM * WN * kWave, 0, s>>>(
          (const T*)a, (const T*)w_t, M, N, K, kchunk, xcds, epi);
      return;
    }
  }
  if constexpr (BM == 32 && BN == 32) {
    // a one-wave block with a K chain of 12 slabs or more keeps two slabs in flight (three
    // 8 KB stages), as the 64x64 tile does: BERT-large S512 B1 1.674 -> 1.549 ms, BERT-base
    // B8 0.470 -> 0.444 (whole forwards, same box), B1 and B16 unchanged
    if ((kchunk + BK - 1) / BK >= kSmallTileDeepSlabs) {
      gemm_kernel<T, BM, BN, WM, WN, Epi, 3><<<grid, WM * WN * kWave, 0, s>>>(
          (const T*)a, (const T*)w_t, M, N, K, kchunk, xcds, epi);
      return;
    }
    // a split-K block of at most three slabs loads them all before its first multiply (four
    // 8 KB stages): one memory round trip instead of one per slab
    if (grid.y > 1 && (kchunk + BK - 1) / BK <= 3) {
      gemm_kernel<T, BM, BN, WM, WN, Epi, 4><<<grid, WM * WN * kWave, 0, s>>>(
          (const T*)a, (const T*)w_t, M, N, K, kchunk, xcds, epi);
      return;
    }
  }
  gemm_kernel<T, BM, BN, WM, WN, Epi><<<grid, WM * WN * kWave, 0, s>>>(
      (const T*)a, (const T*)w_t, M, N, K, kchunk, xcds, epi);
}

// reduce: under split-K, also launch the reduction that finishes the partials with `epi`
// (false: the caller's next kernel consumes the partials itself).
template <typename T, int BM, int BN, int WM, int WN, typename Epi>
static hipError_t gemm_launch_cfg(int M, int N, int K, const void* a, const void* w_t, Epi epi,
                                  const GemmPlan& plan, float* ws, int xcds, hipStream_t s,
                                  bool reduce) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  if (plan.splits > 1) {
    gemm_kernel_launch<T, BM, BN, WM, WN, EpiPartial>(dim3(tiles, plan.splits), plan.kchunk, M, N,
                                                      K, a, w_t, EpiPartial{ws, M, N}, xcds, s);
    if (reduce) {
      const int64_t threads = (int64_t)M * (N / 4);
      splitk_reduce_kernel<Epi><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(ws, plan.splits, M, N, epi);
    }
    return hipGetLastError();
  }
  if constexpr (sizeof(T) == 2 && BM == 256 && WM == 4 && WN == 2) {
    constexpr int BK = GemmCfg<T, BM, BN, WM, WN>::BK;
    if (K % BK == 0 && K / BK >= kPingPongMinSlabs) {
      gemm_pp_kernel<T, BM, BN, Epi><<<tiles, WM * WN * kWave, 0, s>>>(
          (const T*)a, (const T*)w_t, M, N, K, K, xcds, epi);
      return hipGetLastError();
    }
  }
  gemm_kernel_launch<T, BM, BN, WM, WN, Epi>(dim3(tiles), K, M, N, K, a, w_t, epi, xcds, s);
  return hipGetLastError();
}

template <typename T, typename Epi>
static hipError_t gemm_launch(int M, int N, int K, const void* a, const void* w_t, Epi epi,
                              hipStream_t s, float* ws = nullptr, size_t ws_elems = 0,
                              bool reduce = true) {
  constexpr bool wide = sizeof(T) == 2;
  const DeviceInfo di = device_info();
  GemmPlan plan = plan_gemm(M, N, K, (int)sizeof(T), !reduce, di.cus);
  // where the plan splits K and finishes with a reduction launch, or runs one-wave 32x32
  // blocks each through its whole K chain, few rows take the small-M kernel instead (one
  // launch, one round trip of loads, no workspace)
  if constexpr (!Epi::kBlock) {
    const bool small = reduce && (plan.splits > 1 || plan.cfg == TILE_32x32);
    const int tm = small ? small_gemm_tm<T>(M, N, K, di.cus) : 0;
    if (tm) {
      const int tiles = ((M + 32 * tm - 1) / (32 * tm)) * ((N + 31) / 32);
      if (tm == 1)
        gemm_small_kernel<T, Epi, 1><<<tiles, kSmallWaves * kWave, 0, s>>>((const T*)a, (const T*)w_t,
                                                                           M, N, K, epi);
      else
        gemm_small_kernel<T, Epi, 2><<<tiles, kSmallWaves * kWave, 0, s>>>((const T*)a, (const T*)w_t,
                                                                           M, N, K, epi);
      return hipGetLastError();
    }
  }
  if (plan.splits > 1 && (!ws || ws_elems < (size_t)plan.splits * M * N)) {
    plan.splits = 1;
    plan.kchunk = K;
  }
  switch (plan.cfg) {
    case TILE_256x256:
      if constexpr (wide) return gemm_launch_cfg<T, 256, 256, 4, 2>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
      break;
    case TILE_256x192:
      if constexpr (wide) return gemm_launch_cfg<T, 256, 192, 4, 2>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
      break;
    case TILE_256x128: return gemm_launch_cfg<T, 256, 128, 4, 2>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
    case TILE_128x128: return gemm_launch_cfg<T, 128, 128, 2, 2>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
    case TILE_64x64: return gemm_launch_cfg<T, 64, 64, 2, 2>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
    case TILE_32x32: return gemm_launch_cfg<T, 32, 32, 1, 1>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
    case TILE_128x96:
      if constexpr (sizeof(T) == 2) return gemm_launch_cfg<T, 128, 96, 4, 1>(M, N, K, a, w_t, epi, plan, ws, di.xcds, s, reduce);
      break;
    default: break;
  }
  return hipErrorInvalidValue;
}

int linear_splits(ftx_dtype dt, int M, int N, int K, size_t ws_elems, bool sums_partials) {
  const GemmPlan p = plan_gemm(M, N, K, dt == FTX_FP32 ? 4 : 2, sums_partials, device_info().cus);
  return (p.splits > 1 && ws_elems >= (size_t)p.splits * M * N) ? p.splits : 1;
}

hipError_t launch_linear_partials(ftx_dtype dt, int M, int N, int K, const void* a,
                                  const void* w_t, float* ws, size_t ws_elems, hipStream_t s) {
  if (linear_splits(dt, M, N, K, ws_elems, true) < 2) return hipErrorInvalidValue;
  // the epilogue only serves the reduction, which is not launched
  switch (dt) {
    case FTX_FP32:
      return gemm_launch<float>(M, N, K, a, w_t, EpiLinear<float, false>{nullptr, nullptr, M, N}, s, ws, ws_elems, false);
    case FTX_FP16:
      return gemm_launch<f16>(M, N, K, a, w_t, EpiLinear<f16, false>{nullptr, nullptr, M, N}, s, ws, ws_elems, false);
    case FTX_BF16:
      return gemm_launch<bf16>(M, N, K, a, w_t, EpiLinear<bf16, false>{nullptr, nullptr, M, N}, s, ws, ws_elems, false);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t linear_t(int M, int N, int K, const void* a, const void* w_t, const void* bias,
                           bool gelu, bool out_f32, void* c, hipStream_t s, float* ws,
                           size_t wn) {
  if (out_f32) {
    if (gelu) return hipErrorInvalidValue;  // the GELU output is stored in the data type
    return gemm_launch<T>(M, N, K, a, w_t, EpiLinear<T, false, float>{(float*)c, (const T*)bias, M, N}, s, ws, wn);
  }
  if (gelu) return gemm_launch<T>(M, N, K, a, w_t, EpiLinear<T, true>{(T*)c, (const T*)bias, M, N}, s, ws, wn);
  return gemm_launch<T>(M, N, K, a, w_t, EpiLinear<T, false>{(T*)c, (const T*)bias, M, N}, s, ws, wn);
}

hipError_t launch_linear(ftx_dtype dt, int M, int N, int K, const void* a, const void* w_t,
                         const void* bias, bool gelu, void* c, hipStream_t s, bool out_f32,
                         float* ws, size_t ws_elems) {
  switch (dt) {
    case FTX_FP32: return linear_t<float>(M, N, K, a, w_t, bias, gelu, false, c, s, ws, ws_elems);
    case FTX_FP16: return linear_t<f16>(M, N, K, a, w_t, bias, gelu, out_f32, c, s, ws, ws_elems);
    case FTX_BF16: return linear_t<bf16>(M, N, K, a, w_t, bias, gelu, out_f32, c, s, ws, ws_elems);
  }
  return hipErrorInvalidValue;
}

template <int BM_, int BN_, int WM_, int WN_> struct TileShape {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
};

// The projection on the tile the planner picks, unsplit (for epilogues that have no split-K
// form); hipErrorInvalidValue where the plan would split K.
template <typename T, typename Epi>
static hipError_t gemm_launch_whole(int M, int N, int K, const void* a, const void* w_t, Epi epi,
                                    hipStream_t s) {
  const DeviceInfo di = device_info();
  const GemmPlan plan = plan_gemm(M, N, K, (int)sizeof(T), false, di.cus);
  if (plan.splits > 1) return hipErrorInvalidValue;
  auto run = [&](auto cfg) -> hipError_t {
    constexpr int BM = decltype(cfg)::BM, BN = decltype(cfg)::BN, WM = decltype(cfg)::WM, WN = decltype(cfg)::WN;
    const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if constexpr (sizeof(T) == 2 && BM == 256 && WM == 4 && WN == 2) {
      constexpr int BK = GemmCfg<T, BM, BN, WM, WN>::BK;
      if (K % BK == 0 && K / BK >= kPingPongMinSlabs) {
        gemm_pp_kernel<T, BM, BN, Epi><<<tiles, WM * WN * kWave, 0, s>>>(
            (const T*)a, (const T*)w_t, M, N, K, K, di.xcds, epi);
        return hipGetLastError();
      }
    }
    gemm_kernel_launch<T, BM, BN, WM, WN, Epi>(dim3(tiles), K, M, N, K, a, w_t, epi, di.xcds, s);
    return hipGetLastError();
  };
  switch (plan.cfg) {
    case TILE_256x256: if constexpr (sizeof(T) == 2) return run(TileShape<256, 256, 4, 2>{}); break;
    case TILE_256x192: if constexpr (sizeof(T) == 2) return run(TileShape<256, 192, 4, 2>{}); break;
    case TILE_256x128: return run(TileShape<256, 128, 4, 2>{});
    case TILE_128x128: return run(TileShape<128, 128, 2, 2>{});
    case TILE_128x96: if constexpr (sizeof(T) == 2) return run(TileShape<128, 96, 4, 1>{}); break;
    case TILE_64x64: return run(TileShape<64, 64, 2, 2>{});
    default: break;  // 32x32 tiles: one wave holds a row's columns alone, not supported here
  }
  return hipErrorInvalidValue;
}

hipError_t launch_linear_residual_stats(ftx_dtype dt, int M, int N, int K, const void* a,
                                        const void* w_t, const void* bias, const void* x,
                                        void* z, float* zf, float* stats, int ntn, hipStream_t s) {
  int tm, tn, sp;
  plan_linear(dt, M, N, K, device_info().cus, false, &tm, &tn, &sp);
  if (sp != 1 || ntn != (N + tn - 1) / tn || ntn > kMaxStatTiles || N % 8) return hipErrorInvalidValue;
  switch (dt) {
    case FTX_FP16: return gemm_launch_whole<f16>(M, N, K, a, w_t,
        EpiLinearResStats<f16>{(const f16*)x, (const f16*)bias, (f16*)z, zf, (float2*)stats, M, N, ntn}, s);
    case FTX_BF16: return gemm_launch_whole<bf16>(M, N, K, a, w_t,
        EpiLinearResStats<bf16>{(const bf16*)x, (const bf16*)bias, (bf16*)z, zf, (float2*)stats, M, N, ntn}, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_linear_norm_in(ftx_dtype dt, int M, int N, int K, const void* z,
                                 const void* w_t, const float* bias, const float* csum,
                                 const float* stats, int ntn, int bn, bool gelu, void* c,
                                 hipStream_t s) {
  if (ntn < 1 || ntn > kMaxStatTiles || bn < 1 || (K + bn - 1) / bn != ntn) return hipErrorInvalidValue;
  const float2* st = (const float2*)stats;
  switch (dt) {
    case FTX_FP16:
      if (gelu) return gemm_launch_whole<f16>(M, N, K, z, w_t, EpiLinearNormIn<f16, true>{(f16*)c, bias, csum, st, ntn, bn, K, M, N}, s);
      return gemm_launch_whole<f16>(M, N, K, z, w_t, EpiLinearNormIn<f16, false>{(f16*)c, bias, csum, st, ntn, bn, K, M, N}, s);
    case FTX_BF16:
      if (gelu) return gemm_launch_whole<bf16>(M, N, K, z, w_t, EpiLinearNormIn<bf16, true>{(bf16*)c, bias, csum, st, ntn, bn, K, M, N}, s);
      return gemm_launch_whole<bf16>(M, N, K, z, w_t, EpiLinearNormIn<bf16, false>{(bf16*)c, bias, csum, st, ntn, bn, K, M, N}, s);
    default: break;
  }
  return hipErrorInvalidValue;
}

template <typename T, typename TX, bool A_F32>
static hipError_t linear_ln_t(int M, int K, const void* a, const void* w_t, const void* x,
                              const void* bias, const void* gamma, const void* beta, void* y,
                              float* yf, hipStream_t s) {
  constexpr int N = 128;
  typedef EpiLinearLN<T, TX, A_F32> Epi;
  Epi epi{(const TX*)x, (const T*)bias, (const T*)gamma, (const T*)beta, (T*)y, yf, M, N};
  gemm_kernel<T, 64, 128, 2, 2, Epi><<<(M + 63) / 64, 4 * kWave, 0, s>>>(
      (const T*)a, (const T*)w_t, M, N, K, K, device_info().xcds, epi);
  return hipGetLastError();
}

hipError_t launch_linear_layernorm(ftx_dtype dt, int M, int N, int K, const void* a,
                                   const void* w_t, const void* x, bool x_f32, bool a_f32,
                                   const void* bias, const void* gamma, const void* beta,
                                   void* y, float* yf, hipStream_t s) {
  if (N != 128 || M < 1 || K < 8 || K % 8 || K > kMaxInnerDim) return hipErrorInvalidValue;
  if (x_f32 && !a_f32) return hipErrorInvalidValue;
  switch (dt) {
    case FTX_FP32:
      return linear_ln_t<float, float, true>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
    case FTX_FP16:
      if (x_f32) return linear_ln_t<f16, float, true>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
      if (a_f32) return linear_ln_t<f16, f16, true>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
      return linear_ln_t<f16, f16, false>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
    case FTX_BF16:
      if (x_f32) return linear_ln_t<bf16, float, true>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
      if (a_f32) return linear_ln_t<bf16, bf16, true>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
      return linear_ln_t<bf16, bf16, false>(M, K, a, w_t, x, bias, gamma, beta, y, yf, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t heads_t(int B, int S, int nh, int d, const void* x, const void* w, const void* b,
                          int first, int count, void* q, void* k, void* vt, hipStream_t s,
                          float* ws, size_t wn) {
  const int M = B * S, H = nh * d;
  EpiQKV<T> epi{(T*)q, (T*)k, (T*)vt, (const T*)b, S, nh, d, M, count * H, first};
  return gemm_launch<T>(M, count * H, H, x, w, epi, s, ws, wn);
}

hipError_t launch_head_projection(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                  const void* w_t, const void* bias, int first, int count,
                                  void* q, void* k, void* vt, hipStream_t s, float* ws,
                                  size_t ws_elems) {
  if (first < 0 || count < 1 || first + count > 3) return hipErrorInvalidValue;
  switch (dt) {
    case FTX_FP32: return heads_t<float>(B, S, nh, d, x, w_t, bias, first, count, q, k, vt, s, ws, ws_elems);
    case FTX_FP16: return heads_t<f16>(B, S, nh, d, x, w_t, bias, first, count, q, k, vt, s, ws, ws_elems);
    case FTX_BF16: return heads_t<bf16>(B, S, nh, d, x, w_t, bias, first, count, q, k, vt, s, ws, ws_elems);
  }
  return hipErrorInvalidValue;
}

bool qkv_attention_fits(ftx_dtype dt, int S, int nh, int d) {
  return dt != FTX_FP32 && (S == 32 || S == 64 || S == 128 || S == 256) &&
         (d == 64 || (d == 32 && nh % 2 == 0));
}

template <typename T, int SEQ, int D>
static hipError_t qkv_attention_t(int B, int nh, const void* x, const void* w_t, const void* bias,
                                  const int32_t* lens, int s_valid, int causal, void* ctx,
                                  hipStream_t s) {
  const int M = SEQ * B, N = 3 * D * nh, K = D * nh;
  // log2(e) / sqrt(d), rounded once from double as the attention kernel does
  const float scale_log2e = (float)(1.4426950408889634 / sqrt((double)D));
  const int tiles = ((M + 255) / 256) * (N / 192);
  const DeviceInfo di = device_info();
  if constexpr (SEQ <= 128) {
    // 128-row tiles of 4 waves while twice the tiles still fit one per CU (BERT-base S32
    // at batch 64 on 256 CUs: 96 tiles of 256 rows -> 192 of 128, 0.849 -> 0.806 ms; at
    // S64, 192 tiles of 256 rows would become 384 sharing CUs: 1.267 -> 1.287 ms, so they
    // stay), and where the 256-row grid's last round would run at most half full: two
    // 128-row blocks per CU then finish in the time of the full rounds, and each block's
    // attention overlaps the other's K loop.  Alone on 256 CUs (S32, d 64, 12 heads):
    // 6144 rows 38.2 -> 33.7 us, 8192 rows 40.7 -> 36.5, 12288 rows 62.8 -> 55.7; S128 8192
    // rows 42.0 -> 40.5; against 240 tiles 22.7 -> 24.1, 480 tiles 43.5 -> 45.0 and 768
    // tiles 67.9 -> 68.1, where the 256-row grid stays.
    const int rem = tiles % di.cus;
    if (2 * tiles <= di.cus || (tiles > di.cus && rem != 0 && 2 * rem <= di.cus)) {
      typedef EpiQKVAttn<T, SEQ, D, 128> Epi128;
      Epi128 epi{(T*)ctx, (const T*)bias, lens, M, N, s_valid, scale_log2e, causal};
      gemm_kernel<T, 128, 192, 2, 2, Epi128><<<((M + 127) / 128) * (N / 192), 4 * kWave, 0, s>>>(
          (const T*)x, (const T*)w_t, M, N, K, K, di.xcds, epi);
      return hipGetLastError();
    }
  }
  EpiQKVAttn<T, SEQ, D> epi{(T*)ctx, (const T*)bias, lens, M, N, s_valid, scale_log2e, causal};
  constexpr int BK = GemmCfg<T, 256, 192, 4, 2>::BK;
  if (K % BK == 0 && K / BK >= kPingPongMinSlabs)
    gemm_pp_kernel<T, 256, 192, EpiQKVAttn<T, SEQ, D>><<<tiles, 8 * kWave, 0, s>>>(
        (const T*)x, (const T*)w_t, M, N, K, K, di.xcds, epi);
  else
    gemm_kernel<T, 256, 192, 4, 2, EpiQKVAttn<T, SEQ, D>><<<tiles, 8 * kWave, 0, s>>>(
        (const T*)x, (const T*)w_t, M, N, K, K, di.xcds, epi);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t qkv_attention_s(int B, int S, int nh, const void* x, const void* w_t,
                                  const void* bias, const int32_t* lens, int s_valid, int causal,
                                  void* ctx, hipStream_t s) {
  switch (S) {
    case 32: return qkv_attention_t<T, 32, D>(B, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
    case 64: return qkv_attention_t<T, 64, D>(B, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
    case 128: return qkv_attention_t<T, 128, D>(B, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
    case 256: return qkv_attention_t<T, 256, D>(B, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t qkv_attention_d(int B, int S, int nh, int d, const void* x, const void* w_t,
                                  const void* bias, const int32_t* lens, int s_valid, int causal,
                                  void* ctx, hipStream_t s) {
  if (d == 64) return qkv_attention_s<T, 64>(B, S, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
  return qkv_attention_s<T, 32>(B, S, nh, x, w_t, bias, lens, s_valid, causal, ctx, s);
}

hipError_t launch_qkv_attention(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                const void* w_qkv_t, const void* b_qkv, const int32_t* lens,
                                int s_valid, void* ctx, hipStream_t s, bool causal) {
  if (!qkv_attention_fits(dt, S, nh, d) || B < 1 || nh < 1) return hipErrorInvalidValue;
  if (s_valid <= 0 || s_valid > S) s_valid = S;
  const int c = causal ? 1 : 0;
  if (dt == FTX_FP16) return qkv_attention_d<f16>(B, S, nh, d, x, w_qkv_t, b_qkv, lens, s_valid, c, ctx, s);
  return qkv_attention_d<bf16>(B, S, nh, d, x, w_qkv_t, b_qkv, lens, s_valid, c, ctx, s);
}

hipError_t launch_qkv_projection(ftx_dtype dt, int B, int S, int nh, int d, const void* x,
                                 const void* w_qkv_t, const void* b_qkv, void* q, void* k,
                                 void* vt, hipStream_t s, float* ws, size_t ws_elems) {
  return launch_head_projection(dt, B, S, nh, d, x, w_qkv_t, b_qkv, 0, 3, q, k, vt, s, ws,
                                ws_elems);
}

}  // namespace ftx
