// Device-side types and helpers shared by the ftx HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ftx {

typedef _Float16 f16;
typedef __bf16 bf16;

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Vector of N elements of T, and the 16-byte vector of T.
template <typename T, int N> struct VecT;
template <> struct VecT<float, 1> { typedef float type; };
template <> struct VecT<float, 2> { typedef f32x2 type; };
template <> struct VecT<float, 4> { typedef f32x4 type; };
template <> struct VecT<float, 8> { typedef f32x8 type; };
template <> struct VecT<f16, 4> { typedef f16x4 type; };
template <> struct VecT<f16, 8> { typedef f16x8 type; };
template <> struct VecT<bf16, 4> { typedef bf16x4 type; };
template <> struct VecT<bf16, 8> { typedef bf16x8 type; };

template <typename T> struct Vec16 {
  static constexpr int N = 16 / sizeof(T);
  typedef typename VecT<T, N>::type type;
};

template <typename T> __device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// tanh-form GELU, 0.5 u (1 + tanh(y)) with y = sqrt(2/pi) (u + 0.044715 u^3), through the
// identity 0.5 (1 + tanh(y)) = 1 / (1 + e^(-2y)) = 1 / (1 + 2^z), z = -2 log2(e) y.  With
// log2(e) folded into the constants, z = u (c1 + c3 u^2) (the cube as plain products, no
// pow): one multiply-add, two multiplies, one add, and the hardware base-2 exponential and
// reciprocal per element.  Large negative u gives 2^z -> inf, a reciprocal of 0 and a result
// of -0; large positive u gives 2^z -> 0 and the result u.
// 2^x on the hardware exp2 alone, for softmax probabilities 2^((s - max) * scale): results
// below 2^-126 (probabilities that small against the row maximum) flush to 0, where the
// library exp2f wraps the same instruction in a range fix-up (compare, select, ldexp).
__device__ __forceinline__ float exp2_flush(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float gelu_tanh(float u) {
  constexpr float c1 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  constexpr float c3 = c1 * 0.044715f;
  const float z = u * __builtin_fmaf(c3, u * u, c1);
  return u * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// Sum of the split-K partials p[0], p[stride], ..., p[(splits - 1) * stride] (four floats
// each) in split order.  The loads go out four at a time before their additions, so a long
// split costs a quarter of the dependent memory round trips; the additions keep the order.
__device__ __forceinline__ f32x4 sum_partials4(const float* p, size_t stride, int splits) {
  f32x4 acc = *(const f32x4*)p;
  int z = 1;
  for (; z + 4 <= splits; z += 4) {
    const f32x4 v0 = *(const f32x4*)(p + z * stride);
    const f32x4 v1 = *(const f32x4*)(p + (z + 1) * stride);
    const f32x4 v2 = *(const f32x4*)(p + (z + 2) * stride);
    const f32x4 v3 = *(const f32x4*)(p + (z + 3) * stride);
    acc += v0;
    acc += v1;
    acc += v2;
    acc += v3;
  }
  for (; z < splits; ++z) acc += *(const f32x4*)(p + z * stride);
  return acc;
}

// The same sum with every load issued before the first addition (splits <= MAXS): one
// memory round trip for the whole split, the additions still in split order.
template <int MAXS>
__device__ __forceinline__ f32x4 sum_partials_all(const float* p, size_t stride, int splits) {
  f32x4 v[MAXS];
#pragma unroll
  for (int z = 0; z < MAXS; ++z)
    if (z < splits) v[z] = *(const f32x4*)(p + z * stride);
  f32x4 acc = v[0];
#pragma unroll
  for (int z = 1; z < MAXS; ++z)
    if (z < splits) acc += v[z];
  return acc;
}

// The value of the lane 32 away (lane ^ 32), by one v_permlane32_swap in registers instead
// of an LDS round trip.  With both operands x, the swap's first result holds x of lane
// l % 32 and its second x of lane l % 32 + 32, in every lane l.  Only the selected integer
// is cast back to float: casting both results to float and combining them compiled, with
// this toolchain, into code that read the first result twice.
__device__ __forceinline__ float half_swap(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (threadIdx.x & 32) ? r[0] : r[1]);
}

// 16 bytes per lane from byte offset voff + soff of buffer resource r into LDS at
// lds + 16 * lane (buffer_load_dwordx4 ... lds: the LDS address is wave-uniform, the lane
// offset implicit; soff is a wave-uniform byte offset).  An offset at or past the resource's
// byte count reads as zero and touches no memory.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, int voff, void* lds,
                                          int soff = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, soff, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding; LDS and
// scalar counters unconstrained.  The loads into LDS are only tracked by this counter.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the memory fence of __syncthreads() (which would also wait for
// every outstanding load); the empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void workgroup_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Row statistics of z from per-tile pairs (mean, centred sum of squares) over tiles of bn
// columns covering a width of h (ntn <= MAXT tiles; st a pointer or a register array):
// r = 1 / sqrt(var + eps) and s = -mean * r, so that the normalised row is r z + s (before
// gamma and beta).  Chan's merge of the groups, in tile order; the loops are unrolled to
// MAXT so that a register array is indexed by constants only.
template <int MAXT, typename S>
__device__ __forceinline__ float2 merge_row_stats(const S& st, int ntn, int bn, int h, float eps) {
  float mean = 0.f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
    if (t < ntn) mean += st[t].x * (float)min(bn, h - t * bn);
  mean /= (float)h;
  float m2 = 0.f;
#pragma unroll
  for (int t = 0; t < MAXT; ++t)
    if (t < ntn) {
      const float d = st[t].x - mean;
      m2 += st[t].y + (float)min(bn, h - t * bn) * d * d;
    }
  const float r = rsqrtf(m2 / (float)h + eps);
  return make_float2(r, -mean * r);
}

// Most per-tile statistics pairs a row of a folded LayerNorm may have (hidden 1024 in
// 64-column tiles).
constexpr int kMaxStatTiles = 16;

// Sum / max over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, width);
  return v;
}

}  // namespace ftx
