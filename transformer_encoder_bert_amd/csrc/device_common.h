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

// tanh-form GELU, 0.5 u (1 + tanh(sqrt(2/pi)(u + 0.044715 u^3))), evaluated through the
// identity 0.5 (1 + tanh(y)) = 1 / (1 + exp(-2 y)) so that one exp and one divide suffice;
// the cube is written as u*u*u.  Large negative u gives exp -> inf and a result of -0.
__device__ __forceinline__ float gelu_tanh(float u) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  float y = k0 * (u + k1 * u * u * u);
  return u / (1.0f + __expf(-2.0f * y));
}

// Sum / max over groups of `width` consecutive lanes (width a power of two <= 64).
template <int width> __device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = width / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, width);
  return v;
}

}  // namespace ftx
