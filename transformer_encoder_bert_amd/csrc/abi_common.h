// Helpers shared by the C entry points of the encoder and the decoder: the thread-local
// message behind ftx_last_error(), status conversion of HIP errors, and the argument
// checks (dtype, alignment, overlap, device pointers, shapes).  Host code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <initializer_list>
#include <string>

#include "ftx.h"

namespace ftx {

// The calling thread's message of the last failing call (empty after a success).
std::string& last_error_slot();

inline ftx_status fail(ftx_status s, const std::string& msg) {
  last_error_slot() = msg;
  return s;
}

inline ftx_status hip_fail(hipError_t e, const char* what) {
  if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation)
    return fail(FTX_ERR_OUT_OF_MEMORY, std::string(what) + ": " + hipGetErrorString(e));
  return fail(FTX_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
}

#define FTX_HIP(call)                                   \
  do {                                                  \
    hipError_t e_ = (call);                             \
    if (e_ != hipSuccess) return ::ftx::hip_fail(e_, #call); \
  } while (0)

inline size_t dtype_size(ftx_dtype dt) { return dt == FTX_FP32 ? 4 : 2; }
inline bool dtype_ok(int dt) { return dt == FTX_FP32 || dt == FTX_FP16 || dt == FTX_BF16; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// True if `p` points into device memory (or managed memory) of the HIP runtime.  Kernels
// given a host pointer would fault, so every entry point checks its tensor pointers.
inline bool is_device_ptr(const void* p) {
  if (!p) return false;
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged;
}

inline bool all_device(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && !is_device_ptr(p)) return false;
  return true;
}

// Shape checks shared by the handles and the step entry points: size_per_head 32 or 64,
// length at most FTX_MAX_SEQ_LEN (a multiple of 32 unless any_len), hidden at most
// FTX_MAX_HIDDEN, and 32-bit element indices for the largest tensor [B*S][4H].
ftx_status check_shape(int B, int S, int nh, int d, bool any_len = false);

}  // namespace ftx
