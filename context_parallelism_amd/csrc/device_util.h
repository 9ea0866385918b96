// Device helpers shared by the MFMA kernels: scalar views of plan records.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace cpattn {

// Plan records are read through the constant address space so that the
// uniform loads become scalar loads (counted by lgkmcnt, not by the vmcnt
// that tracks the LDS-DMA ring).
template <typename T>
using const_ptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ inline const_ptr<T> scalar_view(const T* p) {
  return (const_ptr<T>)(p);
}
// Copy of plan record i (a struct of int32 words) through a scalar view.
template <typename T>
__device__ inline T scalar_load(const T* p, int64_t i) {
  static_assert(sizeof(T) % 4 == 0, "int32 words");
  const const_ptr<int32_t> q = (const_ptr<int32_t>)(p + i);
  int32_t w[sizeof(T) / 4];
#pragma unroll
  for (size_t k = 0; k < sizeof(T) / 4; ++k) w[k] = q[k];
  T r;
  __builtin_memcpy(&r, w, sizeof(T));
  return r;
}

}  // namespace cpattn
