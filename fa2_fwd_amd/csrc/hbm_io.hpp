// Global-memory accesses of the HBM-bound kernels (row softmax, RMSNorm).
#pragma once

#include <hip/hip_runtime.h>

namespace hfa {

// 16-byte accesses of the HBM-bound kernels.  NT marks the access
// non-temporal (global_load/store ... nt): data touched once, which the caches
// need not keep.  Outputs are written that way; an input is read that way only
// when nothing reads it again.
template <bool NT, class V>
__device__ __forceinline__ V load16(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT, class V>
__device__ __forceinline__ void store16(V* p, V v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

}  // namespace hfa
