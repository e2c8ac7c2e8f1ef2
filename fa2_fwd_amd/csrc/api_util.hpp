// Host-side helpers shared by the C-ABI entry points of libhfa.so: pointer
// checks and the gfx950 device check.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "hfa.h"

namespace hfa {
namespace api {

// Whether the byte ranges [a, a + na) and [b, b + nb) intersect.
inline bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Whether p is not a multiple of the power of two `align`.
inline bool misaligned(const void* p, uintptr_t align) {
  return (reinterpret_cast<uintptr_t>(p) & (align - 1)) != 0;
}

// Whether the current device is a gfx950; cached per device ordinal (one
// table for the whole library, since the function is inline).
inline hfa_status check_device() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return HFA_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return HFA_ERR_NO_DEVICE;
  int st = arch_state[dev].load(std::memory_order_acquire);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return HFA_ERR_NO_DEVICE;
    }
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    arch_state[dev].store(st, std::memory_order_release);
  }
  return st == 1 ? HFA_OK : HFA_ERR_NO_DEVICE;
}

}  // namespace api
}  // namespace hfa
