// C ABI of the row softmax (hfa_softmax_rows in include/hfa.h): validation
// and dispatch between the register-resident and the streaming kernel.
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <cstdint>

#include "hfa.h"
#include "api_util.hpp"
#include "softmax_rows.hpp"

namespace {

using namespace hfa;
using namespace hfa::api;

// 512 threads per row; rows that fit in 32 slots of 4 values per thread (24
// without 16-byte accesses) stay in registers (x read once); wider ones keep
// their first part on chip and read the rest twice.
constexpr int kSoftmaxThreads = 512;

template <int ITEMS, bool VEC>
void launch_resident(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
  hipLaunchKernelGGL((softmax_rows_resident_kernel<kSoftmaxThreads, ITEMS, VEC>), dim3(static_cast<unsigned>(rows)),
                     dim3(kSoftmaxThreads), 0, st, x, y, cols);
}

// Wider rows: 52 slots of every thread held in registers with 16-byte accesses
// (416 KiB of the row over 512 threads; 50 with the element-wise layout, whose
// extra addresses take registers) and 18 in LDS (144 KiB); the rest of the row
// is read twice.
constexpr int kWideLdsSlots = 18;
constexpr int kWideLdsBytes = kWideLdsSlots * kSoftmaxThreads * 16;

template <bool VEC>
hfa_status launch_wide(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
  constexpr int kRegSlots = VEC ? 52 : 50;
  auto kernel = softmax_rows_wide_kernel<kSoftmaxThreads, kRegSlots, kWideLdsSlots, 6, 8, VEC>;
  static std::once_flag flag;
  static hipError_t err = hipSuccess;
  std::call_once(flag, [&] {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                              kWideLdsBytes);
  });
  if (err != hipSuccess) return HFA_ERR_LAUNCH;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(rows)), dim3(kSoftmaxThreads), kWideLdsBytes, st, x, y,
                     cols);
  return HFA_OK;
}

template <bool VEC>
hfa_status launch_softmax(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t per = (cols + kSoftmaxThreads * 4 - 1) / (kSoftmaxThreads * 4);  // slots per thread
  // register-resident up to 32 slots with 16-byte accesses, 24 with the
  // element-wise layout (whose per-element addresses take more registers)
  constexpr int kResidentMax = VEC ? 32 : 24;
  if (per > kResidentMax) return launch_wide<VEC>(x, y, rows, cols, st);
  if constexpr (VEC) {
    if (per > 24) {
      launch_resident<32, VEC>(x, y, rows, cols, st);
      return HFA_OK;
    }
  }
  if (per > 16)
    launch_resident<24, VEC>(x, y, rows, cols, st);
  else if (per <= 1)
    launch_resident<1, VEC>(x, y, rows, cols, st);
  else if (per <= 2)
    launch_resident<2, VEC>(x, y, rows, cols, st);
  else if (per <= 4)
    launch_resident<4, VEC>(x, y, rows, cols, st);
  else if (per <= 8)
    launch_resident<8, VEC>(x, y, rows, cols, st);
  else
    launch_resident<16, VEC>(x, y, rows, cols, st);
  return HFA_OK;
}

}  // namespace

extern "C" {

hfa_status hfa_softmax_rows(const float* x, float* y, int64_t rows, int64_t cols, void* stream) {
  if (!x || !y) return HFA_ERR_NULL;
  if (rows < 1 || cols < 1 || rows > INT_MAX) return HFA_ERR_SHAPE;
  if (cols > (INT64_MAX / 4) / rows) return HFA_ERR_SHAPE;
  if (misaligned(x, 4) || misaligned(y, 4)) return HFA_ERR_ALIGN;
  const size_t bytes = static_cast<size_t>(rows) * static_cast<size_t>(cols) * sizeof(float);
  if (x != y && overlaps(x, bytes, y, bytes)) return HFA_ERR_ALIAS;
  const hfa_status dev = check_device();
  if (dev != HFA_OK) return dev;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hfa_status ls = cols % 4 == 0 && !misaligned(x, 16) && !misaligned(y, 16)
                            ? launch_softmax<true>(x, y, rows, cols, st)
                            : launch_softmax<false>(x, y, rows, cols, st);
  if (ls != HFA_OK) return ls;
  return hipGetLastError() == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

}  // extern "C"
