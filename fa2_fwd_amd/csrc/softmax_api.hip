// C ABI of the row softmax (hfa_softmax_rows in include/hfa.h): validation
// and dispatch between the register-resident and the streaming kernel.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "hfa.h"
#include "api_util.hpp"
#include "softmax_rows.hpp"

namespace {

using namespace hfa;
using namespace hfa::api;

// 512 threads per row; rows that fit in 16 slots of 4 values per thread stay
// in registers, wider ones stream (x read twice).
constexpr int kSoftmaxThreads = 512;

template <int ITEMS, bool VEC>
void launch_resident(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
  hipLaunchKernelGGL((softmax_rows_resident_kernel<kSoftmaxThreads, ITEMS, VEC>), dim3(static_cast<unsigned>(rows)),
                     dim3(kSoftmaxThreads), 0, st, x, y, cols);
}

template <bool VEC>
void launch_softmax(const float* x, float* y, int64_t rows, int64_t cols, hipStream_t st) {
  const int64_t per = (cols + kSoftmaxThreads * 4 - 1) / (kSoftmaxThreads * 4);  // slots per thread
  if (per <= 1)
    launch_resident<1, VEC>(x, y, rows, cols, st);
  else if (per <= 2)
    launch_resident<2, VEC>(x, y, rows, cols, st);
  else if (per <= 4)
    launch_resident<4, VEC>(x, y, rows, cols, st);
  else if (per <= 8)
    launch_resident<8, VEC>(x, y, rows, cols, st);
  else if (per <= 16)
    launch_resident<16, VEC>(x, y, rows, cols, st);
  else
    hipLaunchKernelGGL((softmax_rows_stream_kernel<kSoftmaxThreads, 8, VEC>), dim3(static_cast<unsigned>(rows)),
                       dim3(kSoftmaxThreads), 0, st, x, y, cols);
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
  if (cols % 4 == 0 && !misaligned(x, 16) && !misaligned(y, 16))
    launch_softmax<true>(x, y, rows, cols, st);
  else
    launch_softmax<false>(x, y, rows, cols, st);
  return hipGetLastError() == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

}  // extern "C"
