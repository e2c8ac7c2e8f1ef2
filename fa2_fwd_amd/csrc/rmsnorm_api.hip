// C ABI of the fused residual add + RMS normalisation (hfa_rmsnorm in
// include/hfa.h): validation and the choice of row-group size.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "hfa.h"
#include "api_util.hpp"
#include "rmsnorm.hpp"

namespace {

using namespace hfa;
using namespace hfa::api;

constexpr int64_t kRmsMaxCols = 65536;

template <typename T, int NT, int G, int ITEMS, bool VEC, bool HAS_RES>
void launch_rms(const T* x, const T* r, const T* w, T* y, T* s, int64_t rows, int64_t cols, float eps,
                hipStream_t st) {
  constexpr int64_t per_wg = NT / G;
  const int64_t grid = (rows + per_wg - 1) / per_wg;
  hipLaunchKernelGGL((rmsnorm_kernel<T, NT, G, ITEMS, VEC, HAS_RES>), dim3(static_cast<unsigned>(grid)), dim3(NT),
                     0, st, x, r, w, y, s, rows, static_cast<int>(cols), eps);
}

// Row groups of G threads with ITEMS 16-byte slots each: one wave per row up to
// 256 slots, then wider groups at 4 slots per thread, then more slots per
// thread, at most 64 values per thread (16 fp32 or 8 bf16 slots).
template <typename T, bool VEC, bool HAS_RES>
void dispatch_rms(const T* x, const T* r, const T* w, T* y, T* s, int64_t rows, int64_t cols, float eps,
                  hipStream_t st) {
  constexpr int PER = RmsElt<T>::kPerSlot;
  const int64_t slots = (cols + PER - 1) / PER;
  if (slots <= 64)
    launch_rms<T, 256, 64, 1, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 128)
    launch_rms<T, 256, 64, 2, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 256)
    launch_rms<T, 256, 64, 4, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 512)
    launch_rms<T, 256, 128, 4, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 1024)
    launch_rms<T, 256, 256, 4, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 2048)
    launch_rms<T, 512, 512, 4, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if (slots <= 4096)
    launch_rms<T, 512, 512, 8, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  else if constexpr (PER == 4) {
    if (slots <= 8192)
      launch_rms<T, 512, 512, 16, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
    else
      launch_rms<T, 1024, 1024, 16, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  } else {
    launch_rms<T, 1024, 1024, 8, VEC, HAS_RES>(x, r, w, y, s, rows, cols, eps, st);
  }
}

template <typename T>
void dispatch_rms(const void* x, const void* r, const void* w, void* y, void* s, int64_t rows, int64_t cols,
                  float eps, bool vec, hipStream_t st) {
  auto X = static_cast<const T*>(x), R = static_cast<const T*>(r), W = static_cast<const T*>(w);
  auto Y = static_cast<T*>(y), S = static_cast<T*>(s);
  if (r) {
    if (vec)
      dispatch_rms<T, true, true>(X, R, W, Y, S, rows, cols, eps, st);
    else
      dispatch_rms<T, false, true>(X, R, W, Y, S, rows, cols, eps, st);
  } else {
    if (vec)
      dispatch_rms<T, true, false>(X, R, W, Y, S, rows, cols, eps, st);
    else
      dispatch_rms<T, false, false>(X, R, W, Y, S, rows, cols, eps, st);
  }
}

// An output may be exactly an input (in place) but must not partly overlap
// one, and must not overlap the weight or the other output.
bool bad_alias(const void* out, const void* x, const void* r, size_t bytes) {
  if (out != x && overlaps(out, bytes, x, bytes)) return true;
  if (r && out != r && overlaps(out, bytes, r, bytes)) return true;
  return false;
}

}  // namespace

extern "C" {

hfa_status hfa_rmsnorm(const void* x, const void* residual, const void* weight, void* y, void* residual_out,
                       int64_t rows, int64_t cols, float eps, hfa_dtype dtype, void* stream) {
  if (!x || !weight || !y || (residual && !residual_out)) return HFA_ERR_NULL;
  if (dtype != HFA_F32 && dtype != HFA_BF16) return HFA_ERR_UNSUPPORTED;
  if (rows < 1 || cols < 1 || cols > kRmsMaxCols || rows > INT_MAX) return HFA_ERR_SHAPE;
  if (!std::isfinite(eps) || !(eps > 0.0f)) return HFA_ERR_EPS;
  const size_t elt = dtype == HFA_F32 ? 4 : 2;
  void* s = residual ? residual_out : nullptr;
  const void* ptrs[5] = {x, residual, weight, y, s};
  for (const void* p : ptrs)
    if (p && misaligned(p, elt)) return HFA_ERR_ALIGN;
  const size_t bytes = static_cast<size_t>(rows) * static_cast<size_t>(cols) * elt;
  const size_t wbytes = static_cast<size_t>(cols) * elt;
  if (bad_alias(y, x, residual, bytes) || overlaps(y, bytes, weight, wbytes)) return HFA_ERR_ALIAS;
  if (s && (bad_alias(s, x, residual, bytes) || overlaps(s, bytes, weight, wbytes) || overlaps(s, bytes, y, bytes)))
    return HFA_ERR_ALIAS;
  const hfa_status dev = check_device();
  if (dev != HFA_OK) return dev;
  const int per = dtype == HFA_F32 ? 4 : 8;
  bool vec = cols % per == 0;
  for (const void* p : ptrs)
    if (p && misaligned(p, 16)) vec = false;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == HFA_F32)
    dispatch_rms<float>(x, residual, weight, y, s, rows, cols, eps, vec, st);
  else
    dispatch_rms<__bf16>(x, residual, weight, y, s, rows, cols, eps, vec, st);
  return hipGetLastError() == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

}  // extern "C"
