// Row softmax of an fp32 matrix for gfx950: y[r, :] = softmax(x[r, :]).
//
// The stable row softmax of the book chapter "Triton and kernel fusion"
// (section "Fusion": subtract the row max, exponentiate, sum, divide; one read
// of x and one write of y instead of about eight passes), extended to rows
// wider than what one block holds by the route its stretch exercise names: a
// running max and a running sum (the online normalisation identity of
// neuralmasteryai "Hardware Acceleration & Custom Kernels", section 2, step 2).
//
// One workgroup per row.  Every thread folds its elements into a pair (m, l)
// = (max, sum of exp(x - m)); pairs are merged by the same identity,
//     (m, l) + (m', l') = (M, l e^(m - M) + l' e^(m' - M)),  M = max(m, m'),
// first across the 64 lanes of a wave, then across the waves through LDS.
//
//  * Resident path (cols <= NT * 4 * ITEMS): the thread's elements stay in
//    registers between the reduction and the output: x is read once, with
//    non-temporal loads.
//  * Wide path: the first part of the row stays on chip between the passes
//    (registers, then LDS: about half of the on-chip space of a CU), the rest
//    updates the running pair chunk by chunk as it streams through and is read
//    a second time, last chunk first, to write y.
//
// y is written with non-temporal stores.  Exponentials are exp2 of
// (x - M) * log2(e), the difference taken first so that large |x| loses no
// accuracy.  Element i of a row is read and written by
// the same thread, and every read precedes the reduction barrier, so y may be
// x itself.
#pragma once

#include "common.hpp"
#include "hbm_io.hpp"

namespace hfa {

constexpr float kLog2eF = 1.44269504088896340736f;

struct SoftmaxPair {
  float m, l;  // running max and running sum of exp(x - m)
};

// The merge identity.  An empty pair (-inf, 0) is neutral; the weights of the
// two sides are formed only for a finite joint max.
__device__ __forceinline__ SoftmaxPair merge_pairs(SoftmaxPair a, SoftmaxPair b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return {M, 0.0f};
  const float wa = a.m == -INFINITY ? 0.0f : exp2_hw((a.m - M) * kLog2eF);
  const float wb = b.m == -INFINITY ? 0.0f : exp2_hw((b.m - M) * kLog2eF);
  return {M, a.l * wa + b.l * wb};
}

// Fold n values (-inf marks an absent one) into a running pair.
template <int NV>
__device__ __forceinline__ SoftmaxPair fold_values(SoftmaxPair p, const float (&v)[NV]) {
  float cm = v[0];
#pragma unroll
  for (int i = 1; i < NV; ++i) cm = fmaxf(cm, v[i]);
  const float M = fmaxf(p.m, cm);
  if (M == -INFINITY) return p;
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) s += v[i] == -INFINITY ? 0.0f : exp2_hw((v[i] - M) * kLog2eF);
  const float w = p.m == -INFINITY ? 0.0f : exp2_hw((p.m - M) * kLog2eF);
  return {M, p.l * w + s};
}

// Merge the pairs of all threads of the workgroup; every thread gets the total.
template <int NT>
__device__ __forceinline__ SoftmaxPair merge_workgroup(SoftmaxPair p, SoftmaxPair* lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const SoftmaxPair o = {__shfl_xor(p.m, off), __shfl_xor(p.l, off)};
    p = merge_pairs(p, o);
  }
  const int wave = thread_id() >> 6;
  if ((thread_id() & 63) == 0) lds[wave] = p;
  __syncthreads();
  SoftmaxPair t = lds[0];
#pragma unroll
  for (int w = 1; w < NT / 64; ++w) t = merge_pairs(t, lds[w]);
  return t;
}

// Element e (0..3) of slot s of thread tid: 16-byte vectors when VEC (row
// width a multiple of 4 and 16-byte aligned rows), else a coalesced scalar
// layout.
template <int NT, bool VEC>
__device__ __forceinline__ int64_t slot_index(int64_t base, int s, int tid, int e) {
  return VEC ? base + (static_cast<int64_t>(s) * NT + tid) * 4 + e : base + (static_cast<int64_t>(s) * 4 + e) * NT + tid;
}

// NT_LOAD: the row is read only once (resident path), so the read is
// non-temporal; the streaming path reads x twice and keeps it cacheable.
template <int NT, bool VEC, int SLOTS, bool NT_LOAD>
__device__ __forceinline__ void load_slots(const float* xr, int64_t base, int64_t cols, int tid, float (&v)[SLOTS * 4]) {
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    if (VEC) {
      const int64_t i0 = slot_index<NT, true>(base, s, tid, 0);
      if (i0 < cols) {
        const f32x4 q = load16<NT_LOAD>(reinterpret_cast<const f32x4*>(xr + i0));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * s + e] = q[e];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * s + e] = -INFINITY;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = slot_index<NT, false>(base, s, tid, e);
        v[4 * s + e] = i < cols ? xr[i] : -INFINITY;
      }
    }
  }
}

template <int NT, bool VEC, int SLOTS>
__device__ __forceinline__ void store_slots(float* yr, int64_t base, int64_t cols, int tid, const float (&v)[SLOTS * 4],
                                            float M, float inv) {
#pragma unroll
  for (int s = 0; s < SLOTS; ++s) {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = exp2_hw((v[4 * s + e] - M) * kLog2eF) * inv;
    if (VEC) {
      const int64_t i0 = slot_index<NT, true>(base, s, tid, 0);
      if (i0 < cols) store16<true>(reinterpret_cast<f32x4*>(yr + i0), f32x4{o[0], o[1], o[2], o[3]});
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = slot_index<NT, false>(base, s, tid, e);
        if (i < cols) yr[i] = o[e];
      }
    }
  }
}

// Resident path: the row's NT * 4 * ITEMS slots stay in registers.
template <int NT, int ITEMS, bool VEC>
__global__ __launch_bounds__(NT) void softmax_rows_resident_kernel(const float* x, float* y, int64_t cols) {
  __shared__ SoftmaxPair lds[NT / 64];
  const int tid = thread_id();
  const int64_t row = group_id();
  const float* xr = x + row * cols;
  float* yr = y + row * cols;
  float v[ITEMS * 4];
  load_slots<NT, VEC, ITEMS, true>(xr, 0, cols, tid, v);
  const SoftmaxPair p = merge_workgroup<NT>(fold_values(SoftmaxPair{-INFINITY, 0.0f}, v), lds);
  store_slots<NT, VEC, ITEMS>(yr, 0, cols, tid, v, p.m, 1.0f / p.l);
}

// Slots of the wide kernel, addressed as a wave-uniform base (the row, plus
// the slot's offset) and one 32-bit lane offset shared by every slot, so that
// no per-slot address is held in vector registers.  VEC: slot s of thread t is
// the 16 bytes at element (s NT + t) 4 of the row; else element e of it is
// element (4 s + e) NT + t.  lane4 = 4 t.  Elements past the row read as -inf.
template <int NT, bool VEC, int N, bool NT_LOAD>
__device__ __forceinline__ void wide_load(const float* xr, int64_t s0, int64_t cols, uint32_t lane4,
                                          float (&v)[N * 4]) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int64_t slot0 = (s0 + u) * NT * 4;  // first element of the slot
    if (VEC) {
      const float* base = xr + slot0;
      f32x4 q = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (static_cast<int64_t>(lane4) < cols - slot0)
        q = load16<NT_LOAD>(reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(base) + 4 * lane4));
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * u + e] = q[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* base = xr + slot0 + e * NT;
        v[4 * u + e] = static_cast<int64_t>(lane4 / 4) < cols - slot0 - e * NT
                           ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(base) + lane4)
                           : -INFINITY;
      }
    }
  }
}

template <int NT, bool VEC, int N>
__device__ __forceinline__ void wide_store(float* yr, int64_t s0, int64_t cols, uint32_t lane4, const float (&v)[N * 4],
                                           float M, float inv) {
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int64_t slot0 = (s0 + u) * NT * 4;
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = exp2_hw((v[4 * u + e] - M) * kLog2eF) * inv;
    if (VEC) {
      if (static_cast<int64_t>(lane4) < cols - slot0)
        store16<true>(reinterpret_cast<f32x4*>(reinterpret_cast<char*>(yr + slot0) + 4 * lane4),
                      f32x4{o[0], o[1], o[2], o[3]});
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (static_cast<int64_t>(lane4 / 4) < cols - slot0 - e * NT)
          *reinterpret_cast<float*>(reinterpret_cast<char*>(yr + slot0 + e * NT) + lane4) = o[e];
    }
  }
}

// Wide rows: the first RS slots of every thread stay in registers and the next
// LS slots in LDS (dynamic, LS * NT * 16 bytes) between the two passes; only
// the slots after them are read a second time, last first (the likeliest to be
// in the caches).  Loads in flight per thread: all RS at once, then UL per
// step over the LDS slots and US per step over the rest.
template <int NT, int RS, int LS, int UL, int US, bool VEC>
__global__ __launch_bounds__(NT) void softmax_rows_wide_kernel(const float* x, float* y, int64_t cols) {
  static_assert(LS % UL == 0, "the LDS slots are read in whole steps");
  __shared__ SoftmaxPair lds[NT / 64];
  extern __shared__ f32x4 held[];  // [LS][NT]
  const int tid = thread_id();
  const int64_t row = uniform_sgpr(group_id());
  const float* xr = x + row * cols;
  float* yr = y + row * cols;
  // 4 tid: the lane's first element within a slot (VEC; its byte offset is
  // 16 tid), or the byte offset of its element within each quarter (scalar)
  const uint32_t lane4 = 4u * static_cast<uint32_t>(tid);
  constexpr int64_t SLOT = static_cast<int64_t>(NT) * 4;
  const int64_t nslots = (cols + SLOT - 1) / SLOT;
  float r[RS * 4];
  wide_load<NT, VEC, RS, true>(xr, 0, cols, lane4, r);
  SoftmaxPair p = fold_values(SoftmaxPair{-INFINITY, 0.0f}, r);
  const int lsteps = static_cast<int>(nslots > RS ? min<int64_t>((nslots - RS + UL - 1) / UL, LS / UL) : 0);
  for (int st = 0; st < lsteps; ++st) {
    float v[UL * 4];
    wide_load<NT, VEC, UL, true>(xr, RS + st * UL, cols, lane4, v);
    p = fold_values(p, v);
#pragma unroll
    for (int u = 0; u < UL; ++u)
      held[(st * UL + u) * NT + tid] = f32x4{v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]};
  }
  constexpr int64_t KEPT = RS + LS;  // slots held on chip
  for (int64_t s = KEPT; s < nslots; s += US) {
    float v[US * 4];
    wide_load<NT, VEC, US, false>(xr, s, cols, lane4, v);
    p = fold_values(p, v);
  }
  p = merge_workgroup<NT>(p, lds);
  const float inv = 1.0f / p.l;
  if (nslots > KEPT) {
    for (int64_t s = KEPT + (nslots - 1 - KEPT) / US * US; s >= KEPT; s -= US) {
      float v[US * 4];
      wide_load<NT, VEC, US, false>(xr, s, cols, lane4, v);
      wide_store<NT, VEC, US>(yr, s, cols, lane4, v, p.m, inv);
    }
  }
  for (int st = 0; st < lsteps; ++st) {
    float v[UL * 4];
#pragma unroll
    for (int u = 0; u < UL; ++u) {
      const f32x4 h = held[(st * UL + u) * NT + tid];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * u + e] = h[e];
    }
    wide_store<NT, VEC, UL>(yr, RS + st * UL, cols, lane4, v, p.m, inv);
  }
  wide_store<NT, VEC, RS>(yr, 0, cols, lane4, r, p.m, inv);
}

}  // namespace hfa
