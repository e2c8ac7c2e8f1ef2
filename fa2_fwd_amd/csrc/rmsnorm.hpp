// Fused residual add + RMS normalisation for gfx950:
//     s = x + residual           (fp32 add; s = x without a residual)
//     y = s / sqrt(mean_j s_j^2 + eps) * w
// The normalisation is the TritonForge "Fused RMSNorm" card's formula; the
// fused residual form, with s returned as a second output, is the book chapter
// "Triton and kernel fusion", section "Fused residual add + RMSNorm" (two reads
// and two writes per element instead of five passes).  Elements are fp32 or
// bf16; all arithmetic is fp32, and bf16 outputs are rounded once (nearest
// even) from the fp32 values.
//
// Each row is owned by a group of G threads (one wave, or up to 16 waves of a
// workgroup); a workgroup of NT threads holds NT / G rows.  Every thread keeps
// ITEMS slots of 16 bytes of the row in registers, so x and the residual are
// read once: the sum of squares is reduced over the group (wave shuffles, then
// LDS across the group's waves) and the same registers are normalised and
// written (16-byte accesses to x, the residual and the outputs are
// non-temporal: each is touched once; the weight row, read by every row,
// stays cacheable).  Element i of a row is read and written by one thread, and all its
// reads precede its writes, so y and s may be written over x or the residual.
#pragma once

#include "common.hpp"
#include "hbm_io.hpp"

namespace hfa {

template <typename T>
struct RmsElt;

template <>
struct RmsElt<float> {
  static constexpr int kPerSlot = 4;  // elements per 16-byte slot
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
  template <bool NT = false>
  __device__ static void load_slot(const float* p, float (&v)[4]) {
    const f32x4 q = load16<NT>(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = q[e];
  }
  __device__ static void store_slot(float* p, const float (&v)[4]) {
    store16<true>(reinterpret_cast<f32x4*>(p), f32x4{v[0], v[1], v[2], v[3]});
  }
};

template <>
struct RmsElt<__bf16> {
  static constexpr int kPerSlot = 8;
  __device__ static float load(const __bf16* p) { return static_cast<float>(*p); }
  __device__ static void store(__bf16* p, float v) { *p = static_cast<__bf16>(v); }
  template <bool NT = false>
  __device__ static void load_slot(const __bf16* p, float (&v)[8]) {
    const bf16x8 q = load16<NT>(reinterpret_cast<const bf16x8*>(p));
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(q[e]);
  }
  __device__ static void store_slot(__bf16* p, const float (&v)[8]) {
    bf16x8 q;
#pragma unroll
    for (int e = 0; e < 8; ++e) q[e] = static_cast<__bf16>(v[e]);
    store16<true>(reinterpret_cast<bf16x8*>(p), q);
  }
};

// Column of element e of slot s for lane t of a G-thread row group: whole
// 16-byte slots per lane when VEC, else a coalesced element-strided layout.
// Rows hold at most 65536 elements, so columns fit an int.
template <int G, int PER, bool VEC>
__device__ __forceinline__ int rms_col(int s, int t, int e) {
  return VEC ? (s * G + t) * PER + e : (s * PER + e) * G + t;
}

template <int G>
__device__ __forceinline__ float group_sum(float v, float* lds) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if constexpr (G > 64) {
    const int wave = thread_id() >> 6;
    if ((thread_id() & 63) == 0) lds[wave] = v;
    __syncthreads();
    const int first = (wave / (G / 64)) * (G / 64);
    v = lds[first];
#pragma unroll
    for (int w = 1; w < G / 64; ++w) v += lds[first + w];
  }
  return v;
}

template <typename T, int NT, int G, int ITEMS, bool VEC, bool HAS_RES>
__global__ __launch_bounds__(NT) void rmsnorm_kernel(const T* x, const T* res, const T* w, T* y, T* s_out,
                                                     int64_t rows, int cols, float eps) {
  static_assert(NT % G == 0 && G % 64 == 0, "row groups are whole waves");
  using E = RmsElt<T>;
  constexpr int PER = E::kPerSlot;
  __shared__ float lds[NT / 64];
  const int t = thread_id() % G;
  const int64_t row = static_cast<int64_t>(group_id()) * (NT / G) + thread_id() / G;
  const bool live = row < rows;
  const int64_t base = live ? row * cols : 0;
  const T* xr = x + base;
  const T* rr = HAS_RES ? res + base : nullptr;
  T* yr = y + base;
  T* sr = HAS_RES ? s_out + base : nullptr;

  float v[ITEMS][PER];
#pragma unroll
  for (int s = 0; s < ITEMS; ++s) {
    if (VEC) {
      const int c0 = rms_col<G, PER, true>(s, t, 0);
      if (live && c0 < cols) {
        E::template load_slot<true>(xr + c0, v[s]);
        if (HAS_RES) {
          float r[PER];
          E::template load_slot<true>(rr + c0, r);
#pragma unroll
          for (int e = 0; e < PER; ++e) v[s][e] += r[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) v[s][e] = 0.0f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int c = rms_col<G, PER, false>(s, t, e);
        float a = 0.0f;
        if (live && c < cols) {
          a = E::load(xr + c);
          if (HAS_RES) a += E::load(rr + c);
        }
        v[s][e] = a;
      }
    }
  }
  // The sum goes out as soon as it exists; its registers stay for the output.
  if (HAS_RES && live) {
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
      if (VEC) {
        const int c0 = rms_col<G, PER, true>(s, t, 0);
        if (c0 < cols) E::store_slot(sr + c0, v[s]);
      } else {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int c = rms_col<G, PER, false>(s, t, e);
          if (c < cols) E::store(sr + c, v[s][e]);
        }
      }
    }
  }
  float sq = 0.0f;
#pragma unroll
  for (int s = 0; s < ITEMS; ++s)
#pragma unroll
    for (int e = 0; e < PER; ++e) sq += v[s][e] * v[s][e];
  sq = group_sum<G>(sq, lds);
  const float inv = 1.0f / sqrtf(sq / static_cast<float>(cols) + eps);
  if (!live) return;
#pragma unroll
  for (int s = 0; s < ITEMS; ++s) {
    if (VEC) {
      const int c0 = rms_col<G, PER, true>(s, t, 0);
      if (c0 < cols) {
        float wv[PER], o[PER];
        E::load_slot(w + c0, wv);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] = v[s][e] * inv * wv[e];
        E::store_slot(yr + c0, o);
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int c = rms_col<G, PER, false>(s, t, e);
        if (c < cols) E::store(yr + c, v[s][e] * inv * E::load(w + c));
      }
    }
  }
}

}  // namespace hfa
