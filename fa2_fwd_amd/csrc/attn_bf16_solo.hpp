// bf16 attention forward for grids too small to fill the GPU with the
// 256-row ping-pong workgroups of attn_bf16.hpp (neuralmasteryai "Hardware
// Acceleration & Custom Kernels", section 2, steps 1-2; the same online
// normalisation).  A workgroup is 4 waves, one per SIMD, of 32 query rows
// each (128 rows): twice the workgroups of the 256-row tiling for a given
// shape, and each wave's chain per key tile is its own matrix-core and
// vector work only, instead of the two phases of a ping-pong pair.
//
// Everything per wave is the 256-row kernel's: the MFMA mapping (S^T = K Q^T
// with the key permutation that leaves P in the B-operand layout of
// O^T = V^T P^T), the LDS swizzles, the log2-domain lazy running max and the
// epilogue.  What differs is the streaming: every wave requests its quarter
// of both the K and the V tile (global_load_lds_dwordx4, HBM straight to
// LDS), AHEAD = 2 tiles ahead, and one barrier per step separates the steps.
// Step j computes the scores of tile j, then the output products of tile
// j - 1 (which keep the matrix core busy during the softmax of tile j, the
// order of the 256-row kernel's MFMA phase), then that softmax.  So K_j is
// read in step j and V_j in step j + 1: K has a ring of 3 tiles, V one of 4.
// After the barrier of step j, tile j is complete in LDS (each wave waited
// for its own requests first) and no wave still reads K_{j-1} or V_{j-2},
// whose slots then take tile j + 2.
#pragma once

#include "attn_bf16.hpp"

namespace hfa {

template <int D_, int KT_ = 64>
struct Bf16SoloTile {
  static constexpr int D = D_;        // head dim (64 or 128)
  static constexpr int KT = KT_;      // keys per K/V tile
  static constexpr int NW = 4;        // waves per workgroup, one per SIMD
  static constexpr int WQ = 32;       // queries per wave
  static constexpr int BR = WQ * NW;  // queries per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int ROWB = D * 2;  // bytes per K or V row in LDS (XOR-swizzled, unpadded)
  static constexpr int TILEB = KT * ROWB;
  static constexpr int CH = D / 8;   // 16-byte chunks per row
  static constexpr int NBUF = 3;     // K ring depth (tiles)
  static constexpr int NBUF_V = 4;   // V ring depth: V_j is read one step after K_j
  static constexpr int AHEAD = NBUF - 1;
  static constexpr int LD = TILEB / (NW * 64 * 16);  // 16-byte requests per lane per tile and tensor
  static constexpr int LDS_BYTES = (NBUF + NBUF_V) * TILEB;  // K ring, then V ring
  static_assert(LD >= 1 && TILEB % (NW * 64 * 16) == 0, "a tile must split into whole load instructions");
  static_assert(CH == 8 || CH == 16, "swizzles are defined for d = 64 and d = 128");
  static_assert(KT % 32 == 0, "whole 32-key MFMA blocks");
  static_assert(AHEAD == 2, "the wait below counts one newer tile");
};

// Compiled for two waves per SIMD (at most 256 registers a wave) although a
// workgroup runs one: with the whole register file the compiler keeps the
// accumulators in accumulation registers and moves them for every vector use.
template <class T>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(2))) void attn_fwd_bf16_solo_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int total_wg, float c2, int q_mode) {
  constexpr int D = T::D, KT = T::KT, ROWB = T::ROWB, TILEB = T::TILEB, NBUF = T::NBUF;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const kbuf = smem;                 // K ring
  char* const vbuf = smem + NBUF * TILEB;  // V ring

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = uniform_sgpr(tid >> 6);
  const int i32 = lane & 31, hh = lane >> 5;

  // Workgroup-uniform indices in scalar registers, so that the request
  // addresses below are formed with scalar arithmetic: a vector write of a
  // scalar operand would need wait states before the inline-assembly load
  // reads it, which the compiler does not insert.
  const int tile = xcd_remap(group_id(), total_wg);
  const int bh = uniform_sgpr(tile / n_qt);
  const int qt = uniform_sgpr(tile - bh * n_qt);
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;
  __bf16* Oh = O + head;
  const int qrow0 = qt * T::BR + wave * T::WQ;
  const int ntiles = (N + KT - 1) / KT;

  // ---- K/V requests.  One load instruction writes 1 KiB of LDS in lane
  // order; wave w fills chunks (w LD + u) 64 + lane of the tile, and the XOR
  // swizzle is realised by choosing each lane's source chunk.
  int koff[T::LD], voff[T::LD];
#pragma unroll
  for (int u = 0; u < T::LD; ++u) {
    const int pos = (wave * T::LD + u) * 64 + lane;
    const int row = pos / T::CH, phys = pos % T::CH;
    koff[u] = (row * D + (phys ^ k_swz<T::CH>(row)) * 8) * 2;
    voff[u] = (row * D + (phys ^ v_swz<T::CH>(row)) * 8) * 2;
  }
  // This wave's LDS destination within a tile buffer, as a scalar LDS address.
  const uint32_t wave_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)smem)) +
                            static_cast<uint32_t>(wave * T::LD * 1024);
  auto issue_tile = [&](int t) __attribute__((always_inline)) {
    if (t >= ntiles) return;
    const int slot = t % NBUF;
    const char* ksrc = reinterpret_cast<const char*>(Kh + static_cast<size_t>(t) * KT * D);
    const char* vsrc = reinterpret_cast<const char*>(Vh + static_cast<size_t>(t) * KT * D);
    const uint32_t kdst = wave_lds + static_cast<uint32_t>(slot * TILEB);
    const uint32_t vdst = wave_lds + static_cast<uint32_t>((NBUF + t % T::NBUF_V) * TILEB);
    if ((t + 1) * KT <= N) {
#pragma unroll
      for (int u = 0; u < T::LD; ++u) dma16_to(ksrc, koff[u], kdst + u * 1024);
#pragma unroll
      for (int u = 0; u < T::LD; ++u) dma16_to(vsrc, voff[u], vdst + u * 1024);
    } else {  // ragged last tile: rows past the end re-read the last row
      const int last = N - 1 - t * KT;
#pragma unroll
      for (int u = 0; u < T::LD; ++u) {
        const int row = ((wave * T::LD + u) * 64 + lane) / T::CH;
        const int back = row > last ? (row - last) * D * 2 : 0;
        dma16_to(ksrc, koff[u] - back, kdst + u * 1024);
      }
#pragma unroll
      for (int u = 0; u < T::LD; ++u) {
        const int row = ((wave * T::LD + u) * 64 + lane) / T::CH;
        const int back = row > last ? (row - last) * D * 2 : 0;
        dma16_to(vsrc, voff[u] - back, vdst + u * 1024);
      }
    }
  };

  // ---- Q fragments (B operand of S^T): Q[row = i32][d = 16t + 8hh .. +7],
  // loaded unconditionally (rows past the end read row N - 1 and are zeroed);
  // q_mode folds the sign of the scale into Q.
  u32x4 qf[D / 16];
  {
    const int row = qrow0 + i32;
    const __bf16* qrow = Qh + static_cast<size_t>(min(row, N - 1)) * D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = *reinterpret_cast<const u32x4*>(qrow + 16 * t);
  }
  // The first tiles are requested right behind the Q loads.
#pragma unroll
  for (int t = 0; t < T::AHEAD; ++t) issue_tile(t);
  {
    const bool zero = qrow0 + i32 >= N || q_mode == 0;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      u32x4 x = qf[t];
      if (q_mode < 0) x ^= 0x80008000u;
      if (zero) x = u32x4{0u, 0u, 0u, 0u};
      qf[t] = x;
    }
  }

  // ---- per-lane LDS geometry, as in the 256-row kernel
  const int a8 = i32 >> 3, e4 = (i32 >> 2) & 1, b4 = i32 & 3;
  const int krow = 16 * (a8 >> 1) + 8 * e4 + 4 * (a8 & 1) + b4;
  const int kswz = k_swz<T::CH>(krow);
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;
  const int vrow = 8 * hh + (l16 >> 2);
  const int vswz = v_swz<T::CH>(vrow);
  const int vch = 2 * g16 + ((l16 & 3) >> 1);
  const int vin = (l16 & 1) * 8;
  int vlane[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) vlane[n] = vrow * ROWB + (((4 * n + vch) ^ vswz) << 4) + vin;

  f32x16 acc[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[n][r] = 0.0f;
  float m2 = -INFINITY, l_run = 0.0f;  // running max (log2 units) and denominator
  bf16x8 pf[KT / 16];                  // P of the last softmax, consumed one step later

  // ---- O^T += V_t^T P_t^T: key chunk c of 16 keys, column block n of 32
  auto output_products = [&](int t) __attribute__((always_inline)) {
    const char* vt = vbuf + (t % T::NBUF_V) * TILEB;
#pragma unroll
    for (int c = 0; c < KT / 16; ++c)
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        const int off = vlane[n] + 16 * c * ROWB;
        const s16x4 lo = lds_read_tr16(vt, off);
        const s16x4 hi = lds_read_tr16(vt, off + 4 * ROWB);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], acc[n], 0, 0, 0);
      }
  };

  // One key tile.  first: tile 0 (the running max starts at its row max);
  // last: the final tile (nothing requested after it; keys past N masked).
  auto step = [&](int j, auto first_tag, auto last_tag) __attribute__((always_inline)) {
    constexpr bool first = decltype(first_tag)::value;
    constexpr bool last = decltype(last_tag)::value;
    // This wave's requests for tile j are complete once at most the next
    // tile's (2 LD) are in flight; after the barrier every wave's are, and no
    // wave reads tile j - 1 any more.
    if constexpr (last)
      vmcnt_wait<0>();
    else
      vmcnt_wait<2 * T::LD>();
    lds_barrier();
    issue_tile(j + T::AHEAD);  // K into the slot of K_{j-1}, V into that of V_{j-2}
    const char* kt = kbuf + (j % NBUF) * TILEB;

    // ---- S^T = K_j Q^T: lane (i32, hh) register r of s[kb] holds key
    // 32 kb + 16 (r / 8) + 8 hh + r % 8 of the tile for query i32.
    f32x16 s[KT / 32];
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.0f;
#pragma unroll
    for (int t = 0; t < D / 16; ++t)
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb) {
        const u32x4 a = lds_load16(kt, (kb * 32 + krow) * ROWB + (((2 * t + hh) ^ kswz) << 4));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                        __builtin_bit_cast(bf16x8, qf[t]), s[kb], 0, 0, 0);
      }

    // ---- keys past the end get score -inf (weight 0)
    const int key0 = j * KT;
    if (last && key0 + KT > N) {
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7) >= N) s[kb][r] = -INFINITY;
    }

    // ---- the previous tile's output products: independent of this tile's
    // softmax, they keep the matrix core busy while it runs (the order of the
    // 256-row kernel's MFMA phase: scores of tile j, then P_{j-1} V_{j-1})
    if constexpr (!first) output_products(j - 1);

    // ---- online softmax (log2 domain, lazy running max: see attn_bf16.hpp)
    constexpr int NS = KT / 2;
    auto xv = [&](int i) { return s[i / 16][i % 16]; };
    auto xset = [&](int i, float v) { s[i / 16][i % 16] = v; };
    auto row_max = [&]() {
      float part[NS / 4];
#pragma unroll
      for (int u = 0; u < NS / 4; ++u)
        part[u] = fmaxf(fmaxf(xv(4 * u), xv(4 * u + 1)), fmaxf(xv(4 * u + 2), xv(4 * u + 3)));
#pragma unroll
      for (int w = NS / 8; w >= 1; w /= 2)
#pragma unroll
        for (int u = 0; u < w; ++u) part[u] = fmaxf(part[u], part[u + w]);
      return max_xor32(part[0]);
    };
    auto weights = [&]() {
      float pv[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) pv[i] = exp2_hw(xv(i));
#pragma unroll
      for (int c = 0; c < KT / 16; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[c][e] = static_cast<__bf16>(pv[8 * c + e]);
      float part[NS / 4];
#pragma unroll
      for (int u = 0; u < NS / 4; ++u) part[u] = (pv[4 * u] + pv[4 * u + 1]) + (pv[4 * u + 2] + pv[4 * u + 3]);
#pragma unroll
      for (int w = NS / 8; w >= 1; w /= 2)
#pragma unroll
        for (int u = 0; u < w; ++u) part[u] += part[u + w];
      return part[0];
    };
    float tsum;
    if constexpr (first) {
      // m2 is -inf before the first tile: start it at this tile's row max
      // (finite, key 0 is in the tile), so every x <= 0.
#pragma unroll
      for (int i = 0; i < NS; ++i) xset(i, xv(i) * c2);
      m2 = row_max();
#pragma unroll
      for (int i = 0; i < NS; ++i) xset(i, xv(i) - m2);
      tsum = weights();
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) xset(i, fmaf(xv(i), c2, -m2));
      tsum = weights();
      if (__any(!(tsum <= kSumLimit))) {
        const float mx = row_max();  // growth of the row max, log2 units
        const bool grow = mx > kRescaleLog2;
        const float m_new = grow ? m2 + mx : m2;
        const float d = m_new - m2;
        const float alpha = exp2_hw(-d);
        l_run *= alpha;
#pragma unroll
        for (int n = 0; n < D / 32; ++n) acc[n] *= alpha;
        m2 = m_new;
#pragma unroll
        for (int i = 0; i < NS; ++i) xset(i, xv(i) - d);
        tsum = weights();
      }
    }
    l_run += tsum;
  };
  if (ntiles == 1) {
    step(0, std::true_type{}, std::true_type{});
  } else {
    step(0, std::true_type{}, std::false_type{});
    for (int j = 1; j + 1 < ntiles; ++j) step(j, std::false_type{}, std::false_type{});
    step(ntiles - 1, std::false_type{}, std::true_type{});
  }
  output_products(ntiles - 1);  // tile ntiles - 1 is complete since the last step's wait

  // ---- epilogue: normalise, round to bf16, one write of O and of LSE
  const float l_tot = add_xor32(l_run);
  const float inv = 1.0f / l_tot;
  const int row = qrow0 + i32;
  if (row < N) {
    __bf16* orow = Oh + static_cast<size_t>(row) * D;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        bf16x4 o4;
#pragma unroll
        for (int b = 0; b < 4; ++b) o4[b] = static_cast<__bf16>(acc[n][4 * a + b] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * n + 8 * a + 4 * hh) = o4;
      }
    if (hh == 0) {
      const double lse2 = static_cast<double>(m2) + log2(static_cast<double>(l_tot));
      LSE[static_cast<size_t>(bh) * N + row] = static_cast<float>(lse2 * kLn2);
    }
  }
}

}  // namespace hfa
