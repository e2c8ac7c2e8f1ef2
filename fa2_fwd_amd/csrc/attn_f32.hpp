// fp32 attention forward for gfx950: same online-normalisation tiling as the
// bf16 kernel (neuralmasteryai "Hardware Acceleration & Custom Kernels",
// section 2, steps 1-2), built for a 1e-5 absolute error bound on O and LSE.
//
// Precision plan.  A plain fp32 accumulation of the length-d dot products is
// not accurate enough when rows are peaked (scores of tens of units: the
// rounding of the running dot product moves exp(s - m) of the dominant keys
// by more than 1e-5 relative).  So:
//  * S^T = K Q^T runs on the fp64 matrix cores (v_mfma_f64_16x16x4_f64) from
//    the exactly widened fp32 inputs: every product is exact and the sums are
//    fp64.
//  * The running max is kept in the log2 domain and rounded up to an integer
//    m2, so each rescale factor 2^(m2_old - m2_new) is an exact power of two.
//  * s * c - m2 is formed in fp64, rounded once to fp32 and exponentiated on
//    the hardware exp2 unit; P stays fp32 and P V runs on the fp32 matrix
//    cores (v_mfma_f32_16x16x4_f32).
//  * The running denominator is accumulated in fp64, and the log-sum-exp is
//    combined in fp64 and rounded once.
//
// Matrix-core mapping.  S^T: A = 16 key rows of K, B = 16 query rows of Q, the
// contraction index d permuted so that each lane reads d/4 consecutive
// columns; the f64 accumulator gives lane (q = lane % 16, g = lane / 16)
// register r the key 4r + g of the 16-key block.  O^T = V^T P^T: for MFMA r
// of a block the B operand is that lane's own probability of key 4r + g, and
// the A operand is row 4r + g of the V tile, read as 16-byte vectors whose
// four columns feed four different column blocks.  Lane (q, g) accumulates
// output columns of its own query, so the rescale is lane-local.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace hfa {

template <int D_, int QB_, int NW_, int KT_>
struct F32Tile {
  static constexpr int D = D_;        // head dim (64 or 128)
  static constexpr int QB = QB_;      // 16-query blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup
  static constexpr int KT = KT_;      // keys per K/V tile
  static constexpr int WQ = 16 * QB;  // queries per wave
  static constexpr int BR = WQ * NW;  // queries per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int KROWB = (D + 4) * 4;  // padded K row: 8 lanes reading 8 rows hit 8 bank groups
  static constexpr int VROWB = D * 4;        // V rows are read within one row per 16 lanes
  static constexpr int KTILEB = KT * KROWB;
  static constexpr int VTILEB = KT * VROWB;
  static constexpr int CH = D / 4;  // 16-byte chunks per row
  static constexpr int LOADS = KT * CH / NT;
  static constexpr int LDS_BYTES = 2 * (KTILEB + VTILEB);
  static_assert((KT * CH) % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(KT % 16 == 0, "key tile is a whole number of 16-key MFMA blocks");
};

// The values of x in the lane pair (l, l ^ 16) or (l, l ^ 32), in an order that
// depends on the lane (use in symmetric operations only).  gfx950's
// v_permlane16_swap / v_permlane32_swap exchange 16-lane rows on the vector
// unit; both 32-bit halves of the double go through the same exchange.
template <int M>
__device__ __forceinline__ void pair_f64(double x, double& a, double& b) {
  static_assert(M == 16 || M == 32, "row exchanges of 16 or 32 lanes");
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = static_cast<uint32_t>(u), hi = static_cast<uint32_t>(u >> 32);
  auto rl = M == 16 ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                    : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto rh = M == 16 ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                    : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  a = __builtin_bit_cast(double, (static_cast<uint64_t>(rh[0]) << 32) | rl[0]);
  b = __builtin_bit_cast(double, (static_cast<uint64_t>(rh[1]) << 32) | rl[1]);
}
template <int M>
__device__ __forceinline__ double max_xor(double x) {
  double a, b;
  pair_f64<M>(x, a, b);
  return fmax(a, b);
}
template <int M>
__device__ __forceinline__ double add_xor(double x) {
  double a, b;
  pair_f64<M>(x, a, b);
  return a + b;
}

template <class T>
__global__ __launch_bounds__(T::NT) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int total_wg, double c2,
    int q_mode) {
  constexpr int D = T::D, QB = T::QB, KT = T::KT;
  constexpr int DQ = D / 4;  // contraction columns per lane
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;

  const int tile = xcd_remap(blockIdx.x, total_wg);
  const int bh = tile / n_qt, qt = tile - bh * n_qt;
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;
  float* Oh = O + head;
  const int qrow0 = qt * T::BR + wave * T::WQ;

  // ---- Q fragments: lane (i16, g) holds Q[row][g*D/4 + t], t < D/4.  q_mode
  // folds the sign of the scale into Q so that c2 > 0 below.
  const float qmul = static_cast<float>(q_mode);
  f32x4 qf[QB][DQ / 4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 16 + i16;
#pragma unroll
    for (int t4 = 0; t4 < DQ / 4; ++t4) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (row < N) x = *reinterpret_cast<const f32x4*>(Qh + static_cast<size_t>(row) * D + g * DQ + 4 * t4);
      qf[qb][t4] = x * qmul;
    }
  }

  f32x4 acc[QB][D / 16];
  double m2[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m2[qb] = -INFINITY;
    l_run[qb] = 0.0;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[qb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  u32x4 kreg[T::LOADS], vreg[T::LOADS];
  // full: tile j lies wholly below N (no key needs the bounds check).
  auto stage_load = [&](int j, auto full_tag) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_tag)::value;
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = idx / T::CH, ch = idx % T::CH;
      const int key = j * KT + row;
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (full || key < N) {
        kx = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(key) * D + ch * 4);
        vx = *reinterpret_cast<const u32x4*>(Vh + static_cast<size_t>(key) * D + ch * 4);
      }
      kreg[u] = kx;
      vreg[u] = vx;
    }
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
    char* kt = smem + buf * (T::KTILEB + T::VTILEB);
    char* vt = kt + T::KTILEB;
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = idx / T::CH, ch = idx % T::CH;
      lds_store16(kt, row * T::KROWB + ch * 16, kreg[u]);
      lds_store16(vt, row * T::VROWB + ch * 16, vreg[u]);
    }
  };

  const int ntiles = (N + KT - 1) / KT;
  stage_load(0, std::false_type{});
  stage_store(0);
  __syncthreads();

  // One key tile.  buf is the LDS buffer of tile j (j & 1), a compile-time
  // constant in the unrolled loop below so that the buffer offset folds into
  // the LDS instructions; steady: tile j + 1 is wholly below N and tile j is
  // not the last, so no bounds check, no masking and no end-of-loop test.
  auto tile_step = [&](int j, auto buf_tag, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool steady = decltype(steady_tag)::value;
    const int buf = [&] {
      if constexpr (std::is_integral_v<decltype(buf_tag)>)
        return j & 1;
      else
        return static_cast<int>(decltype(buf_tag)::value);
    }();
    if (steady)
      stage_load(j + 1, std::true_type{});
    else if (j + 1 < ntiles)
      stage_load(j + 1, std::false_type{});
    const char* kt = smem + buf * (T::KTILEB + T::VTILEB);
    const char* vt = kt + T::KTILEB;

    // ---- S^T = K Q^T in fp64
    f64x4 s[QB][KT / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) s[qb][kb] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
#pragma unroll
      for (int t4 = 0; t4 < DQ / 4; ++t4) {
        const f32x4 kf = __builtin_bit_cast(
            f32x4, lds_load16(kt, (kb * 16 + i16) * T::KROWB + (g * DQ + 4 * t4) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double a = static_cast<double>(kf[e]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            s[qb][kb] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, static_cast<double>(qf[qb][t4][e]),
                                                             s[qb][kb], 0, 0, 0);
        }
      }
    }

    // ---- keys past the end get score -inf
    const int key0 = j * KT;
    if (!steady && key0 + KT > N) {
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = key0 + kb * 16 + 4 * r + g;
          if (key >= N)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
        }
    }

    // ---- online softmax update
    f32x4 p[QB][KT / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      double mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmax(mx, s[qb][kb][r]);
      mx = max_xor<16>(mx);
      mx = max_xor<32>(mx);
      // log2-domain running max, rounded up to an integer: exact rescale factors.
      const double m_new = fmax(m2[qb], ceil(mx * c2));
      const float alpha = exp2_hw(static_cast<float>(m2[qb] - m_new));  // 0 on the first tile
      float ts = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = exp2_hw(static_cast<float>(fma(s[qb][kb][r], c2, -m_new)));
          p[qb][kb][r] = x;
          ts += x;
        }
      l_run[qb] = l_run[qb] * static_cast<double>(alpha) + static_cast<double>(ts);
      m2[qb] = m_new;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) acc[qb][n] *= alpha;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int vrow = kb * 16 + 4 * r + g;
        f32x4 vf[D / 64];
#pragma unroll
        for (int hb = 0; hb < D / 64; ++hb)
          vf[hb] = __builtin_bit_cast(f32x4, lds_load16(vt, vrow * T::VROWB + (64 * hb + 4 * i16) * 4));
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[n >> 2][n & 3], p[qb][kb][r], acc[qb][n], 0, 0, 0);
      }
    }

    if (steady || j + 1 < ntiles) stage_store(buf ^ 1);
    __syncthreads();
  };
  int j = 0;
  for (; j + 3 < ntiles; j += 2) {
    tile_step(j, std::integral_constant<int, 0>{}, std::true_type{});
    tile_step(j + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (; j < ntiles; ++j) tile_step(j, 0, std::false_type{});


  // ---- epilogue.  acc[qb][n][r] is O[q][64*(n/4) + 16g + 4r + n%4].
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const double l_tot = add_xor<32>(add_xor<16>(l_run[qb]));
    const float inv = static_cast<float>(1.0 / l_tot);
    const int row = qrow0 + qb * 16 + i16;
    if (row < N) {
      float* orow = Oh + static_cast<size_t>(row) * D;
#pragma unroll
      for (int hb = 0; hb < D / 64; ++hb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = acc[qb][4 * hb + e][r] * inv;
          *reinterpret_cast<f32x4*>(orow + 64 * hb + 16 * g + 4 * r) = o4;
        }
      if (g == 0) LSE[static_cast<size_t>(bh) * N + row] = static_cast<float>((m2[qb] + log2(l_tot)) * kLn2);
    }
  }
}

}  // namespace hfa
