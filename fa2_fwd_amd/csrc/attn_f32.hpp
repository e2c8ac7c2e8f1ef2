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
//    the hardware exp2 unit, giving the fp32 weights P.
//  * P V runs on the bf16 matrix cores without losing fp32 accuracy: every
//    fp32 value x is the exact sum of three bf16 pieces x = x1 + x2 + x3
//    (x1 holds the leading 8 significant bits, x2 the next 8 of the rest,
//    x3 what is left, which has at most 8), with |x2| <= 2^-7 |x| and
//    |x3| <= 2^-14 |x|.  Of the nine cross products P_a V_b the six with
//    a + b <= 4 are formed (11, 12, 21, 13, 31, 22); the three dropped ones
//    are below 2^-21 of |P V| in each term.  Each bf16 product is exact in
//    the fp32 accumulator, and a bf16 MFMA does 16 times the work of an fp32
//    one in the same time, so the six cost 3/8 of the fp32 product.
//    V is split when its tile is staged into LDS (truncation, so the pieces
//    are exact for every finite value), P when it leaves the softmax (round
//    to nearest even; P <= 1 cannot overflow).
//  * The running denominator is accumulated in fp64, and the log-sum-exp is
//    combined in fp64 and rounded once.
//
// Matrix-core mapping.  S^T: A = 16 key rows of K, B = 16 query rows of Q, the
// contraction index d permuted so that each lane reads d/4 consecutive
// columns; the f64 accumulator gives lane (q = lane % 16, g = lane / 16)
// register r the key 4r + g of the 16-key block.  O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16, one 32-key chunk c at a time: the contraction
// slot 8g + i (i < 8) of lane group g stands for key 16 (i / 4) + 4 (i % 4) + g
// of the chunk, which is exactly the lane's own weight in register i % 4 of
// score block 2c + i / 4, so the B operand is the lane's own P.  The A operand
// (V^T, 16 head-dim columns by the same 32 keys) is stored in LDS in that
// order: each bf16 plane of a tile is [chunk][g][column][i], so a lane reads
// its 8 keys of one column as one 16-byte vector.  Lane (q, g) accumulates
// columns 16 n + 4 g + r of its own query, so the rescale is lane-local.
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
  static constexpr int KTILEB = KT * KROWB;
  static constexpr int VPLANEB = KT * D * 2;  // one bf16 piece of the V tile, [KT/32][4][D][8]
  static constexpr int VTILEB = 3 * VPLANEB;  // the three pieces of the V tile
  static constexpr int CH = D / 4;  // 16-byte chunks per K row
  static constexpr int LOADS = KT * CH / NT;
  // V is staged as (32-key chunk, key class g, column) items of 8 keys each.
  static constexpr int VITEMS = (KT / 32) * 4 * D / NT;
  static constexpr int LDS_BYTES = 2 * (KTILEB + VTILEB);
  static_assert((KT * CH) % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(KT % 32 == 0, "key tile is a whole number of 32-key chunks");
  static_assert(VITEMS >= 1 && ((KT / 32) * 4 * D) % NT == 0, "V items must divide evenly over the threads");
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

  // V item it of this thread: 32-key chunk c, key class g8 (keys 4i' + g8 of
  // the chunk, i' < 8) and column vcol.  Lanes of a wave take consecutive
  // columns, so each of the 8 loads reads whole rows of V.
  u32x4 kreg[T::LOADS];
  float vreg[T::VITEMS][8];
  // full: tile j lies wholly below N (no key needs the bounds check).
  auto stage_load = [&](int j, auto full_tag) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_tag)::value;
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = idx / T::CH, ch = idx % T::CH;
      const int key = j * KT + row;
      u32x4 kx = {0u, 0u, 0u, 0u};
      if (full || key < N) kx = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(key) * D + ch * 4);
      kreg[u] = kx;
    }
#pragma unroll
    for (int it = 0; it < T::VITEMS; ++it) {
      const int item = tid + it * T::NT;
      const int vcol = item % D, cg = item / D;
      const int c = cg >> 2, g8 = cg & 3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = j * KT + 32 * c + 16 * (i >> 2) + 4 * (i & 3) + g8;
        vreg[it][i] = (full || key < N) ? Vh[static_cast<size_t>(key) * D + vcol] : 0.0f;
      }
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
    }
    // Split each V value into three bf16 pieces by truncation: x1 keeps the
    // top 16 bits of x, x2 the top 16 bits of x - x1, x3 = x - x1 - x2 (both
    // differences exact in fp32; x3 has at most 8 significant bits, so its
    // top 16 bits are all of it).  Pieces of two keys share one 32-bit word.
#pragma unroll
    for (int it = 0; it < T::VITEMS; ++it) {
      const int item = tid + it * T::NT;
      u32x4 w1, w2, w3;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t b1[2], b2[2], b3[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float x = vreg[it][2 * h + e];
          b1[e] = __float_as_uint(x) & 0xffff0000u;
          const float r = x - __uint_as_float(b1[e]);
          b2[e] = __float_as_uint(r) & 0xffff0000u;
          b3[e] = __float_as_uint(r - __uint_as_float(b2[e]));
        }
        w1[h] = (b1[0] >> 16) | b1[1];
        w2[h] = (b2[0] >> 16) | b2[1];
        w3[h] = (b3[0] >> 16) | (b3[1] & 0xffff0000u);
      }
      lds_store16(vt, item * 16, w1);
      lds_store16(vt + T::VPLANEB, item * 16, w2);
      lds_store16(vt + 2 * T::VPLANEB, item * 16, w3);
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

    // ---- O^T += V^T P^T on the bf16 matrix cores, six piece products per
    // 32-key chunk.  P is split by round-to-nearest-even: p1 = bf16(p),
    // p2 = bf16(p - p1), p3 = p - p1 - p2 (exact in bf16).
#pragma unroll
    for (int c = 0; c < KT / 32; ++c) {
      // Two weights at a time: one v_cvt_pk_bf16_f32 rounds a pair, and the
      // rounded pair is widened back with a shift and a mask.
      u32x4 p1[QB], p2[QB], p3[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const f32x2 x = {p[qb][2 * c + (h >> 1)][2 * (h & 1)], p[qb][2 * c + (h >> 1)][2 * (h & 1) + 1]};
          const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
          const f32x2 r = x - f32x2{__uint_as_float(w1 << 16), __uint_as_float(w1 & 0xffff0000u)};
          const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
          const f32x2 t = r - f32x2{__uint_as_float(w2 << 16), __uint_as_float(w2 & 0xffff0000u)};
          p1[qb][h] = w1;
          p2[qb][h] = w2;
          p3[qb][h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2));
        }
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        const int off = ((c * 4 + g) * D + 16 * n + i16) * 16;
        const bf16x8 v1 = __builtin_bit_cast(bf16x8, lds_load16(vt, off));
        const bf16x8 v2 = __builtin_bit_cast(bf16x8, lds_load16(vt + T::VPLANEB, off));
        const bf16x8 v3 = __builtin_bit_cast(bf16x8, lds_load16(vt + 2 * T::VPLANEB, off));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const bf16x8 q1 = __builtin_bit_cast(bf16x8, p1[qb]), q2 = __builtin_bit_cast(bf16x8, p2[qb]),
                       q3 = __builtin_bit_cast(bf16x8, p3[qb]);
          f32x4 a = acc[qb][n];
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, q2, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v3, q1, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, q3, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, q1, a, 0, 0, 0);
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, q2, a, 0, 0, 0);
          acc[qb][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, q1, a, 0, 0, 0);
        }
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


  // ---- epilogue.  acc[qb][n][r] is O[q][16n + 4g + r].
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const double l_tot = add_xor<32>(add_xor<16>(l_run[qb]));
    const float inv = static_cast<float>(1.0 / l_tot);
    const int row = qrow0 + qb * 16 + i16;
    if (row < N) {
      float* orow = Oh + static_cast<size_t>(row) * D;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) *reinterpret_cast<f32x4*>(orow + 16 * n + 4 * g) = acc[qb][n] * inv;
      if (g == 0) LSE[static_cast<size_t>(bh) * N + row] = static_cast<float>((m2[qb] + log2(l_tot)) * kLn2);
    }
  }
}

}  // namespace hfa
