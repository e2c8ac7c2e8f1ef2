// bf16 attention forward for gfx950: O = softmax(Q K^T * scale) V and its
// log-sum-exp, computed tile by tile with the online normalisation identity
// (neuralmasteryai "Hardware Acceleration & Custom Kernels", section 2,
// steps 1-2): one workgroup owns a block of query rows held in registers,
// K/V tiles stream through double-buffered LDS, and the running max, running
// denominator and running output sums are rescaled as each key tile arrives,
// so no score ever reaches HBM.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//
//  * Scores are formed transposed, S^T = K Q^T: the A operand is 32 key rows
//    of K (from LDS), the B operand is 32 query rows of Q (registers).  In
//    the 32x32 accumulator each lane then owns ONE query (lane % 32) and 16 of
//    the 32 keys, so the row max and row sum are lane-local plus one exchange
//    with the lane 32 apart.
//  * The keys fed into the A operand are permuted (row i of the MFMA reads
//    key pi(i)) so that accumulator registers r = 0..7 / 8..15 of the lane
//    half h hold the 8 consecutive keys 16*c + 8h + (r % 8) of chunk c.
//    That is exactly the B-operand layout of the next product, so P never
//    leaves registers:
//  * O^T = V^T P^T: the A operand is V^T (8 consecutive keys of one head-dim
//    column per lane), read from the row-major V tile with the gfx950
//    transposing LDS load (ds_read_b64_tr_b16, 4 keys x 16 columns per 16
//    lanes); the B operand is P rounded to bf16.  Each lane's accumulator
//    again belongs to its own query, so the per-row rescale is a lane-local
//    multiply.
#pragma once

#include "common.hpp"

namespace hfa {

template <int D_, int QB_, int NW_>
struct Bf16Tile {
  static constexpr int D = D_;        // head dim (64 or 128)
  static constexpr int QB = QB_;      // 32-query blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup
  static constexpr int KT = 64;       // keys per K/V tile
  static constexpr int WQ = 32 * QB;  // queries per wave
  static constexpr int BR = WQ * NW;  // queries per workgroup (row-tile height)
  static constexpr int NT = 64 * NW;  // threads per workgroup
  static constexpr int ROWB = D * 2;  // bytes per K or V row in LDS (XOR-swizzled, unpadded)
  static constexpr int TILEB = KT * ROWB;
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int LOADS = KT * CH / NT;   // chunks per thread per tile per tensor
  static constexpr int LDS_BYTES = 2 * 2 * TILEB;  // two buffers of (K tile, V tile)
  static_assert((KT * CH) % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(CH >= 8, "row must span all eight 16-byte bank groups");
};

// K rows: eight consecutive lanes of an S MFMA read the rows pi(0..7) =
// {0,1,2,3,8,9,10,11} (+4, +16, +20 for the other lane octets); this XOR puts
// those eight 16-byte reads on eight different bank groups.
__device__ __forceinline__ int k_swz(int row) { return (row & 3) | ((row >> 1) & 4); }
// V rows: one transposing read covers 4 consecutive rows x 32 bytes per 16
// lanes; XOR by an even value per row spreads the 4 rows over all banks.
__device__ __forceinline__ int v_swz(int row) { return (row & 3) << 1; }

template <class T>
__global__ __launch_bounds__(T::NT) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int total_wg, float c2,
    int q_mode) {
  constexpr int D = T::D, QB = T::QB, KT = T::KT, ROWB = T::ROWB, TILEB = T::TILEB;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, hh = lane >> 5;

  const int tile = xcd_remap(blockIdx.x, total_wg);
  const int bh = tile / n_qt, qt = tile - bh * n_qt;
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head;
  const __bf16* Vh = V + head;
  __bf16* Oh = O + head;
  const int qrow0 = qt * T::BR + wave * T::WQ;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[row = i32][d = 16t + 8hh .. +7].
  // q_mode folds the sign of the scale into Q (+1 keep, -1 negate, 0 zero) so
  // that the softmax below always works with a positive log2-domain scale c2.
  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + i32;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < N) x = *reinterpret_cast<const u32x4*>(Qh + static_cast<size_t>(row) * D + 16 * t + 8 * hh);
      if (q_mode < 0) x ^= 0x80008000u;
      if (q_mode == 0) x = u32x4{0u, 0u, 0u, 0u};
      qf[qb][t] = x;
    }
  }

  // ---- per-lane LDS geometry (invariant over the key loop)
  // S MFMA row i32 reads key pi(i32) of each 32-key block.
  const int a8 = i32 >> 3, e4 = (i32 >> 2) & 1, b4 = i32 & 3;
  const int krow = 16 * (a8 >> 1) + 8 * e4 + 4 * (a8 & 1) + b4;
  const int kswz = k_swz(krow);
  // Transposing V read: in each 16-lane group, lane l16 reads row 4u + l16/4 of
  // the group's 4 rows at columns 16*g16 + 4*(l16 % 4) .. +3 of the 32-column block.
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;
  const int vrow = 8 * hh + (l16 >> 2);
  const int vswz = v_swz(vrow);
  const int vch = 2 * g16 + ((l16 & 3) >> 1);
  const int vin = (l16 & 1) * 8;

  f32x16 acc[QB][D / 32];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][n][r] = 0.0f;
  }

  // ---- K/V staging: global -> registers -> LDS (swizzled), double-buffered.
  u32x4 kreg[T::LOADS], vreg[T::LOADS];
  auto stage_load = [&](int j) {
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = idx / T::CH, ch = idx % T::CH;
      const int key = j * KT + row;
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (key < N) {
        kx = *reinterpret_cast<const u32x4*>(Kh + static_cast<size_t>(key) * D + ch * 8);
        vx = *reinterpret_cast<const u32x4*>(Vh + static_cast<size_t>(key) * D + ch * 8);
      }
      kreg[u] = kx;
      vreg[u] = vx;
    }
  };
  auto stage_store = [&](int buf) {
    char* kt = smem + buf * 2 * TILEB;
    char* vt = kt + TILEB;
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = idx / T::CH, ch = idx % T::CH;
      lds_store16(kt, row * ROWB + ((ch ^ k_swz(row)) << 4), kreg[u]);
      lds_store16(vt, row * ROWB + ((ch ^ v_swz(row)) << 4), vreg[u]);
    }
  };

  const int ntiles = (N + KT - 1) / KT;
  stage_load(0);
  stage_store(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) stage_load(j + 1);
    const char* kt = smem + buf * 2 * TILEB;
    const char* vt = kt + TILEB;

    // ---- S^T = K Q^T for this tile (fp32 accumulators)
    f32x16 s[QB][KT / 32];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.0f;
#pragma unroll
    for (int kb = 0; kb < KT / 32; ++kb) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        const u32x4 kf = lds_load16(kt, (kb * 32 + krow) * ROWB + (((2 * t + hh) ^ kswz) << 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, kf), __builtin_bit_cast(bf16x8, qf[qb][t]), s[qb][kb], 0, 0, 0);
      }
    }

    // ---- keys past the end of the sequence get score -inf (weight 0)
    const int key0 = j * KT;
    if (key0 + KT > N) {
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key >= N)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
        }
    }

    // ---- online softmax update: running max, rescale factor, probabilities
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run[qb], mx);
      const float alpha = exp2_hw((m_run[qb] - m_new) * c2);  // 0 on the first tile
      const float mc = m_new * c2;
      float ts = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_hw(fmaf(s[qb][kb][r], c2, -mc));
          s[qb][kb][r] = p;
          ts += p;
        }
      l_run[qb] = l_run[qb] * alpha + ts;
      m_run[qb] = m_new;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][n][r] *= alpha;
    }

    // ---- O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int c = 0; c < KT / 16; ++c) {
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[qb][e] = static_cast<__bf16>(s[qb][c >> 1][8 * (c & 1) + e]);
#pragma unroll
      for (int n = 0; n < D / 32; ++n) {
        const int base = (16 * c + vrow) * ROWB + (((4 * n + vch) ^ vswz) << 4) + vin;
        const s16x4 lo = lds_read_tr16(vt, base);
        const s16x4 hi = lds_read_tr16(vt, base + 4 * ROWB);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb], acc[qb][n], 0, 0, 0);
      }
    }

    if (j + 1 < ntiles) stage_store(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, round to bf16, one write of O and of LSE
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = add_xor32(l_run[qb]);
    const float inv = 1.0f / l_tot;
    const int row = qrow0 + qb * 32 + i32;
    if (row < N) {
      __bf16* orow = Oh + static_cast<size_t>(row) * D;
#pragma unroll
      for (int n = 0; n < D / 32; ++n)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          bf16x4 o4;
#pragma unroll
          for (int b = 0; b < 4; ++b) o4[b] = static_cast<__bf16>(acc[qb][n][4 * a + b] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * n + 8 * a + 4 * hh) = o4;
        }
      if (hh == 0) {
        const double lse2 = static_cast<double>(m_run[qb]) * static_cast<double>(c2) + log2(static_cast<double>(l_tot));
        LSE[static_cast<size_t>(bh) * N + row] = static_cast<float>(lse2 * kLn2);
      }
    }
  }
}

}  // namespace hfa
