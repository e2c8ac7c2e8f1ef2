// fp32 attention forward for gfx950: same online-normalisation tiling as the
// bf16 kernel (neuralmasteryai "Hardware Acceleration & Custom Kernels",
// section 2, steps 1-2), built for a 1e-5 absolute error bound on O and LSE.
//
// Precision plan.  A plain fp32 accumulation of the length-d dot products is
// not accurate enough when rows are peaked (scores of tens of units: the
// rounding of the running dot product moves exp(s - m) of the dominant keys
// by more than 1e-5 relative).  So:
//  * S^T = K Q^T is formed exactly (up to one fp64 rounding) on the int8
//    matrix cores by error-free slicing (the Ozaki scheme: K. Ozaki,
//    T. Ogita, S. Oishi, S. M. Rump, "Error-free transformations of matrix
//    multiplication by using fast routines of matrix multiplication and its
//    applications", Numer. Algorithms 59, 2012; its integer form after
//    Ootomo, Ozaki and Yokota, "DGEMM on integer matrix multiplication
//    unit", IJHPCA 2024).  Each row x of Q and of K is written with a power
//    of two 2^e above its largest magnitude as
//        x = 2^(e-6) * sum_{a<5} s_a 2^(-7a) + r,   s_a integers, |s_a| <= 64,
//    with |r| <= 2^(e-35) (zero for every element within 2^-11 of the row
//    maximum, since fp32 carries 24 significant bits).  The slice products
//    sum_d s_a(q) s_b(k) are exact in the int32 accumulators; those with
//    a + b <= 5 are formed (19 of 25; each dropped one is below 2^-40 of
//    max|q| max|k| per column), grouped by a + b, and combined in fp64.
//    int8 MFMAs run at 64 times the fp64 rate, so the 19 cost 0.3 of the
//    fp64 product.
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
// K/V staging, two routes with the same LDS image and therefore the same
// bits: every workgroup formats each key tile itself as it stages it (slices
// and exponents of K, pieces of V), or, given a workspace, f32_pack_kernel
// formats every tile once per call and the attention kernel copies the tile
// images from HBM into LDS as they are (global_load_lds_dwordx4).
//
// Matrix-core mapping.  S^T on v_mfma_i32_16x16x64_i8: A = one slice of 16
// key rows (64 head-dim columns per instruction, lane group g holding columns
// 16g .. 16g + 15), B = one slice of 16 query rows in the same column order;
// the int32 result gives lane (q = lane % 16, g = lane / 16) register r the
// key 4g + r of the 16-key block.  O^T = V^T P^T on
// v_mfma_f32_16x16x32_bf16, one 32-key chunk c at a time: the contraction
// slot 8g + i (i < 8) of lane group g stands for key 16 (i / 4) + 4 g + i % 4
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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int D_, int QB_, int NW_, int KT_>
struct F32Tile {
  static constexpr int D = D_;        // head dim (64 or 128)
  static constexpr int QB = QB_;      // 16-query blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup
  static constexpr int KT = KT_;      // keys per K/V tile
  static constexpr int WQ = 16 * QB;  // queries per wave
  static constexpr int BR = WQ * NW;  // queries per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int NSL = 5;           // int8 slices per fp32 value
  static constexpr int KSROW = D == 64 ? 96 : D;  // bytes per key row of one slice plane (see kswz)
  static constexpr int KSPLANEB = KT * KSROW;
  static constexpr int KEXPB = NSL * KSPLANEB;  // offset of the per-key exponents (int32)
  static constexpr int KTILEB = KEXPB + KT * 4;  // the slice planes, then each key's exponent
  static constexpr int VPLANEB = KT * D * 2;  // one bf16 piece of the V tile, [KT/32][4][D][8]
  static constexpr int VTILEB = 3 * VPLANEB;  // the three pieces of the V tile
  static constexpr int CH = D / 4;  // 16-byte chunks per K row
  static constexpr int LOADS = KT * CH / NT;
  // V is staged as (32-key chunk, key class g, column) items of 8 keys each.
  static constexpr int VITEMS = (KT / 32) * 4 * D / NT;
  static constexpr int MISCB = 2 * (KTILEB + VTILEB);  // per-wave key statistics for the exactness check
  static constexpr int LDS_BYTES = MISCB + NW * (CH + 1) * 4;
  // Pre-formatted tiles (f32_pack_kernel), PACKB bytes each: the K image of
  // an LDS buffer followed by the tile's key statistics (CH floats and one
  // int), padded to KPADB, then the V image (VPADB), each part a whole number
  // of rounds of 16-byte copies by all NT threads.  In LDS the two K parts
  // come first (buffer b at b KPADB) and the two V parts after them, so that
  // every K read of either buffer lies within the 64 KiB an LDS instruction's
  // immediate offset reaches from one base.
  static constexpr int STATB = 4 * (CH + 1);
  static constexpr int ROUNDB = 16 * NT;
  static constexpr int KPADB = (KTILEB + STATB + ROUNDB - 1) / ROUNDB * ROUNDB;
  static constexpr int VPADB = (VTILEB + ROUNDB - 1) / ROUNDB * ROUNDB;
  static constexpr int PACKB = KPADB + VPADB;
  static constexpr int PCOPIES = PACKB / ROUNDB;  // 16-byte copies per thread per tile
  static constexpr int KCOPIES = KPADB / ROUNDB;  // of which into the K part
  static constexpr int P_MISCB = 2 * PACKB;
  static constexpr int P_LDS_BYTES = P_MISCB + NW * (CH + 1) * 4;
  static_assert(KTILEB % 16 == 0, "the statistics start 16-byte aligned");
  static_assert(2 * KPADB <= 65536, "both K parts lie within 64 KiB");
  static_assert((KT * CH) % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(KT % 32 == 0, "key tile is a whole number of 32-key chunks");
  static_assert(CH == 16 || CH == 32, "a K row spans 16 or 32 lanes (d = 64 or 128)");
  static_assert(VITEMS >= 1 && ((KT / 32) * 4 * D) % NT == 0, "V items must divide evenly over the threads");
};

// K slice planes, laid out for conflict-free LDS access on gfx950 (measured
// with SQ_LDS_BANK_CONFLICT on probe patterns):
//  * The score reads take 16 bytes per lane: chunk g (+ 4h) of 16 consecutive
//    rows, the four lane groups g side by side.  With rows at an odd multiple
//    of 32 bytes apart these are conflict-free; with rows 64 or 80 bytes apart
//    (any XOR of the chunk tried) they cost 4 extra cycles per read.  So d = 64
//    rows are 96 bytes apart (32 bytes of padding).  At d = 128, rows 128
//    bytes apart with chunk c stored at chunk c ^ ((r / 2) % 8) are
//    conflict-free.
//  * The staging stores take 4 bytes per lane, 4 rows of 64 bytes (d = 64) or
//    2 of 128 bytes (d = 128) per wave instruction; they are conflict-free when
//    those rows cover disjoint 64-dword bank windows.  96-byte rows start 24
//    dwords apart, so a wave stores rows of one parity within a group of 8
//    (stage_row): windows at 0, 48, 32, 16 or 24, 8, 56, 40.
template <int D>
__device__ __forceinline__ int kswz(int row) {
  return D == 64 ? 0 : (row >> 1) & 7;
}
// The key row (within a tile) that staging position q (= thread index / CH,
// per load) takes: at d = 64, positions 8k + m go to rows 8k + 2 (m % 4) + m / 4.
template <int D>
__device__ __forceinline__ int stage_row(int q) {
  return D == 64 ? (q & ~7) | ((q & 3) << 1) | ((q >> 2) & 1) : q;
}

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

// Largest value over each row of 16 lanes (DPP: swap neighbours, swap
// pairs, mirror within 8, mirror within 16).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float max_row16(float x) {
  x = fmaxf(x, dpp_f32<0xB1>(x));   // quad_perm [1, 0, 3, 2]
  x = fmaxf(x, dpp_f32<0x4E>(x));   // quad_perm [2, 3, 0, 1]
  x = fmaxf(x, dpp_f32<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_f32<0x140>(x));  // row_mirror
  return x;
}
__device__ __forceinline__ float add_xor16_f32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Largest value over the lane pair (l, l ^ 16) / (l, l ^ 32).
__device__ __forceinline__ float max_xor16_f32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exponent e with |x| < 2^e for the largest magnitude m of a row (0 when the
// row is all zero, whose slices are then all zero).
__device__ __forceinline__ int row_exponent(float m) { return __builtin_amdgcn_frexp_expf(m); }

// The five int8 slices of four values of one row whose magnitudes are below
// 2^e: x = 2^(e-6) sum_a s_a 2^(-7a) + r with |s_a| <= 64 and |r| <= 2^(e-35).
// Slice a is the remainder rounded to the grid 2^(-7a) (after scaling by
// 2^(6-e)): adding 1.5 * 2^(23-7a) rounds it to nearest even and leaves the
// integer s_a in the low byte of the sum's bit pattern; subtracting the
// rounded value back is exact.  w[a] packs s_a of the four values, value 0 in
// the low byte.
__device__ __forceinline__ void slice5(f32x4 x, int e, uint32_t (&w)[5]) {
  float r[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = __builtin_amdgcn_ldexpf(x[k], 6 - e);
#pragma unroll
  for (int a = 0; a < 5; ++a) {
    const float M = 12582912.0f / static_cast<float>(1 << (7 * a));  // 1.5 * 2^(23 - 7a), exact
    uint32_t b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float f = r[k] + M;
      b[k] = __float_as_uint(f);
      if (a < 4) r[k] -= f - M;
    }
    w[a] = (b[0] & 0xffu) | ((b[1] & 0xffu) << 8) | ((b[2] & 0xffu) << 16) | (b[3] << 24);
  }
}

#ifndef HFA_F32_SKEW
#define HFA_F32_SKEW 1
#endif

// Workgroup barrier that waits only for this wave's LDS operations.
__device__ __forceinline__ void lds_barrier_f32() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Largest bound on the error of an int8-slice score (natural-log units) that
// a tile may have and keep the int8 products: 2^-22, so that with scores off
// by at most this much, O moves by at most 2^-22 (max v - min v) and the
// log-sum-exp by 2^-22 -- a small part of the 1e-5 budget.
constexpr double kExactScoreBound = 0x1p-22;

// Exact recomputation of one wave's query rows (16 QB rows from qrow0), for
// waves whose int8-slice scores are not accurate enough (inputs whose rows mix
// magnitudes far apart, so that a small entry of one row meets a large entry
// of the other).  Everything comes straight from memory, no LDS and no
// barrier; the same online normalisation, with both products on the fp64
// matrix cores (v_mfma_f64_16x16x4_f64):
//  * S^T = K Q^T per 16-key block: A row i reads key 4 (i % 4) + i / 4 of the
//    block (the f64 product leaves register r of lane group g with output row
//    4 r + g, so lane (i16, g) register r holds key 4 g + r for query i16);
//    lane group g contracts the columns g d/4 .. g d/4 + d/4 - 1.  Each
//    product of two fp32 values is exact in fp64, the sums are fp64.
//  * The running max is in log2 units, rounded up to an integer, so rescale
//    factors are exact powers of two; weights p = exp2 of the fp64 argument
//    rounded to fp32 (as in the fast path), kept in fp64.
//  * O^T += V^T P^T per 16-column block n: A = V[key 4 g + t][16 n + i16],
//    B = the lane's own weight of key 4 g + t (register t), for t < 4; lane
//    (i16, g) register r accumulates column 16 n + 4 r + g of query i16.
template <int D, int QB>
__device__ __forceinline__ void exact_rows_impl(const float* __restrict__ Qh, const float* __restrict__ Kh,
                                                         const float* __restrict__ Vh, float* __restrict__ Oh,
                                                         float* __restrict__ lse_h, int N, int qrow0, double c2,
                                                         float qmul, int lane) {
  constexpr int DQ = D / 4;
  const int i16 = lane & 15, g = lane >> 4;
  const int pi = 4 * (i16 & 3) + (i16 >> 2);  // key of A row i16 within a 16-key block
  f64x4 acc[QB][D / 16];
  double m2[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m2[qb] = -INFINITY;
    l_run[qb] = 0.0;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[qb][n] = f64x4{0.0, 0.0, 0.0, 0.0};
  }
  for (int k0 = 0; k0 < N; k0 += 16) {
    f64x4 s[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = f64x4{0.0, 0.0, 0.0, 0.0};
    const float* krow = Kh + (min(k0 + pi, N - 1) * D + g * DQ);
#pragma unroll 2
    for (int t4 = 0; t4 < DQ / 4; ++t4) {
      const f32x4 kf = *reinterpret_cast<const f32x4*>(krow + 4 * t4);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = min(qrow0 + 16 * qb + i16, N - 1);
        const f32x4 qf = *reinterpret_cast<const f32x4*>(Qh + (row * D + g * DQ + 4 * t4)) * qmul;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[qb] = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(kf[e]), static_cast<double>(qf[e]), s[qb],
                                                       0, 0, 0);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      double mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (k0 + 4 * g + r >= N) s[qb][r] = -INFINITY;
        mx = fmax(mx, s[qb][r]);
      }
      mx = max_xor<32>(max_xor<16>(mx));
      const double m_new = fmax(m2[qb], ceil(mx * c2));
      const double alpha = __builtin_amdgcn_ldexp(1.0, static_cast<int>(fmax(m2[qb] - m_new, -1022.0)));
      double p[4], ts = 0.0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = static_cast<double>(exp2_hw(static_cast<float>(fma(s[qb][r], c2, -m_new))));
        ts += p[r];
      }
      l_run[qb] = l_run[qb] * alpha + ts;
      m2[qb] = m_new;
#pragma unroll
      for (int n = 0; n < D / 16; ++n) {
        f64x4 a = acc[qb][n] * alpha;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float vv = Vh[min(k0 + 4 * g + t, N - 1) * D + 16 * n + i16];
          a = __builtin_amdgcn_mfma_f64_16x16x4f64(static_cast<double>(vv), p[t], a, 0, 0, 0);
        }
        acc[qb][n] = a;
      }
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const double l_tot = add_xor<32>(add_xor<16>(l_run[qb]));
    const int row = qrow0 + 16 * qb + i16;
    if (row < N) {
      float* orow = Oh + row * D;
#pragma unroll
      for (int n = 0; n < D / 16; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) orow[16 * n + 4 * r + g] = static_cast<float>(acc[qb][n][r] / l_tot);
      if (g == 0) lse_h[row] = static_cast<float>((m2[qb] + log2(l_tot)) * kLn2);
    }
  }
}

// ---- S^T = K Q^T from the int8 slices for one 16-key block (slices ks of
// the block's key rows, ek their exponents) and one 16-query block (slices
// qsb): the slice products with a + b = t accumulate exactly in acc_t
// (|acc_t| < 2^21), and s = 2^(eq + ek - 12) sum_t acc_t 2^(-7t) is
// 2^(eq - 47) 2^ek (acc01 2^28 + acc23 2^14 + acc45) with acc01 = 2^7 acc_0 +
// acc_1 etc. formed exactly in int32.  This returns s 2^(47 - eq) 2^e_add,
// exact in fp64 up to the one rounding of the sum.  The query's factor
// 2^(eq - 47) is the same for all its keys, so it can go into c2 instead
// (e_add = 0, and c2q below), saving an add per score.  The d = 64 tiles do
// that except the unpacked 256-row one, where the per-query-block c2q would
// not fit in its registers; the d = 128 tiles keep the factor here
// (e_add = eq - 47): folded, their packed 64-row tile ran 8 % slower.  Either
// way the products with c2 are the same bits.
template <class T>
__device__ __forceinline__ f64x4 score_block_f32(const i32x4 (&ks)[T::D / 64][T::NSL],
                                                 const u32x4 (&qsb)[T::D / 64][T::NSL], i32x4 ek, int e_add) {
  i32x4 at[2 * T::NSL - 4];
#pragma unroll
  for (int t = 0; t < 2 * T::NSL - 4; ++t) at[t] = i32x4{0, 0, 0, 0};
#pragma unroll
  for (int h = 0; h < T::D / 64; ++h)
#pragma unroll
    for (int a2 = 0; a2 < T::NSL; ++a2)
#pragma unroll
      for (int b2 = 0; b2 < T::NSL; ++b2)
        if (a2 + b2 <= 5)
          at[a2 + b2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ks[h][a2], __builtin_bit_cast(i32x4, qsb[h][b2]),
                                                              at[a2 + b2], 0, 0, 0);
  f64x4 s;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int a01 = at[0][r] * 128 + at[1][r];
    const int a23 = at[2][r] * 128 + at[3][r];
    const int a45 = at[4][r] * 128 + at[5][r];
    const double x = fma(static_cast<double>(a01), 268435456.0,
                         fma(static_cast<double>(a23), 16384.0, static_cast<double>(a45)));
    s[r] = __builtin_amdgcn_ldexp(x, ek[r] + e_add);
  }
  return s;
}

// ---- online softmax update of one 16-query block over a key tile: scores
// sb (the true scores times a power of two, see score_block_f32), weights pb
// out; running max m2 (log2 units), denominator l and output sums accb
// updated.  c2q is |scale| log2(e) times the inverse power of two, so sb c2q
// is the score in log2 units: power-of-two factors being exact, the products
// equal those of the true scores with |scale| log2(e).
template <class T>
__device__ __forceinline__ void softmax_block_f32(const f64x4 (&sb)[T::KT / 16], f32x4 (&pb)[T::KT / 16], double& m2,
                                                  double& l, f32x4 (&accb)[T::D / 16], double c2q) {
  double mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < T::KT / 16; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmax(mx, sb[kb][r]);
  mx = max_xor<16>(mx);
  mx = max_xor<32>(mx);
  // log2-domain running max, rounded up to an integer: exact rescale factors.
  const double m_new = fmax(m2, ceil(mx * c2q));
  const float alpha = exp2_hw(static_cast<float>(m2 - m_new));  // 0 on the first tile
  float ts = 0.0f;
#pragma unroll
  for (int kb = 0; kb < T::KT / 16; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float x = exp2_hw(static_cast<float>(fma(sb[kb][r], c2q, -m_new)));
      pb[kb][r] = x;
      ts += x;
    }
  l = l * static_cast<double>(alpha) + static_cast<double>(ts);
  m2 = m_new;
#pragma unroll
  for (int n = 0; n < T::D / 16; ++n) accb[n] *= alpha;
}

// Formats K and V once per call for the packed attention kernel: workgroup
// (bh, j) writes tile j of head bh exactly as the attention kernel's own
// staging leaves it in an LDS buffer (int8 slice planes and row exponents of
// K, bf16 pieces of V, keys at or past N zero), followed by the tile's key
// statistics for the exactness check: per column chunk the largest L1 norm
// of a key row's chunk, then the largest key exponent.  The thread mapping
// and the arithmetic are those of the staging, so both paths feed the matrix
// cores the same bytes and give identical results.
template <class T>
__global__ __launch_bounds__(T::NT) void f32_pack_kernel(const float* __restrict__ K, const float* __restrict__ V,
                                                         char* __restrict__ ws, int N, int ntiles) {
  constexpr int D = T::D, KT = T::KT, CH = T::CH;
  __shared__ float red_a[T::NW][CH];
  __shared__ int red_e[T::NW];
  const int tid = thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int blk = group_id();
  const int bh = uniform_sgpr(blk / ntiles);
  const int j = uniform_sgpr(blk - bh * ntiles);
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  const float* Kh = K + head;
  const float* Vh = V + head;
  char* kt = ws + static_cast<size_t>(blk) * T::PACKB;
  char* vt = kt + T::KPADB;

  float kmax_a = 0.0f;
  int kmax_e = -1024;
#pragma unroll
  for (int u = 0; u < T::LOADS; ++u) {
    const int idx = tid + u * T::NT;
    const int row = stage_row<D>(idx / CH), ch = idx % CH;
    const int key = j * KT + row;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (key < N) x = *reinterpret_cast<const f32x4*>(Kh + (key * D + ch * 4));
    float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    kmax_a = fmaxf(kmax_a, (fabsf(x[0]) + fabsf(x[1])) + (fabsf(x[2]) + fabsf(x[3])));
    mx = max_row16(mx);
    if constexpr (CH == 32) mx = max_xor16_f32(mx);
    const int e = row_exponent(mx);
    uint32_t w[T::NSL];
    slice5(x, e, w);
    const int off = row * T::KSROW + (((ch >> 2) ^ kswz<D>(row)) << 4) + 4 * (ch & 3);
#pragma unroll
    for (int a2 = 0; a2 < T::NSL; ++a2) *reinterpret_cast<uint32_t*>(kt + off + a2 * T::KSPLANEB) = w[a2];
    if (ch == 0) *reinterpret_cast<int*>(kt + T::KEXPB + 4 * row) = e;
    kmax_e = max(kmax_e, e);
  }
  // V items as in the staging: 32-key chunk c, key class g8, column vcol;
  // three bf16 pieces by truncation, pieces of two keys per 32-bit word.
#pragma unroll
  for (int it = 0; it < T::VITEMS; ++it) {
    const int item = tid + it * T::NT;
    const int vcol = item % D, cg = item / D;
    const int c = cg >> 2, g8 = cg & 3;
    float xv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = j * KT + 32 * c + 16 * (i >> 2) + 4 * g8 + (i & 3);
      xv[i] = key < N ? Vh[key * D + vcol] : 0.0f;
    }
    u32x4 w1, w2, w3;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      uint32_t b1[2], b2[2], b3[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x = xv[2 * h + e];
        b1[e] = __float_as_uint(x) & 0xffff0000u;
        const float r = x - __uint_as_float(b1[e]);
        b2[e] = __float_as_uint(r) & 0xffff0000u;
        b3[e] = __float_as_uint(r - __uint_as_float(b2[e]));
      }
      w1[h] = (b1[0] >> 16) | b1[1];
      w2[h] = (b2[0] >> 16) | b2[1];
      w3[h] = (b3[0] >> 16) | (b3[1] & 0xffff0000u);
    }
    *reinterpret_cast<u32x4*>(vt + item * 16) = w1;
    *reinterpret_cast<u32x4*>(vt + T::VPLANEB + item * 16) = w2;
    *reinterpret_cast<u32x4*>(vt + 2 * T::VPLANEB + item * 16) = w3;
  }
  // The tile's statistics: lanes l, l + CH, ... of a wave share a column chunk.
#pragma unroll
  for (int m = 1; m < 64; m *= 2) {
    kmax_e = max(kmax_e, __shfl_xor(kmax_e, m));
    if (m >= CH) kmax_a = fmaxf(kmax_a, __shfl_xor(kmax_a, m));
  }
  if (lane < CH) red_a[wave][lane] = kmax_a;
  if (lane == 0) red_e[wave] = kmax_e;
  __syncthreads();
  char* st = kt + T::KTILEB;
  if (tid < CH) {
    float m = 0.0f;
#pragma unroll
    for (int w = 0; w < T::NW; ++w) m = fmaxf(m, red_a[w][tid]);
    reinterpret_cast<float*>(st)[tid] = m;
  } else if (tid == CH) {
    int m = -1024;
#pragma unroll
    for (int w = 0; w < T::NW; ++w) m = max(m, red_e[w]);
    reinterpret_cast<int*>(st)[CH] = m;
  }
}

// PACKED: K and V tiles come pre-formatted from f32_pack_kernel (`packed`,
// [B*H][ntiles][PACKB]) and are copied into LDS as they are, with no staging
// arithmetic; otherwise the workgroup formats every tile itself.
//
// 4-wave workgroups are compiled for two waves per SIMD, i.e. at most 256
// registers a wave: allowed the whole register file, the compiler parks plain
// values in accumulation registers and pays a v_accvgpr move for each use.
#ifndef HFA_F32_NW4_WAVES_PER_EU
#define HFA_F32_NW4_WAVES_PER_EU 2
#endif
template <class T, bool PACKED = false>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::NW == 4 ? HFA_F32_NW4_WAVES_PER_EU : 1)))
void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int total_wg, double c2,
    int q_mode, const char* __restrict__ packed) {
  constexpr int D = T::D, QB = T::QB, KT = T::KT;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = thread_id();
  const int lane = tid & 63, wave = tid >> 6;
  const int i16 = lane & 15, g = lane >> 4;
  // With 8 waves, waves 4..7 (one per SIMD) take the tile's phases in another
  // order: they store their half of the next tile at the start of the
  // interval instead of at its end (and request the one after it straight
  // away), so their staging work overlaps the other wave's score products and
  // the other wave's staging overlaps their P V products.
  constexpr bool kSkew = HFA_F32_SKEW && T::NW == 8 && !PACKED;
  const bool late = kSkew && __builtin_amdgcn_readfirstlane(tid >> 6) >= T::NW / 2;

  // Workgroup-uniform indices, kept in scalar registers (the division runs on
  // the vector unit; left there, every per-head pointer below would occupy
  // vector registers for the whole kernel).
  const int tile = xcd_remap(group_id(), total_wg);
  const int bh = uniform_sgpr(tile / n_qt);
  const int qt = uniform_sgpr(tile - bh * n_qt);
  // Per-head pointers (wave-uniform); offsets within a head fit in 32 bits
  // (N d < 2^31), so per-lane row offsets stay 32-bit.
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  float* const lse_h = LSE + static_cast<size_t>(bh) * N;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;
  float* Oh = O + head;
  const int qrow0 = qt * T::BR + wave * T::WQ;

  const int ntiles = (N + KT - 1) / KT;
  // Packed tiles: buffer b holds a tile's K part at smem + b * KPADB and its V
  // part at smem + 2 KPADB + b * VPADB; each of the NT threads copies 16 bytes
  // per round, wave w's lanes filling 1 KiB of the round.
  const char* blobs = PACKED ? packed + static_cast<size_t>(bh) * static_cast<size_t>(ntiles) * T::PACKB : nullptr;
  // The round moves the scalar source and LDS bases; the lane's offset is one
  // register, recomputed from an opaque thread index (not kept across the loop).
  // The LDS addresses are scalar: the buffer base plus this wave's 1 KiB.
  const uint32_t wave_lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)smem)) +
                            1024u * static_cast<uint32_t>(uniform_sgpr(tid >> 6));
  auto copy_tile = [&](int jj, int b) __attribute__((always_inline)) {
    const char* src = blobs + static_cast<size_t>(jj) * T::PACKB;
    const uint32_t kdst = wave_lds + b * T::KPADB;
    const uint32_t vdst = wave_lds + 2 * T::KPADB + b * T::VPADB;
    int voff = tid;
    asm volatile("" : "+v"(voff));
    voff *= 16;
#pragma unroll
    for (int u = 0; u < T::PCOPIES; ++u)
      dma16_to(src + u * T::ROUNDB, voff,
               u < T::KCOPIES ? kdst + u * T::ROUNDB : vdst + (u - T::KCOPIES) * T::ROUNDB);
  };
  // V item it of this thread: 32-key chunk c, key class g8 (keys
  // 16 (i / 4) + 4 g8 + i % 4 of the chunk, i < 8) and column vcol.  Lanes of a
  // wave take consecutive columns, so each of the 8 loads reads whole rows.
  u32x4 kreg[T::LOADS];
  float vreg[T::VITEMS][8];
  // full: tile j lies wholly below N (no key needs the bounds check).
  auto stage_load = [&](int j, auto full_tag) __attribute__((always_inline)) {
    constexpr bool full = decltype(full_tag)::value;
    // In the 256-row tile, an opaque copy of the thread index, as in
    // stage_store: the per-lane address parts are recomputed here instead of
    // being spilled across the key loop (and reloaded inside it).  The other
    // tilings have the registers to keep them.
    int tid_here = tid;
    if constexpr (T::QB >= 2) asm volatile("" : "+v"(tid_here));
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid_here + u * T::NT;
      const int row = stage_row<D>(idx / T::CH), ch = idx % T::CH;
      const int key = j * KT + row;
      u32x4 kx = {0u, 0u, 0u, 0u};
      if (full || key < N) kx = *reinterpret_cast<const u32x4*>(Kh + (key * D + ch * 4));
      kreg[u] = kx;
    }
#pragma unroll
    for (int it = 0; it < T::VITEMS; ++it) {
      const int item = tid_here + it * T::NT;
      const int vcol = item % D, cg = item / D;
      const int c = cg >> 2, g8 = cg & 3;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = j * KT + 32 * c + 16 * (i >> 2) + 4 * g8 + (i & 3);
        vreg[it][i] = (full || key < N) ? Vh[key * D + vcol] : 0.0f;
      }
    }
  };
  // The first K/V tile is requested before the Q loads, so that the two HBM
  // round trips overlap.
  if constexpr (PACKED)
    copy_tile(0, 0);
  else
    stage_load(0, std::false_type{});

  // ---- Q slices (B operand of S^T): lane (i16, g) holds, for each 64-column
  // block h, columns 64h + 16g .. 64h + 16g + 15 of its query row, as five
  // int8 slices under the row's exponent eq.  q_mode folds the sign of the
  // scale into Q so that c2 > 0 below.
  const float qmul = static_cast<float>(q_mode);
  u32x4 qs[QB][D / 64][T::NSL];
  int eq[QB];
  // Where the query exponent goes (see score_block_f32): c2q[qb] =
  // 2^(eq - 47) c2 with e_add = 0, or c2 with e_add = eq - 47.
  constexpr bool kFoldEq = D == 64 && (PACKED || QB == 1);
  double c2q[QB];
  // The wave's query statistics for the exactness check of each key tile:
  // the largest 2^e_q and the largest L1 norm sum_c |q_c| over its rows.
  float wave_b = 0.0f, wave_a = 0.0f;
  // Every query block's loads first, unconditional (rows past the end read
  // row N - 1 and are zeroed below): a load under a lane mask is waited for
  // on the spot.
  f32x4 xq[QB][D / 64][4];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4)
        xq[qb][h][t4] = *reinterpret_cast<const f32x4*>(
            Qh + (min(qrow0 + qb * 16 + i16, N - 1) * D + 64 * h + 16 * g + 4 * t4));
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 16 + i16;
    f32x4 x[D / 64][4];
    float mx = 0.0f, l1 = 0.0f;
    const float qrow_mul = row < N ? qmul : 0.0f;
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        const f32x4 v = xq[qb][h][t4] * qrow_mul;
        x[h][t4] = v;
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
        l1 += (fabsf(v[0]) + fabsf(v[1])) + (fabsf(v[2]) + fabsf(v[3]));
      }
    mx = max_xor32(max_xor16_f32(mx));
    l1 = add_xor32(add_xor16_f32(l1));
    eq[qb] = row_exponent(mx);
    c2q[qb] = kFoldEq ? __builtin_amdgcn_ldexp(c2, eq[qb] - 47) : c2;
    if (mx > 0.0f) wave_b = fmaxf(wave_b, __builtin_amdgcn_ldexpf(1.0f, eq[qb]));
    wave_a = fmaxf(wave_a, l1);
#pragma unroll
    for (int h = 0; h < D / 64; ++h)
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        uint32_t w[T::NSL];
        slice5(x[h][t4], eq[qb], w);
#pragma unroll
        for (int a2 = 0; a2 < T::NSL; ++a2) qs[qb][h][a2][t4] = w[a2];
      }
  }

  // Every lane of a 16-lane row holds one query; the four rows hold the same
  // queries, so a row reduction gives the wave's maxima (kept in scalar
  // registers: they are only needed after the key loop).
  wave_b = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(max_row16(wave_b))));
  wave_a = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(max_row16(wave_a))));
  // The largest exponent of the key rows this thread stages, and the largest
  // L1 norm of its column chunk of them.
  int kmax_e = -1024;
  float kmax_a = 0.0f;

  f32x4 acc[QB][D / 16];
  double m2[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m2[qb] = -INFINITY;
    l_run[qb] = 0.0;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) acc[qb][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto stage_store = [&](int buf) __attribute__((always_inline)) {
    char* kt = smem + buf * (T::KTILEB + T::VTILEB);
    char* vt = kt + T::KTILEB;
    // K rows as int8 slices under each row's own exponent.  The CH lanes
    // holding one row (16 or 32 consecutive lanes) agree on its largest
    // magnitude first.
#pragma unroll
    for (int u = 0; u < T::LOADS; ++u) {
      const int idx = tid + u * T::NT;
      const int row = stage_row<D>(idx / T::CH), ch = idx % T::CH;
      const f32x4 x = __builtin_bit_cast(f32x4, kreg[u]);
      float mx = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
      // this lane's part of the row's L1 norm (its column chunk is the same in
      // every row it stages: ch = tid % CH)
      kmax_a = fmaxf(kmax_a, (fabsf(x[0]) + fabsf(x[1])) + (fabsf(x[2]) + fabsf(x[3])));
      mx = max_row16(mx);
      if constexpr (T::CH == 32) mx = max_xor16_f32(mx);
      const int e = row_exponent(mx);
      uint32_t w[T::NSL];
      slice5(x, e, w);
      // One opaque address for this lane's five slice stores (the planes are
      // immediate offsets from it), recomputed here like the thread index.
      int off0 = row * T::KSROW + (((ch >> 2) ^ kswz<D>(row)) << 4) + 4 * (ch & 3);
      asm volatile("" : "+v"(off0));
#pragma unroll
      for (int a2 = 0; a2 < T::NSL; ++a2) *reinterpret_cast<uint32_t*>(kt + off0 + a2 * T::KSPLANEB) = w[a2];
      if (ch == 0) {
        // the row again from an opaque thread index: its address is not kept
        // (or spilled) across the key loop
        int tid_e = tid;
        asm volatile("" : "+v"(tid_e));
        *reinterpret_cast<int*>(kt + T::KEXPB + 4 * stage_row<D>((tid_e + u * T::NT) / T::CH)) = e;
      }
      kmax_e = max(kmax_e, e);
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

  if constexpr (PACKED) {
    // tile 0 was requested before the Q loads
    vmcnt_wait<0>();
    __syncthreads();
  } else {
    stage_store(0);  // tile 0 was requested before the Q loads
    if (late && ntiles > 1) stage_load(1, std::false_type{});
    __syncthreads();
  }

  // One key tile.  buf is the LDS buffer of tile j (j & 1), a compile-time
  // constant in the unrolled loop below so that the buffer offset folds into
  // the LDS instructions; steady: every tile requested in this step (j + 1,
  // or j + 2 for the late waves) is wholly below N and tile j is not the
  // last, so no bounds check, no masking and no end-of-loop test.  The next
  // tile goes into the other buffer, which no wave reads during this tile:
  // the early waves request it at the start and store it at the end, the
  // late waves store it at the start (requested one tile earlier).
  auto tile_step = [&](int j, auto buf_tag, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool steady = decltype(steady_tag)::value;
    const int buf = [&] {
      if constexpr (std::is_integral_v<decltype(buf_tag)>)
        return j & 1;
      else
        return static_cast<int>(decltype(buf_tag)::value);
    }();
    if constexpr (PACKED) {
      if (steady || j + 1 < ntiles) copy_tile(j + 1, buf ^ 1);
    } else if constexpr (kSkew) {
      if (late) {
        // the late waves' half of tile j + 1, requested at the start of tile
        // j - 1, then their request for tile j + 2
        if (steady || j + 1 < ntiles) stage_store(buf ^ 1);
        if (steady)
          stage_load(j + 2, std::true_type{});
        else if (j + 2 < ntiles)
          stage_load(j + 2, std::false_type{});
      } else {
        if (steady)
          stage_load(j + 1, std::true_type{});
        else if (j + 1 < ntiles)
          stage_load(j + 1, std::false_type{});
      }
    } else {
      if (steady)
        stage_load(j + 1, std::true_type{});
      else if (j + 1 < ntiles)
        stage_load(j + 1, std::false_type{});
    }
    const char* kt = smem + buf * (PACKED ? T::KPADB : T::KTILEB + T::VTILEB);
    const char* vt = PACKED ? smem + 2 * T::KPADB + buf * T::VPADB : kt + T::KTILEB;

    // ---- S^T = K Q^T from the int8 slices: for each 16-key block, the slice
    // products with a + b = t accumulate exactly in acc_t (|acc_t| < 2^21),
    // then s = 2^(eq + ek - 12) sum_t acc_t 2^(-7t) in fp64, combined as
    // 2^-35 (acc01 2^28 + acc23 2^14 + acc45) with acc01 = 2^7 acc_0 + acc_1
    // etc. formed exactly in int32.
    f64x4 s[QB][KT / 16];
    f32x4 p[QB][KT / 16];
    // ---- keys past the end get score -inf
    const int key0 = j * KT;
    if constexpr (PACKED && QB > 1) {
      // One query block at a time (its scores, then its softmax): only one
      // block's fp64 scores are live, and the softmax of a block can overlap
      // the score products of the next.  The K slices are read once per block.
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int kb = 0; kb < KT / 16; ++kb) {
          i32x4 ks[D / 64][T::NSL];
#pragma unroll
          for (int h = 0; h < D / 64; ++h)
#pragma unroll
            for (int a2 = 0; a2 < T::NSL; ++a2)
              ks[h][a2] = __builtin_bit_cast(i32x4, lds_load16(kt, a2 * T::KSPLANEB + (kb * 16 + i16) * T::KSROW +
                                                                       (((4 * h + g) ^ kswz<D>(i16)) << 4)));
          const i32x4 ek = __builtin_bit_cast(i32x4, lds_load16(kt, T::KEXPB + (kb * 16 + 4 * g) * 4));
          s[qb][kb] = score_block_f32<T>(ks, qs[qb], ek, kFoldEq ? 0 : eq[qb] - 47);
        }
        if (!steady && key0 + KT > N) {
#pragma unroll
          for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (key0 + kb * 16 + 4 * g + r >= N) s[qb][kb][r] = -INFINITY;
        }
        softmax_block_f32<T>(s[qb], p[qb], m2[qb], l_run[qb], acc[qb], c2q[qb]);
        // The next block reads the K slices from LDS again: without this the
        // compiler keeps every 16-key block's slices in registers from the
        // first block to the second, and the tile spills.
        if (qb + 1 < QB) asm volatile("" ::: "memory");
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KT / 16; ++kb) {
        i32x4 ks[D / 64][T::NSL];
#pragma unroll
        for (int h = 0; h < D / 64; ++h)
#pragma unroll
          for (int a2 = 0; a2 < T::NSL; ++a2)
            ks[h][a2] = __builtin_bit_cast(
                i32x4, lds_load16(kt, a2 * T::KSPLANEB + (kb * 16 + i16) * T::KSROW + (((4 * h + g) ^ kswz<D>(i16)) << 4)));
        const i32x4 ek = __builtin_bit_cast(i32x4, lds_load16(kt, T::KEXPB + (kb * 16 + 4 * g) * 4));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = score_block_f32<T>(ks, qs[qb], ek, kFoldEq ? 0 : eq[qb] - 47);
      }
      if (!steady && key0 + KT > N) {
#pragma unroll
        for (int kb = 0; kb < KT / 16; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = key0 + kb * 16 + 4 * g + r;
            if (key >= N)
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) softmax_block_f32<T>(s[qb], p[qb], m2[qb], l_run[qb], acc[qb], c2q[qb]);
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

    if constexpr (PACKED) {
      // the tile's key statistics, then the wait for this wave's copies of
      // the next tile
      const char* st = kt + T::KTILEB;
      kmax_a = fmaxf(kmax_a, reinterpret_cast<const float*>(st)[lane % T::CH]);
      kmax_e = max(kmax_e, reinterpret_cast<const int*>(st)[T::CH]);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (kSkew) {
      if (!late && (steady || j + 1 < ntiles)) stage_store(buf ^ 1);
      // LDS traffic only: the late waves' requests for tile j + 2 stay in flight
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (steady || j + 1 < ntiles) stage_store(buf ^ 1);
      __syncthreads();
    }
  };
  int j = 0;
  // A trip of two steady tiles requests tiles up to j + 2 (j + 3 for the late
  // waves of the skewed order) and needs them whole.
  for (; j + (kSkew ? 4 : 3) < ntiles; j += 2) {
    tile_step(j, std::integral_constant<int, 0>{}, std::true_type{});
    tile_step(j + 1, std::integral_constant<int, 1>{}, std::true_type{});
  }
  for (; j < ntiles; ++j) tile_step(j, 0, std::false_type{});


  // The lane and the wave's first query row, recomputed after the key loop
  // from an opaque copy of the thread index: nothing the epilogue needs is
  // kept (or spilled) across the loop.
  int tid_after = tid;
  asm volatile("" : "+v"(tid_after));
  const int lane_after = tid_after & 63;
  const int wave_after = uniform_sgpr(tid_after >> 6);
  const int qrow0_after = qt * T::BR + wave_after * T::WQ;

  // ---- exactness check.  The workgroup's largest key exponent, and a bound
  // on its largest key L1 norm (the sum over the column chunks of each
  // chunk's largest L1 norm, over every row staged by any thread), go through
  // LDS; each wave bounds the error of its int8-slice scores with them and its
  // own query statistics,
  //   |ds| <= |scale| (2^-35 (2^e_k A_q + 2^e_q A_k) + d 2^-40 2^(e_q + e_k)),
  // A = sum_c |x_c| of the row (the 2^-35 terms are the slicing residuals
  // |r| <= 2^(e-35) against the other row's entries, the last the dropped
  // slice products, a + b >= 6, below 3.02 d 2^-42 2^(e_q + e_k), with room
  // for the fp64 combination and the residual products), here with the
  // largest e and A of either side.  A wave whose bound exceeds
  // kExactScoreBound recomputes its rows exactly.
  {
    // lanes l, l + CH, ... of a wave share a column chunk
#pragma unroll
    for (int m = 1; m < 64; m *= 2) {
      kmax_e = max(kmax_e, __shfl_xor(kmax_e, m));
      if (m >= T::CH) kmax_a = fmaxf(kmax_a, __shfl_xor(kmax_a, m));
    }
    int* kst = reinterpret_cast<int*>(smem + (PACKED ? T::P_MISCB : T::MISCB));
    if (lane_after < T::CH) kst[wave_after * T::CH + lane_after] = __float_as_int(kmax_a);
    if (lane_after == 0) kst[T::NW * T::CH + wave_after] = kmax_e;
    lds_barrier_f32();
    float ak = 0.0f;
#pragma unroll
    for (int c = 0; c < T::CH; ++c) {
      float m = 0.0f;
#pragma unroll
      for (int w = 0; w < T::NW; ++w) m = fmaxf(m, __int_as_float(kst[w * T::CH + c]));
      ak += m;
    }
    kmax_a = ak;
#pragma unroll
    for (int w = 0; w < T::NW; ++w) kmax_e = max(kmax_e, kst[T::NW * T::CH + w]);
    const double abs_scale = c2 * kLn2;
    const double bq = wave_b > 0.0f ? static_cast<double>(wave_b) : 0.0;
    const double bk = __builtin_amdgcn_ldexp(1.0, kmax_e);
    const double bound = abs_scale * (__builtin_amdgcn_ldexp(bk * wave_a + bq * kmax_a, -35) +
                                      __builtin_amdgcn_ldexp(bq * bk, -40) * D);
    if (bound > kExactScoreBound) {
      exact_rows_impl<D, QB>(Qh, Kh, Vh, Oh, lse_h, N, qrow0_after, c2, qmul, lane_after);
      return;
    }
  }

  // ---- epilogue.  acc[qb][n][r] is O[q][16n + 4g + r].
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const double l_tot = add_xor<32>(add_xor<16>(l_run[qb]));
    const float inv = static_cast<float>(1.0 / l_tot);
    const int row = qrow0_after + qb * 16 + (lane_after & 15);
    if (row < N) {
      float* orow = Oh + row * D + 4 * (lane_after >> 4);
#pragma unroll
      for (int n = 0; n < D / 16; ++n) *reinterpret_cast<f32x4*>(orow + 16 * n) = acc[qb][n] * inv;
      if (lane_after < 16) lse_h[row] = static_cast<float>((m2[qb] + log2(l_tot)) * kLn2);
    }
  }
}

}  // namespace hfa
