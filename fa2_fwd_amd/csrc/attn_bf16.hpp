// bf16 attention forward for gfx950: O = softmax(Q K^T * scale) V and its
// log-sum-exp, computed tile by tile with the online normalisation identity
// (neuralmasteryai "Hardware Acceleration & Custom Kernels", section 2,
// steps 1-2): each wave owns 32 query rows held in registers, K/V tiles
// stream through rings of LDS buffers, and the running max, running
// denominator and running output sums are rescaled as key tiles arrive, so
// no score ever reaches HBM.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//
//  * Scores are formed transposed, S^T = K Q^T: the A operand is 32 key rows
//    of K (from LDS), the B operand is the wave's 32 query rows (registers).
//    In the 32x32 accumulator each lane then owns ONE query (lane % 32) and 16
//    of the 32 keys, so the row max and row sum are lane-local plus one
//    exchange with the lane 32 apart (v_permlane32_swap).
//  * The keys fed into the A operand are permuted (row i of the MFMA reads
//    key pi(i)) so that accumulator registers r = 0..7 / 8..15 of lane half h
//    hold the 8 consecutive keys 16*c + 8h + (r % 8) of chunk c.  That is
//    exactly the B-operand layout of the next product, so P never leaves
//    registers.
//  * O^T = V^T P^T: the A operand is V^T (8 consecutive keys of one head-dim
//    column per lane), read from the row-major V tile with the gfx950
//    transposing LDS load (ds_read_b64_tr_b16, 4 keys x 16 columns per 16
//    lanes); the B operand is P rounded to bf16.  Each lane's accumulator
//    again belongs to its own query, so the per-row rescale is lane-local.
//
// Schedule ("ping-pong").  The 8 waves form two groups, one wave of each per
// SIMD, offset by half a tile.  A wave alternates an MFMA phase (S_j = K_j
// Q^T together with the previous tile's P_{j-1} V_{j-1}: software pipelined)
// and a VALU phase (softmax of S_j, rescale, P_j).  Workgroup barriers
// separate the phases, and since the second group enters the loop one
// barrier later, in every interval one wave of each SIMD issues matrix-core
// work while the other runs its softmax on the vector unit.
//
// LDS tiles: K_t and V_t live in buffer t % NBUF of two rings filled
// straight from HBM.  In its VALU phase j, group 0 requests K_{j+3} and
// group 1 requests V_{j+3}; at the end of its next MFMA phase each waits for
// the tile that is read first after the following barrier (group 0: K_{j+1}
// at the end of MFMA phase j, read ahead by both groups' VALU phases;
// group 1: V_j, read by group 0's next MFMA phase).  Across the barrier
// intervals a buffer is refilled only after both groups finished reading its
// previous tile (tests/test_schedule_model.py checks both properties).
//
// Loop shape.  While more than NBUF + AHEAD tiles remain, the loop runs
// "steady" trips of NBUF tiles, one per ring slot, with the slot a
// compile-time constant (LDS offsets fold into instruction immediates) and
// no bounds, ragged-tile or masking checks; each group runs its own copy of
// these trips, so its HBM wait count is an immediate too.  The last tiles
// go through a general step that checks everything at run time.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace hfa {

#ifndef HFA_NBUF
#define HFA_NBUF 4
#endif

template <int D_, int QB_, int NW_, int KT_ = 64>
struct Bf16Tile {
  static constexpr int D = D_;        // head dim (64 or 128)
  static constexpr int QB = QB_;      // 32-query blocks per wave
  static constexpr int NW = NW_;      // waves per workgroup (two ping-pong groups)
  static constexpr int KT = KT_;      // keys per K/V tile (64 or 128)
  static constexpr int WQ = 32 * QB;  // queries per wave
  static constexpr int BR = WQ * NW;  // queries per workgroup (row-tile height)
  static constexpr int NT = 64 * NW;  // threads per workgroup
  static constexpr int ROWB = D * 2;  // bytes per K or V row in LDS (XOR-swizzled, unpadded)
  static constexpr int TILEB = KT * ROWB;
  static constexpr int CH = D / 8;             // 16-byte chunks per row
  static constexpr int NBUF = HFA_NBUF;        // LDS ring depth, tiles per tensor
  static constexpr int AHEAD = NBUF - 1;       // tiles of each stream requested ahead
  static constexpr int LD = TILEB / (4 * 64 * 16);  // 16-byte loads per lane per tile (one group of 4 waves)
  static constexpr int LDS_BYTES = 2 * NBUF * TILEB;  // K ring and V ring
  static_assert(LD >= 1 && TILEB % (4 * 64 * 16) == 0, "a tile must split into whole load instructions");
  static_assert(CH == 8 || CH == 16, "swizzles are defined for d = 64 and d = 128");
  static_assert(NW == 8, "the ping-pong schedule pairs two waves per SIMD");
};

// LDS serves 16 lanes x 16 bytes per clock (64 banks); a 16-byte access
// occupies one of 16 "bank groups" given by (byte address / 16) mod 16.  The
// swizzles below XOR the 16-byte chunk index within a row (CH chunks per row)
// so that every group of lanes served together hits 16 different groups:
//
// K rows: lanes 0..15 (and 16..31) of an S MFMA read 16 different rows at the
// same logical chunk; writes put 16 consecutive chunks of one row (CH = 16) or
// of two rows (CH = 8) on 16 lanes.
template <int CH>
__device__ __forceinline__ int k_swz(int row) {
  return CH == 16 ? (row & 15) : ((row >> 1) & 7);
}
// V rows: one transposing read covers 4 consecutive rows x 4 chunks per 32
// lanes; the XOR moves whole 4-chunk blocks so the four rows land apart.
template <int CH>
__device__ __forceinline__ int v_swz(int row) {
  return CH == 16 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

#ifndef HFA_SCHED_GROUPS
#define HFA_SCHED_GROUPS 1
#endif
#ifndef HFA_PF
#define HFA_PF 2
#endif
#ifndef HFA_LAZY_MAX
#define HFA_LAZY_MAX 1
#endif
#ifndef HFA_PIN_SOFTMAX
#define HFA_PIN_SOFTMAX 1
#endif

// Largest growth of the running max (log2 units) absorbed without rescaling.
constexpr float kRescaleLog2 = 8.0f;
// Largest lane sum of one tile's weights accepted without forming the max.
constexpr float kSumLimit = 65536.0f;

#ifndef HFA_RING_UNROLL
#define HFA_RING_UNROLL 1
#endif

#ifndef HFA_MFMA_PRIO
#define HFA_MFMA_PRIO 1
#endif

// Wave issue priority (s_setprio).  The SIMD arbiter otherwise favours the
// older of its two waves, so the softmax of group 0 would take issue slots
// from the MFMA phase of group 1; the wave in its MFMA phase runs at the
// raised priority instead, and the matrix core is fed first.
__device__ __forceinline__ void wave_prio(bool mfma_phase) {
  __builtin_amdgcn_sched_barrier(0);
  if (mfma_phase)
    __builtin_amdgcn_s_setprio(HFA_MFMA_PRIO);
  else
    __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup barrier that waits only for this wave's LDS operations: global
// loads issued before it stay in flight.  The memory clobber keeps the
// compiler from moving any memory access across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);  // no instruction (MFMAs included) crosses the barrier
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Key split.  With SPLIT, the keys of each (batch, head) are cut into
// `nsplit` ranges of `split_tiles` key tiles; workgroup (bh, split, q-tile)
// runs the same loop over its range only and writes, instead of O and LSE,
// its partial result: the range's normalised output O_s = acc / l (fp32) to
// part_o[split][bh][row][:] and its log-sum-exp in log2 units, m2 + log2 l,
// to part_lse[split][bh][row].  attn_merge_bf16_kernel combines the ranges
// by the same identity as the running update.
struct SplitArgs {
  int nsplit;       // key ranges per head (1: no split)
  int split_tiles;  // key tiles per range
  float* part_o;    // [nsplit][BH][N][D]
  float* part_lse;  // [nsplit][BH][N]
};

template <class T, bool SPLIT>
__global__ __launch_bounds__(T::NT) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int N, int n_qt, int total_wg, float c2,
    int q_mode, SplitArgs sa) {
  constexpr int D = T::D, QB = T::QB, KT = T::KT, ROWB = T::ROWB, TILEB = T::TILEB;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const kbuf = smem;                    // K ring: NBUF tile buffers
  char* const vbuf = smem + T::NBUF * TILEB;  // V ring: NBUF tile buffers

  const int tid = thread_id();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const int grp = wave >> 2;  // ping-pong group; waves w and w + 4 share a SIMD
  const int i32 = lane & 31, hh = lane >> 5;

  // Logical tile order: q-tile fastest, then the key range, then the head,
  // so that the workgroups sharing a head's key range are neighbours (and,
  // after xcd_remap, on one XCD).
  const int tile = xcd_remap(group_id(), total_wg);
  const int grp_id = tile / n_qt, qt = tile - grp_id * n_qt;
  const int sp = SPLIT ? grp_id % sa.nsplit : 0;
  const int bh = SPLIT ? grp_id / sa.nsplit : grp_id;
  const size_t head = static_cast<size_t>(bh) * static_cast<size_t>(N) * D;
  // This workgroup's keys: [key_begin, key_begin + nkeys).
  const int key_begin = SPLIT ? sp * sa.split_tiles * KT : 0;
  const int nkeys = SPLIT ? min(N - key_begin, sa.split_tiles * KT) : N;
  const __bf16* Qh = Q + head;
  const __bf16* Kh = K + head + static_cast<size_t>(key_begin) * D;
  const __bf16* Vh = V + head + static_cast<size_t>(key_begin) * D;
  __bf16* Oh = O + head;
  const int qrow0 = qt * T::BR + wave * T::WQ;

  // ---- Q fragments (B operand of S^T = K Q^T): Q[row = i32][d = 16t + 8hh .. +7].
  // q_mode folds the sign of the scale into Q (+1 keep, -1 negate, 0 zero) so
  // that the softmax below always works with a positive log2-domain scale c2.
  // Rows past the end load row N - 1 and are zeroed: every lane issues the
  // same unconditional loads back to back (a load under a lane mask made the
  // compiler wait for it on the spot, one HBM round trip before the K/V
  // requests below).
  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + i32;
    const __bf16* qrow = Qh + static_cast<size_t>(min(row, N - 1)) * D + 8 * hh;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[qb][t] = *reinterpret_cast<const u32x4*>(qrow + 16 * t);
    const bool zero = row >= N || q_mode == 0;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      u32x4 x = qf[qb][t];
      if (q_mode < 0) x ^= 0x80008000u;
      if (zero) x = u32x4{0u, 0u, 0u, 0u};
      qf[qb][t] = x;
    }
  }

  // ---- per-lane LDS geometry (invariant over the key loop)
  // S MFMA row i32 reads key pi(i32) of each 32-key block.
  const int a8 = i32 >> 3, e4 = (i32 >> 2) & 1, b4 = i32 & 3;
  const int krow = 16 * (a8 >> 1) + 8 * e4 + 4 * (a8 & 1) + b4;
  const int kswz = k_swz<T::CH>(krow);
  // Transposing V read: in each 16-lane group, lane l16 reads row 4u + l16/4 of
  // the group's 4 rows at columns 16*g16 + 4*(l16 % 4) .. +3 of the 32-column block.
  const int l16 = lane & 15, g16 = (lane >> 4) & 1;
  const int vrow = 8 * hh + (l16 >> 2);
  const int vswz = v_swz<T::CH>(vrow);
  const int vch = 2 * g16 + ((l16 & 3) >> 1);
  const int vin = (l16 & 1) * 8;

  f32x16 acc[QB][D / 32];
  float m2[QB], l_run[QB];  // running max (log2 units: max score * c2) and denominator
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m2[qb] = -INFINITY;
    l_run[qb] = 0.0f;
#pragma unroll
    for (int n = 0; n < D / 32; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][n][r] = 0.0f;
  }

  const int ntiles = (nkeys + KT - 1) / KT;

  // ---- K/V streaming: HBM -> LDS directly (global_load_lds_dwordx4), no
  // registers.  Group 0 streams the K tiles, group 1 the V tiles, each into a
  // ring of NBUF tile buffers (tile t in buffer t % NBUF), AHEAD tiles before
  // first use.  One load instruction writes 64 consecutive 16-byte LDS chunks
  // in lane order, so the XOR swizzle is realised by choosing each lane's
  // source chunk.  Keys past the end are clamped to the last row: their
  // scores are masked to -inf and their weights are exactly zero.
  const int wig = wave & 3;  // wave within its group
  const __bf16* const stream_src = grp == 0 ? Kh : Vh;
  char* const stream_ring = grp == 0 ? kbuf : vbuf;
  // Per-lane source offsets (bytes) of this lane's LD chunks within a tile:
  // the same for every tile except a ragged last one.
  int dma_off[T::LD];
#pragma unroll
  for (int u = 0; u < T::LD; ++u) {
    const int pos = (wig * T::LD + u) * 64 + lane;  // 16-byte chunk position within the tile
    const int row = pos / T::CH, phys = pos % T::CH;
    const int ch = phys ^ (grp == 0 ? k_swz<T::CH>(row) : v_swz<T::CH>(row));
    dma_off[u] = (row * D + ch * 8) * 2;
  }
  // Ring slot of tile t: t % NBUF, or a compile-time constant equal to it
  // (the unrolled loop below passes one, so slot addresses fold into the
  // immediate offsets of the LDS instructions).
  auto slot_of = [&](int t, auto slot) __attribute__((always_inline)) -> int {
    if constexpr (std::is_integral_v<decltype(slot)>)
      return t % T::NBUF;
    else
      return decltype(slot)::value;
  };
  // steady: the caller guarantees t < ntiles - 1 (a full tile that exists).
  auto issue_tile = [&](int t, auto slot, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool steady = decltype(steady_tag)::value;
    if (!steady && t >= ntiles) return;
    char* dst = stream_ring + slot_of(t, slot) * TILEB;
    const char* tile_src = reinterpret_cast<const char*>(stream_src + static_cast<size_t>(t) * KT * D);
    if (steady || (t + 1) * KT <= nkeys) {
#pragma unroll
      for (int u = 0; u < T::LD; ++u) dma16(tile_src, dma_off[u], dst + (wig * T::LD + u) * 1024);
    } else {  // ragged last tile: rows past the end re-read the last row
      const int last = nkeys - 1 - t * KT;
#pragma unroll
      for (int u = 0; u < T::LD; ++u) {
        const int row = ((wig * T::LD + u) * 64 + lane) / T::CH;
        const int off = dma_off[u] - (row > last ? (row - last) * D * 2 : 0);
        dma16(tile_src, off, dst + (wig * T::LD + u) * 1024);
      }
    }
  };

  // ---- matrix-core work of one interval: S_j = K_j Q^T and, when with_pv,
  // acc += V_{j-1}^T P_{j-1}^T.  The 2 x (D/16) score MFMAs and the
  // (KT/16) x (D/32) output MFMAs are issued as one interleaved sequence of
  // steps (one of each per step, on independent accumulators), with each
  // step's LDS operands requested PF steps ahead, so neither the matrix-core
  // dependency latency nor the LDS latency is exposed.
  f32x16 s[QB][KT / 32];
  bf16x8 pf[QB][KT / 16];
  constexpr int SSTEPS = (KT / 32) * (D / 16);  // score MFMAs per tile (per query block)
  constexpr int VSTEPS = (KT / 16) * (D / 32);  // output MFMAs per tile (per query block)
  static_assert(SSTEPS == VSTEPS, "score and output products have the same MFMA count");
  constexpr int STEPS = SSTEPS;
  constexpr int PF = HFA_PF;  // prefetch distance in steps
  auto k_off = [&](int i) {  // step i: key block i % 2, d-step i / 2
    const int kb = i % (KT / 32), t = i / (KT / 32);
    return (kb * 32 + krow) * ROWB + (((2 * t + hh) ^ kswz) << 4);
  };
  // The lane-dependent part of each column block's V address, formed once:
  // the key chunk and the ring slot then only add constants.
  int vlane[D / 32];
#pragma unroll
  for (int n = 0; n < D / 32; ++n) vlane[n] = vrow * ROWB + (((4 * n + vch) ^ vswz) << 4) + vin;
  auto v_off = [&](int i) {  // step i: column block i % (D/32), key chunk i / (D/32)
    const int n = i % (D / 32), c = i / (D / 32);
    return vlane[n] + 16 * c * ROWB;
  };
  // The MFMA phase is a sequence of operations, each one MFMA with its LDS
  // operand: the SSTEPS score MFMAs first (so the scores are complete, and
  // the softmax can start, while the output MFMAs still run), then the
  // output MFMAs.  Operands are requested PF operations ahead; the first PF
  // of them are read in the VALU phase before, across the barrier.
  constexpr int NOPS = SSTEPS + VSTEPS;
  auto op_is_score = [&](int i, bool with_pv) { return !with_pv || i < SSTEPS; };
  auto op_step = [&](int i, bool with_pv) {  // index of the score or output step of operation i
    return (!with_pv || i < SSTEPS) ? i : i - SSTEPS;
  };
  // The operands read before the barrier (the first PF operations) are K
  // operands only: V tiles are published one interval later (see the waits).
  static_assert(PF <= SSTEPS, "only score operands are read ahead of the MFMA phase");
  u32x4 opnd[PF + 1];
  auto load_op = [&](int i, bool with_pv, const char* kt, const char* vt) __attribute__((always_inline)) -> u32x4 {
    const int st = op_step(i, with_pv);
    if (op_is_score(i, with_pv)) return lds_load16(kt, k_off(st));
    const s16x4 lo = lds_read_tr16(vt, v_off(st));
    const s16x4 hi = lds_read_tr16(vt, v_off(st) + 4 * ROWB);
    return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto prefetch_operands = [&](int j, auto with_pv_tag, auto slot) __attribute__((always_inline)) {  // first PF operations of MFMA phase j
    constexpr bool with_pv = decltype(with_pv_tag)::value;
    const int sj = slot_of(j, slot);
    const char* kt = kbuf + sj * TILEB;
    const char* vt = vbuf + ((sj + T::NBUF - 1) % T::NBUF) * TILEB;
#pragma unroll
    for (int i = 0; i < PF; ++i) opnd[i] = load_op(i, with_pv, kt, vt);
  };
  auto mfma_phase = [&](int j, auto with_pv_tag, auto prefetched_tag, auto slot) __attribute__((always_inline)) {
    constexpr bool with_pv = decltype(with_pv_tag)::value;
    constexpr bool prefetched = decltype(prefetched_tag)::value;
    constexpr int nops = with_pv ? NOPS : SSTEPS;
    const int sj = slot_of(j, slot);
    const char* kt = kbuf + sj * TILEB;
    const char* vt = vbuf + ((sj + T::NBUF - 1) % T::NBUF) * TILEB;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = 0.0f;
    if (!prefetched) prefetch_operands(j, with_pv_tag, slot);
#pragma unroll
    for (int i = 0; i < nops; ++i) {
      if (i + PF < nops) opnd[(i + PF) % (PF + 1)] = load_op(i + PF, with_pv, kt, vt);
      const int st = op_step(i, with_pv);
      const u32x4 a = opnd[i % (PF + 1)];
      if (op_is_score(i, with_pv)) {
        const int kb = st % (KT / 32), t = st / (KT / 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                              __builtin_bit_cast(bf16x8, qf[qb][t]), s[qb][kb], 0, 0, 0);
      } else {
        const int n = st % (D / 32), c = st / (D / 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[qb][c], acc[qb][n],
                                                               0, 0, 0);
      }
    }
#if HFA_SCHED_GROUPS
    // Pin the order: per operation the operand reads of a later one (1 read
    // for a score operand, 2 transposing reads for an output operand), then
    // this operation's MFMA.
    if constexpr (!with_pv) {
      if (!prefetched) __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
      for (int i = 0; i < nops; ++i) {
        if (i + PF < nops) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      }
    } else {
      if (!prefetched) __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);  // PF <= SSTEPS score operands
#pragma unroll
      for (int i = 0; i < SSTEPS - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      }
#pragma unroll
      for (int i = SSTEPS - PF; i < nops - PF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      }
#pragma unroll
      for (int i = nops - PF; i < nops; ++i) __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
    }
#endif
  };
  // final output product of the last tile, without scores
  auto mfma_pv_only = [&](int j) __attribute__((always_inline)) {
    const char* vt = vbuf + (j % T::NBUF) * TILEB;
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      const int n = i % (D / 32), c = i / (D / 32);
      const s16x4 lo = lds_read_tr16(vt, v_off(i));
      const s16x4 hi = lds_read_tr16(vt, v_off(i) + 4 * ROWB);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][c], acc[qb][n], 0, 0, 0);
    }
  };

  // ---- vector work of one interval: online softmax update of tile j.
  // The running max is kept in log2 units (m2 = max score * c2).  It only
  // moves when it would grow by more than kRescaleLog2 for some lane of the
  // wave: a stale max keeps every weight <= 2^kRescaleLog2, which the fp32
  // sums and the bf16 P represent with unchanged relative precision, and the
  // final division by the denominator removes it exactly.
  //
  // Only the first tile forms its row max up front.  Later tiles turn their
  // scores in place into x = s * c2 - m2 and exponentiate straight away; a
  // lane sum of the weights above kSumLimit implies a weight above
  // kSumLimit / (KT/2) = 2^11, a growth beyond kRescaleLog2, and only then is
  // the row max of x formed, the rescale applied and the weights redone (a
  // rare, wave-uniform branch).  Every weight stays <= kSumLimit either way.
  auto softmax = [&](int j, auto first_tag, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool first = decltype(first_tag)::value;
    constexpr bool steady = decltype(steady_tag)::value;  // tile j is not the last: no key past nkeys
    const int key0 = j * KT;
    if (!steady && key0 + KT > nkeys) {  // keys past the end of the range get score -inf (weight 0)
#pragma unroll
      for (int kb = 0; kb < KT / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
          if (key >= nkeys)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb][r] = -INFINITY;
        }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // The lane's KT/2 values of this tile, flattened; reductions run as
      // balanced trees so the vector pipe is not held up by one serial chain.
      constexpr int NS = KT / 2;
      auto xv = [&](int i) { return s[qb][i / 16][i % 16]; };
      auto xset = [&](int i, float v) { s[qb][i / 16][i % 16] = v; };
      auto row_max = [&]() {  // max over the row (this lane and the lane 32 apart)
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
      // weights p = 2^x rounded to bf16 into P, and their lane sum
      auto weights = [&]() {
        float pv[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) pv[i] = exp2_hw(xv(i));
#pragma unroll
        for (int c = 0; c < KT / 16; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[qb][c][e] = static_cast<__bf16>(pv[8 * c + e]);
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
      if constexpr (first || !HFA_LAZY_MAX) {
        if constexpr (first) {
          // m2 is -inf before the first tile: start it at this tile's row max
          // (finite, key 0 is in the tile), so every x <= 0.
#pragma unroll
          for (int i = 0; i < NS; ++i) xset(i, xv(i) * c2);
          m2[qb] = row_max();
#pragma unroll
          for (int i = 0; i < NS; ++i) xset(i, xv(i) - m2[qb]);
        } else {
#pragma unroll
          for (int i = 0; i < NS; ++i) xset(i, fmaf(xv(i), c2, -m2[qb]));
          const float mx = row_max();
          const bool grow = mx > kRescaleLog2;
          if (__any(grow)) {
            const float m_new = grow ? m2[qb] + mx : m2[qb];
            const float d = m_new - m2[qb];
            const float alpha = exp2_hw(-d);
            l_run[qb] *= alpha;
#pragma unroll
            for (int n = 0; n < D / 32; ++n) acc[qb][n] *= alpha;
            m2[qb] = m_new;
#pragma unroll
            for (int i = 0; i < NS; ++i) xset(i, xv(i) - d);
          }
        }
        tsum = weights();
      } else {
#pragma unroll
        for (int i = 0; i < NS; ++i) xset(i, fmaf(xv(i), c2, -m2[qb]));
        tsum = weights();  // m2 is finite after the first tile: no x is NaN
        if (__any(!(tsum <= kSumLimit))) {
          const float mx = row_max();  // growth of the row max, log2 units
          const bool grow = mx > kRescaleLog2;
          const float m_new = grow ? m2[qb] + mx : m2[qb];
          const float d = m_new - m2[qb];
          const float alpha = exp2_hw(-d);
          l_run[qb] *= alpha;
#pragma unroll
          for (int n = 0; n < D / 32; ++n) acc[qb][n] *= alpha;
          m2[qb] = m_new;
#pragma unroll
          for (int i = 0; i < NS; ++i) xset(i, xv(i) - d);
          tsum = weights();
        }
      }
      l_run[qb] += tsum;
#if HFA_PIN_SOFTMAX
      // An empty statement that consumes P and the denominator: the compiler
      // would otherwise sink the exponentials below the wait for the next
      // K/V tile that follows, exposing HBM latency in this phase.
#pragma unroll
      for (int c = 0; c < KT / 16; ++c) asm volatile("" ::"v"(__builtin_bit_cast(u32x4, pf[qb][c])));
      asm volatile("" ::"v"(l_run[qb]));
#endif
    }
  };

  // Wait until this group's request for tile t is complete.  Requests go
  // out in tile order and only for tiles < ntiles, so the number that may
  // still be in flight is LD times the number of tiles requested after t.
  auto wait_tile = [&](int t, int newest) __attribute__((always_inline)) {
    const int after = min(newest, ntiles - 1) - t;
    static_assert(T::AHEAD <= 4, "wait counts are spelled out up to three newer tiles");
    if (after <= 0)
      vmcnt_wait<0>();
    else if (after == 1)
      vmcnt_wait<T::LD>();
    else if (after == 2 || T::AHEAD < 4)
      vmcnt_wait<2 * T::LD>();
    else
      vmcnt_wait<3 * T::LD>();
  };

  // ---- prologue: the first AHEAD tiles of each stream; K_0 (group 0) must
  // be complete before the first barrier.
#pragma unroll
  for (int t = 0; t < T::AHEAD; ++t) issue_tile(t, 0, std::false_type{});
  if (grp == 0) wait_tile(0, T::AHEAD - 1);
  lds_barrier();
  if (grp == 1) lds_barrier();  // group 1 runs half a tile behind

  // One tile: the MFMA phase (scores of tile j, P V of tile j - 1) and the
  // wait that completes the tile read first after its closing barrier:
  // group 0 needs K_{j+1} (operands read ahead in both groups' next VALU
  // phases), group 1 needs V_j (read by group 0's next MFMA phase).  Each
  // was requested AHEAD tiles earlier, three to four intervals before.
  // Then the VALU phase: the first LDS operands of the next MFMA phase, the
  // HBM request for tile j + AHEAD of this group's stream and the softmax of
  // tile j.  Tile 0 is peeled off so that the accumulator flows straight
  // through the loop body.
  // steady: tiles j - 1 + AHEAD and j + AHEAD exist and are not the last, so
  // the wait counts are fixed and no request needs a bounds or ragged check.
  auto close_mfma_phase = [&](int j, auto steady_tag, auto grp_tag) __attribute__((always_inline)) {
    constexpr bool steady = decltype(steady_tag)::value;
    constexpr int g = decltype(grp_tag)::value;  // -1: read the group at run time
    if constexpr (steady && g == 0) {
      vmcnt_wait<(T::AHEAD - 2) * T::LD>();
    } else if constexpr (steady && g == 1) {
      vmcnt_wait<(T::AHEAD - 1) * T::LD>();
    } else if constexpr (steady) {
      if (grp == 0)
        vmcnt_wait<(T::AHEAD - 2) * T::LD>();
      else
        vmcnt_wait<(T::AHEAD - 1) * T::LD>();
    } else {
      if (grp == 0)
        wait_tile(j + 1, j - 1 + T::AHEAD);
      else
        wait_tile(j, j - 1 + T::AHEAD);
    }
    lds_barrier();
  };
  auto next_slot = [&](auto slot, auto step) __attribute__((always_inline)) {
    if constexpr (std::is_integral_v<decltype(slot)>)
      return slot;
    else
      return std::integral_constant<int, (decltype(slot)::value + decltype(step)::value) % T::NBUF>{};
  };
  auto valu_phase = [&](int j, auto first_tag, auto slot, auto steady_tag) __attribute__((always_inline)) {
    constexpr bool steady = decltype(steady_tag)::value;
    if (steady || j + 1 < ntiles)
      prefetch_operands(j + 1, std::true_type{}, next_slot(slot, std::integral_constant<int, 1>{}));
    issue_tile(j + T::AHEAD, next_slot(slot, std::integral_constant<int, T::AHEAD>{}), steady_tag);
    softmax(j, first_tag, steady_tag);
    lds_barrier();
  };
  auto step = [&](int j, auto slot, auto steady_tag, auto grp_tag) __attribute__((always_inline)) {
    wave_prio(true);
    mfma_phase(j, std::true_type{}, std::true_type{}, slot);
    wave_prio(false);
    close_mfma_phase(j, steady_tag, grp_tag);
    valu_phase(j, std::false_type{}, slot, steady_tag);
  };
  using RtGrp = std::integral_constant<int, -1>;
  wave_prio(true);
  mfma_phase(0, std::false_type{}, std::false_type{}, 0);
  wave_prio(false);
  close_mfma_phase(0, std::false_type{}, RtGrp{});
  valu_phase(0, std::true_type{}, 0, std::false_type{});
  int j = 1;
#if HFA_RING_UNROLL
  // NBUF tiles per trip with the ring slot of each known at compile time
  // (j % NBUF == 1 at the top of a trip).  A trip runs only while every step
  // in it is steady: its last step, j + 3, requests tile j + 3 + AHEAD, which
  // must be below ntiles - 1.
  static_assert(T::NBUF == 4 && T::AHEAD == 3, "the unrolled trip is written for a 4-slot ring");
  auto trips = [&](auto grp_tag) __attribute__((always_inline)) {
    for (; j + 3 + T::AHEAD < ntiles - 1; j += 4) {
      step(j, std::integral_constant<int, 1>{}, std::true_type{}, grp_tag);
      step(j + 1, std::integral_constant<int, 2>{}, std::true_type{}, grp_tag);
      step(j + 2, std::integral_constant<int, 3>{}, std::true_type{}, grp_tag);
      step(j + 3, std::integral_constant<int, 0>{}, std::true_type{}, grp_tag);
    }
  };
  // One copy of the trips per group, so the group's wait count is an
  // immediate rather than a branch in every phase.
  if (grp == 0)
    trips(std::integral_constant<int, 0>{});
  else
    trips(std::integral_constant<int, 1>{});
#endif
  for (; j < ntiles; ++j) step(j, 0, std::false_type{}, RtGrp{});
  wave_prio(true);
  mfma_pv_only(ntiles - 1);
  wave_prio(false);
  if (grp == 0) lds_barrier();  // both groups execute the same number of barriers

  // ---- epilogue of a key range: its normalised output and log-sum-exp
  if constexpr (SPLIT) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = add_xor32(l_run[qb]);
      const float inv = 1.0f / l_tot;
      const int row = qrow0 + qb * 32 + i32;
      if (row < N) {
        const size_t prow = (static_cast<size_t>(sp) * (total_wg / (n_qt * sa.nsplit)) + bh) * N + row;
        float* orow = sa.part_o + prow * D;
#pragma unroll
        for (int n = 0; n < D / 32; ++n)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            f32x4 o4;
#pragma unroll
            for (int b = 0; b < 4; ++b) o4[b] = acc[qb][n][4 * a + b] * inv;
            *reinterpret_cast<f32x4*>(orow + 32 * n + 8 * a + 4 * hh) = o4;
          }
        if (hh == 0) sa.part_lse[prow] = m2[qb] + log2f(l_tot);
      }
    }
    return;
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
        const double lse2 =
            static_cast<double>(m2[qb]) + log2(static_cast<double>(l_tot));
        LSE[static_cast<size_t>(bh) * N + row] = static_cast<float>(lse2 * kLn2);
      }
    }
  }
}

// Combines the key ranges of a split launch, one query row per group of
// D/8 threads (8 columns each): with lse_s = m2_s + log2 l_s of range s
// (log2 units), M = max_s lse_s and w_s = 2^(lse_s - M),
//     O = sum_s w_s O_s / sum_s w_s,    LSE = ln 2 (M + log2 sum_s w_s),
// the identity of the running update applied to whole ranges.  O is rounded
// to bf16 once; the log-sum-exp is combined in fp64.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_bf16_kernel(const float* __restrict__ part_o,
                                                              const float* __restrict__ part_lse,
                                                              __bf16* __restrict__ O, float* __restrict__ LSE,
                                                              int rows, int nsplit) {
  constexpr int TPR = D / 8;  // threads per row
  const int row = group_id() * (256 / TPR) + thread_id() / TPR;
  const int c0 = (thread_id() % TPR) * 8;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_lse[static_cast<size_t>(s) * rows + row]);
  float wsum = 0.0f;
  f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsplit; ++s) {
    const size_t pr = static_cast<size_t>(s) * rows + row;
    const float w = exp2_hw(part_lse[pr] - m);
    const f32x4* src = reinterpret_cast<const f32x4*>(part_o + pr * D + c0);
    a0 += w * src[0];
    a1 += w * src[1];
    wsum += w;
  }
  const float inv = 1.0f / wsum;
  bf16x8 o8;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o8[e] = static_cast<__bf16>(a0[e] * inv);
    o8[4 + e] = static_cast<__bf16>(a1[e] * inv);
  }
  *reinterpret_cast<bf16x8*>(O + static_cast<size_t>(row) * D + c0) = o8;
  if (c0 == 0) LSE[row] = static_cast<float>((static_cast<double>(m) + log2(static_cast<double>(wsum))) * kLn2);
}

}  // namespace hfa
