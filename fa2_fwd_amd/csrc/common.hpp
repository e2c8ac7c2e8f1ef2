// Shared device helpers for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) void lds_void;

constexpr double kLn2 = 0.69314718055994530942;

// Thread and workgroup indices read through the compiler builtins.  These
// kernels are built without IEEE mode (-mno-amdgpu-ieee), and the runtime's
// threadIdx/blockIdx helpers, built with it, are then not inlined: each read
// becomes a call, and the workgroup index comes back in a vector register, so
// the compiler no longer knows that it is uniform.
__device__ __forceinline__ int thread_id() { return static_cast<int>(__builtin_amdgcn_workitem_id_x()); }
__device__ __forceinline__ int group_id() { return static_cast<int>(__builtin_amdgcn_workgroup_id_x()); }

// Workgroups are handed out round-robin over the 8 XCDs (wg % 8 selects the
// XCD).  Remap the hardware id so that each XCD receives one contiguous range
// of logical tiles: tiles of one (batch, head) then share that XCD's L2 for
// their common K/V stream.  A bijection on [0, total).
__device__ __forceinline__ int xcd_remap(int wg, int total) {
  constexpr int kXcd = 8;
  const int per = total / kXcd, rem = total % kXcd;
  const int xcd = wg % kXcd, local = wg / kXcd;
  return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// A wave-uniform int moved to a scalar register.  The empty asm makes the
// value opaque, so the compiler cannot drop the readfirstlane by proving the
// operand uniform (after which everything derived from it would stay in
// vector registers); the readfirstlane itself is the compiler's, placed with
// the wait state that gfx950 needs between a VALU write of the source and the
// read (a hand-written one in inline asm would get none).
__device__ __forceinline__ int uniform_sgpr(int x) {
  asm volatile("" : "+v"(x));
  return __builtin_amdgcn_readfirstlane(x);
}

// 2^x on the hardware exp unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Exchange with the lane 32 apart (v_permlane32_swap): returns {own, partner}
// in an order that depends on the half, so use it only in symmetric ops.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One 16-byte-per-lane HBM -> LDS copy (global_load_lds_dwordx4): lane l
// reads base + voff(l) and writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// base and lds must be wave-uniform.  Issued through inline assembly so that
// the compiler does not make every later LDS read wait for it; completion is
// ordered explicitly with vmcnt_wait and the workgroup barriers.
#ifndef HFA_DMA_ASM
#define HFA_DMA_ASM 1
#endif
__device__ __forceinline__ void dma16(const char* base, int voff, char* lds) {
#if HFA_DMA_ASM
  // readfirstlane returns int: every half goes through uint32_t before it is
  // widened, so the low half is never sign-extended into the high word.
  const uint32_t lds_addr = static_cast<uint32_t>(
      __builtin_amdgcn_readfirstlane(static_cast<int>(reinterpret_cast<uintptr_t>((lds_void*)lds))));
  const uint64_t b = reinterpret_cast<uintptr_t>(base);
  const uint32_t b_lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))));
  const uint32_t b_hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32))));
  const uint64_t sbase = (static_cast<uint64_t>(b_hi) << 32) | static_cast<uint64_t>(b_lo);
  // M0 carries the LDS destination; its previous value is restored, so the
  // statement leaves every register the compiler may rely on unchanged.  A
  // scalar write of M0 needs one wait state before a load to LDS reads it;
  // the compiler cannot see into the statement, so the s_nop is written here.
  // (The scalar operands come from readfirstlane, and a VALU write of an SGPR
  // needs five wait states before a vector-memory read of it; the compiler
  // hoists them out of the key loop, far from any use.)
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "s"(lds_addr), "v"(voff), "s"(sbase)
      : "memory");
#else
  __builtin_amdgcn_global_load_lds(base + voff, (lds_void*)lds, 16, 0, 0);
#endif
}

// The same copy with operands the caller keeps in scalar registers: a
// wave-uniform global base and the LDS destination as a uniform LDS address
// (no generic-pointer conversion and no readfirstlane here).  The caller
// forms both with scalar arithmetic, so no vector instruction writes them.
__device__ __forceinline__ void dma16_to(const char* base, int voff, uint32_t lds_addr) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void vmcnt_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_store16(char* lds, int byte_off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + byte_off) = v;
}
__device__ __forceinline__ u32x4 lds_load16(const char* lds, int byte_off) {
  return *reinterpret_cast<const u32x4*>(lds + byte_off);
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane j supplies the address of 4 consecutive 16-bit elements; lane i
// receives element (i % 4) of the vectors read by lanes i/4, 4 + i/4, 8 + i/4
// and 12 + i/4.  With lane j pointing at row j/4, columns 4*(j%4)..+3 of a
// 4 x 16 block, lane i therefore gets column i of the 4 rows.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* lds, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(lds) + byte_off));
}

}  // namespace hfa
