// C ABI of the attention forward in libhfa.so (declared in include/hfa.h):
// argument validation, device check, kernel dispatch and graph capture.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>

#include "hfa.h"
#include "attn_bf16.hpp"
#include "attn_bf16_solo.hpp"
#include "attn_f32.hpp"
#include "api_util.hpp"

// Scratch of the allocation-free key split (hfa_attn_fwd_split_noalloc): 64 MiB,
// one copy per GPU the library runs on, held until the process ends.
constexpr int64_t kScratchBytes = int64_t{64} << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

using namespace hfa;
using namespace hfa::api;

// Tile configurations, one per (dtype, head dim).  The macros exist so that
// a tile sweep can build variants with -D; the defaults are the tuned choice.
#ifndef HFA_BF16_D128_TILE
#define HFA_BF16_D128_TILE 1, 8
#endif
#ifndef HFA_BF16_D64_TILE
#define HFA_BF16_D64_TILE 1, 8
#endif
// bf16, d = 64, unsplit calls with at least kBf16LongKeys keys: 128-key tiles
// (twice the work per barrier interval; measured +2 to +5 % from N = 4096 on,
// -3 % at N = 1024).
#ifndef HFA_BF16_D64_LONG_TILE
#define HFA_BF16_D64_LONG_TILE 1, 8, 128
#endif
// fp32, d = 64: the largest of three tilings whose grid still gives every CU
// a workgroup -- 256 rows (two 16-query blocks per wave, 8 waves), 128 rows
// (one block per wave, 8 waves) -- and 64-row workgroups (4 waves) for shapes
// too small to fill the CUs even so, where more workgroups mean more of the
// chip at work.
#ifndef HFA_F32_D64_BIG_TILE
#define HFA_F32_D64_BIG_TILE 2, 8, 64
#endif
#ifndef HFA_F32_D64_SMALL_TILE
#define HFA_F32_D64_SMALL_TILE 1, 8, 64
#endif
#ifndef HFA_F32_D64_TINY_TILE
#define HFA_F32_D64_TINY_TILE 1, 4, 64
#endif
// fp32, d = 128: 128-row workgroups (one block per wave, 8 waves), and
// 64-row ones (4 waves) for shapes whose 128-row grid leaves CUs idle.
#ifndef HFA_F32_D128_TILE
#define HFA_F32_D128_TILE 1, 8, 32
#endif
#ifndef HFA_F32_D128_TINY_TILE
#define HFA_F32_D128_TINY_TILE 1, 4, 32
#endif
using Bf16D128 = Bf16Tile<128, HFA_BF16_D128_TILE>;
using Bf16D64 = Bf16Tile<64, HFA_BF16_D64_TILE>;
using Bf16D64Long = Bf16Tile<64, HFA_BF16_D64_LONG_TILE>;
constexpr int64_t kBf16LongKeys = 4096;
// bf16, 128-row workgroups of 4 waves (no ping-pong) for grids of 256-row
// workgroups that leave compute units idle and are not split.
#ifndef HFA_BF16_SOLO
#define HFA_BF16_SOLO 1
#endif
#ifndef HFA_BF16_SOLO_MAX_N_D128
#define HFA_BF16_SOLO_MAX_N_D128 4096
#endif
using Bf16SoloD128 = Bf16SoloTile<128>;
using Bf16SoloD64 = Bf16SoloTile<64>;
static_assert(Bf16D64Long::BR == Bf16D64::BR, "both d = 64 tilings cover the same query rows");
using F32D64Big = F32Tile<64, HFA_F32_D64_BIG_TILE>;
using F32D64Small = F32Tile<64, HFA_F32_D64_SMALL_TILE>;
using F32D64Tiny = F32Tile<64, HFA_F32_D64_TINY_TILE>;
using F32D128 = F32Tile<128, HFA_F32_D128_TILE>;
using F32D128Tiny = F32Tile<128, HFA_F32_D128_TINY_TILE>;
static_assert(F32D128Tiny::PACKB == F32D128::PACKB && F32D128Tiny::KT == F32D128::KT,
              "both d = 128 tilings use the same packed tile images");

constexpr double kLog2e = 1.44269504088896340736;  // 1 / ln 2
constexpr int64_t kComputeUnits = 256;  // gfx950 (MI350 series): 8 XCDs x 32 CUs

// Whether a grid of B_r-row workgroups gives every compute unit one.
bool fills_cus(int64_t BH, int64_t N, int64_t br) { return BH * ((N + br - 1) / br) >= kComputeUnits; }

// fp32, d = 64 tiling of a shape: 2 = 256 rows, 1 = 128 rows, 0 = 64 rows.
// Each tiling runs one workgroup per compute unit, so a launch takes
// ceil(workgroups / CUs) rounds of one workgroup's time, which grows with its
// rows over the tiling's throughput per row.  Relative throughputs measured
// on the device (µs per row and key over many shapes): 128-row tiles 0.86
// and 64-row tiles 0.6 of the 256-row tile's.  The tiling with the least
// rounds x rows / throughput wins, the larger one on a tie.
double f32_tiling_cost(int64_t BH, int64_t N, int64_t br, double rel_rate) {
  const int64_t groups = BH * ((N + br - 1) / br);
  return static_cast<double>((groups + kComputeUnits - 1) / kComputeUnits) * static_cast<double>(br) / rel_rate;
}
int f32_d64_tiling(int64_t BH, int64_t N) {
  const double big = f32_tiling_cost(BH, N, F32D64Big::BR, 1.0);
  const double small = f32_tiling_cost(BH, N, F32D64Small::BR, 0.86);
  const double tiny = f32_tiling_cost(BH, N, F32D64Tiny::BR, 0.6);
  if (big <= small && big <= tiny) return 2;
  return small <= tiny ? 1 : 0;
}

// Raise the dynamic-LDS limit of a kernel once per process (per device the
// attribute is a property of the function).
template <class Kernel>
hfa_status ensure_lds(Kernel kernel, int bytes, std::once_flag& flag, hipError_t& err) {
  std::call_once(flag, [&] {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  });
  return err == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

// Scale handling shared by both kernels: the kernels take a positive
// log2-domain multiplier c2 = |scale| * log2(e) and fold the sign of the
// scale into Q (q_mode = +1, -1, or 0 for scale == 0, where every score is 0).
struct ScaleArgs {
  double c2;
  int q_mode;
};
ScaleArgs split_scale(float scale) {
  if (scale == 0.0f) return {1.0, 0};
  const double s = static_cast<double>(scale);
  return {std::fabs(s) * kLog2e, s < 0 ? -1 : 1};
}

// Key split of a bf16 launch: `nsplit` ranges of `tiles` key tiles each
// (every range non-empty); nsplit == 1 is the plain launch.
struct KeySplit {
  int64_t nsplit;
  int64_t tiles;
};
constexpr int64_t kMaxSplits = 32;
// Keys per K/V tile of the bf16 kernel for head dim d: ranges are whole tiles.
constexpr int64_t key_tile(int64_t d) { return d == 128 ? Bf16D128::KT : Bf16D64::KT; }

KeySplit make_split(int64_t N, int64_t d, int64_t want) {
  const int64_t kt = key_tile(d);
  const int64_t ntiles = (N + kt - 1) / kt;
  const int64_t s = std::max<int64_t>(1, std::min<int64_t>({want, ntiles, kMaxSplits}));
  const int64_t tiles = (ntiles + s - 1) / s;
  return {(ntiles + tiles - 1) / tiles, tiles};
}

// The split hfa_attn_fwd_split chooses when asked for none in particular:
// shapes whose 256-row tiles give fewer workgroups than compute units split
// their keys into as many ranges as still fit one round of workgroups on the
// compute units, each range at least kMinSplitKeys keys long (shorter ranges
// lose more to the partial results' round trip through memory and the
// per-workgroup start-up than they gain; measured on the device).
constexpr int64_t kMinSplitKeys = 2048;
int64_t auto_splits(hfa_dtype dtype, int64_t BH, int64_t N, int64_t d) {
  if (dtype != HFA_BF16) return 1;
  const int64_t br = d == 128 ? Bf16D128::BR : Bf16D64::BR;
  const int64_t grid = BH * ((N + br - 1) / br);
  if (grid >= kComputeUnits) return 1;
  const int64_t want = std::min<int64_t>(kComputeUnits / grid, N / kMinSplitKeys);
  return want < 2 ? 1 : make_split(N, d, want).nsplit;
}

// Workspace bytes of a split launch: the partial outputs [nsplit][BH][N][d]
// fp32, then the partial log-sum-exps [nsplit][BH][N] fp32.
int64_t split_workspace_bytes(int64_t nsplit, int64_t BH, int64_t N, int64_t d) {
  return nsplit <= 1 ? 0 : nsplit * BH * N * (d + 1) * 4;
}

// With launch == false only the one-time kernel attributes are set (before a
// stream capture, which must contain nothing but the launches).  A split
// launch (ks.nsplit > 1) writes its partial results to `work` and merges them
// into o and lse with a second kernel.
template <class T, bool kCanSplit = true>
hfa_status launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                       int64_t N, float scale, hipStream_t stream, bool launch, KeySplit ks = {1, 0},
                       void* work = nullptr) {
  static std::once_flag flag, flag_split;
  static hipError_t err = hipSuccess, err_split = hipSuccess;
  auto kernel = attn_fwd_bf16_kernel<T, false>;
  if (ensure_lds(kernel, T::LDS_BYTES, flag, err) != HFA_OK) return HFA_ERR_LAUNCH;
  if constexpr (kCanSplit) {
    if (ensure_lds(attn_fwd_bf16_kernel<T, true>, T::LDS_BYTES, flag_split, err_split) != HFA_OK)
      return HFA_ERR_LAUNCH;
  } else {
    if (ks.nsplit > 1) return HFA_ERR_UNSUPPORTED;  // the dispatch never asks this tiling for a split
  }
  if (!launch) return HFA_OK;
  const int64_t n_qt = (N + T::BR - 1) / T::BR;
  const int64_t total = BH * n_qt * ks.nsplit;
  if (total > INT_MAX || BH * N > INT_MAX) return HFA_ERR_SHAPE;
  const ScaleArgs sa = split_scale(scale);
  SplitArgs sp{static_cast<int>(ks.nsplit), static_cast<int>(ks.tiles), nullptr, nullptr};
  auto chosen = kernel;
  if constexpr (kCanSplit) {
    if (ks.nsplit > 1) {
      sp.part_o = static_cast<float*>(work);
      sp.part_lse = sp.part_o + ks.nsplit * BH * N * T::D;
      chosen = attn_fwd_bf16_kernel<T, true>;
    }
  }
  hipLaunchKernelGGL(chosen, dim3(static_cast<unsigned>(total)), dim3(T::NT), T::LDS_BYTES, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                     static_cast<__bf16*>(o), lse, static_cast<int>(N), static_cast<int>(n_qt),
                     static_cast<int>(total), static_cast<float>(sa.c2), sa.q_mode, sp);
  if (hipGetLastError() != hipSuccess) return HFA_ERR_LAUNCH;
  if (ks.nsplit > 1) {
    const int64_t rows = BH * N;
    constexpr int64_t rows_per_block = 256 / (T::D / 8);
    hipLaunchKernelGGL(attn_merge_bf16_kernel<T::D>, dim3(static_cast<unsigned>((rows + rows_per_block - 1) /
                                                                                  rows_per_block)),
                       dim3(256), 0, stream, sp.part_o, sp.part_lse, static_cast<__bf16*>(o), lse,
                       static_cast<int>(rows), static_cast<int>(ks.nsplit));
    if (hipGetLastError() != hipSuccess) return HFA_ERR_LAUNCH;
  }
  return HFA_OK;
}

template <class T>
hfa_status launch_bf16_solo(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                            int64_t N, float scale, hipStream_t stream, bool launch) {
  static std::once_flag flag;
  static hipError_t err = hipSuccess;
  auto kernel = attn_fwd_bf16_solo_kernel<T>;
  if (ensure_lds(kernel, T::LDS_BYTES, flag, err) != HFA_OK) return HFA_ERR_LAUNCH;
  if (!launch) return HFA_OK;
  const int64_t n_qt = (N + T::BR - 1) / T::BR;
  const int64_t total = BH * n_qt;
  if (total > INT_MAX || BH * N > INT_MAX) return HFA_ERR_SHAPE;
  const ScaleArgs sa = split_scale(scale);
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(total)), dim3(T::NT), T::LDS_BYTES, stream,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k), static_cast<const __bf16*>(v),
                     static_cast<__bf16*>(o), lse, static_cast<int>(N), static_cast<int>(n_qt),
                     static_cast<int>(total), static_cast<float>(sa.c2), sa.q_mode);
  return hipGetLastError() == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

// Whether an unsplit bf16 call runs the 128-row 4-wave kernel: its grid
// (twice the 256-row one) still fits one round over the compute units, and at
// d = 128 N <= 4096.  Measured against the 256-row kernel: 9-25 % faster on
// such grids (N = 333 to 3000 at d = 64, 128 to 2048 at d = 128), +3 % at
// d = 128, N = 4096, and 1.5 % slower at N = 8192, where the ping-pong pair's
// overlap of two waves per SIMD outweighs the doubled workgroups.
bool bf16_solo(int64_t BH, int64_t N, int64_t d) {
  const int64_t grid = BH * ((N + Bf16D128::BR - 1) / Bf16D128::BR);
  return HFA_BF16_SOLO && 2 * grid <= kComputeUnits && (d == 64 || N <= HFA_BF16_SOLO_MAX_N_D128);
}

// Bytes of pre-formatted K/V tiles (f32_pack_kernel) for B*H heads of N keys.
template <class T>
int64_t f32_pack_bytes(int64_t BH, int64_t N) {
  return BH * ((N + T::KT - 1) / T::KT) * T::PACKB;
}

// ws: workspace of at least f32_pack_bytes<T> bytes for the packed path
// (K and V formatted once, then copied into LDS as they are), or null for the
// path that formats every tile in every workgroup.
template <class T>
hfa_status launch_f32(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH,
                      int64_t N, float scale, hipStream_t stream, bool launch, void* ws = nullptr) {
  static std::once_flag flag, flag_packed;
  static hipError_t err = hipSuccess, err_packed = hipSuccess;
  auto kernel = attn_fwd_f32_kernel<T, false>;
  auto kernel_packed = attn_fwd_f32_kernel<T, true>;
  if (ensure_lds(kernel, T::LDS_BYTES, flag, err) != HFA_OK) return HFA_ERR_LAUNCH;
  if (ensure_lds(kernel_packed, T::P_LDS_BYTES, flag_packed, err_packed) != HFA_OK) return HFA_ERR_LAUNCH;
  if (!launch) return HFA_OK;
  const int64_t n_qt = (N + T::BR - 1) / T::BR;
  const int64_t total = BH * n_qt;
  const int64_t ntiles = (N + T::KT - 1) / T::KT;
  if (total > INT_MAX || BH * ntiles > INT_MAX) return HFA_ERR_SHAPE;
  const ScaleArgs sa = split_scale(scale);
  if (ws) {
    hipLaunchKernelGGL(f32_pack_kernel<T>, dim3(static_cast<unsigned>(BH * ntiles)), dim3(T::NT), 0, stream,
                       static_cast<const float*>(k), static_cast<const float*>(v), static_cast<char*>(ws),
                       static_cast<int>(N), static_cast<int>(ntiles));
    if (hipGetLastError() != hipSuccess) return HFA_ERR_LAUNCH;
  }
  hipLaunchKernelGGL(ws ? kernel_packed : kernel, dim3(static_cast<unsigned>(total)), dim3(T::NT),
                     ws ? T::P_LDS_BYTES : T::LDS_BYTES, stream, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v), static_cast<float*>(o), lse,
                     static_cast<int>(N), static_cast<int>(n_qt), static_cast<int>(total), sa.c2, sa.q_mode,
                     static_cast<const char*>(ws));
  return hipGetLastError() == hipSuccess ? HFA_OK : HFA_ERR_LAUNCH;
}

// Every argument check of hfa_attn_fwd, before any HIP call.
hfa_status validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int64_t B,
                    int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype) {
  if (dtype != HFA_F32 && dtype != HFA_BF16) return HFA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return HFA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse) return HFA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1) return HFA_ERR_SHAPE;
  if (N > INT_MAX / d) return HFA_ERR_SHAPE;
  if (B > INT64_MAX / H) return HFA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > INT_MAX) return HFA_ERR_SHAPE;
  if (!std::isfinite(scale)) return HFA_ERR_SCALE;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4))
    return HFA_ERR_ALIGN;
  const size_t elt = dtype == HFA_F32 ? 4 : 2;
  const size_t n_elems = static_cast<size_t>(BH) * static_cast<size_t>(N) * static_cast<size_t>(d);
  const size_t bytes = n_elems * elt;
  const size_t lse_bytes = static_cast<size_t>(BH) * static_cast<size_t>(N) * sizeof(float);
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes) ||
      overlaps(lse, lse_bytes, q, bytes) || overlaps(lse, lse_bytes, k, bytes) ||
      overlaps(lse, lse_bytes, v, bytes) || overlaps(lse, lse_bytes, o, bytes))
    return HFA_ERR_ALIAS;
  return HFA_OK;
}

// Kernel selection for a validated call; enqueues it on `stream` when launch.
// ks / work: the key split of a bf16 call and its workspace; for fp32, work
// is the packed path's workspace (or null).
hfa_status dispatch(const void* q, const void* k, const void* v, void* o, float* lse, int64_t BH, int64_t N,
                    int64_t d, float scale, hfa_dtype dtype, hipStream_t st, bool launch, KeySplit ks = {1, 0},
                    void* work = nullptr) {
  if (dtype == HFA_BF16) {
    if (ks.nsplit == 1 && bf16_solo(BH, N, d)) {
      if (d == 128) return launch_bf16_solo<Bf16SoloD128>(q, k, v, o, lse, BH, N, scale, st, launch);
      return launch_bf16_solo<Bf16SoloD64>(q, k, v, o, lse, BH, N, scale, st, launch);
    }
    if (d == 128) return launch_bf16<Bf16D128>(q, k, v, o, lse, BH, N, scale, st, launch, ks, work);
    if (ks.nsplit == 1 && N >= kBf16LongKeys)
      return launch_bf16<Bf16D64Long, false>(q, k, v, o, lse, BH, N, scale, st, launch);
    return launch_bf16<Bf16D64>(q, k, v, o, lse, BH, N, scale, st, launch, ks, work);
  }
  if (d == 64) {
    switch (f32_d64_tiling(BH, N)) {
      case 2: return launch_f32<F32D64Big>(q, k, v, o, lse, BH, N, scale, st, launch, work);
      case 1: return launch_f32<F32D64Small>(q, k, v, o, lse, BH, N, scale, st, launch, work);
      default: return launch_f32<F32D64Tiny>(q, k, v, o, lse, BH, N, scale, st, launch, work);
    }
  }
  if (fills_cus(BH, N, F32D128::BR)) return launch_f32<F32D128>(q, k, v, o, lse, BH, N, scale, st, launch, work);
  return launch_f32<F32D128Tiny>(q, k, v, o, lse, BH, N, scale, st, launch, work);
}

// Formatting K and V once per call pays when enough query-row tiles
// (workgroups) of a head share each key tile, each of which would otherwise
// format every key tile itself, and when the heads are long enough for the
// attention work (N^2 per head) to hide the packing pass (N per head).
// Measured on MI355X at d=64: +1-3 % at N=2048 (8 row tiles), +4 % at 4096,
// +7 % at 16384, break-even at N=1024, -23 % at N=200 (one row tile); at
// d=128: +12 % at N=2048, +26 % at 4096.
constexpr int64_t kPackMinRowTiles = 8;
constexpr int64_t kPackMinKeyTiles = 32;

// The fp32 tiling's query rows per workgroup.
int64_t f32_block_rows(int64_t BH, int64_t N, int64_t d) {
  if (d == 128) return fills_cus(BH, N, F32D128::BR) ? F32D128::BR : F32D128Tiny::BR;
  const int t = f32_d64_tiling(BH, N);
  return t == 2 ? F32D64Big::BR : t == 1 ? F32D64Small::BR : F32D64Tiny::BR;
}

bool f32_pack_pays(int64_t BH, int64_t N, int64_t d) {
  const int64_t br = f32_block_rows(BH, N, d);
  const int64_t kt = d == 128 ? F32D128::KT : F32D64Big::KT;
  return (N + br - 1) / br >= kPackMinRowTiles && (N + kt - 1) / kt >= kPackMinKeyTiles;
}

// Workspace bytes of the packed fp32 path for the tiling the call would use.
int64_t f32_workspace_bytes(int64_t BH, int64_t N, int64_t d) {
  if (d == 128) return f32_pack_bytes<F32D128>(BH, N);
  switch (f32_d64_tiling(BH, N)) {
    case 2: return f32_pack_bytes<F32D64Big>(BH, N);
    case 1: return f32_pack_bytes<F32D64Small>(BH, N);
    default: return f32_pack_bytes<F32D64Tiny>(BH, N);
  }
}

// ---- allocation-free key split ----------------------------------------------
// The workspace of hfa_attn_fwd_split_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not
// a device address): it takes each device's address once with
// hipGetSymbolAddress, that device current, and passes that.

// This device's address of `scratch` (nullptr if it cannot be had).
void* scratch_address(int dev) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

// A captured and instantiated sequence of attention launches.
struct hfa_graph_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

extern "C" {

int64_t hfa_block_rows(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d) {
  if (B < 1 || H < 1 || N < 1 || B > INT64_MAX / H) return 0;
  if (dtype == HFA_BF16 && (d == 64 || d == 128)) {
    if (bf16_solo(B * H, N, d)) return Bf16SoloD128::BR;  // unsplit calls; a key split keeps 256 rows
    return d == 128 ? Bf16D128::BR : Bf16D64::BR;
  }
  if (dtype == HFA_F32 && d == 64) {
    const int t = f32_d64_tiling(B * H, N);
    return t == 2 ? F32D64Big::BR : t == 1 ? F32D64Small::BR : F32D64Tiny::BR;
  }
  if (dtype == HFA_F32 && d == 128) return fills_cus(B * H, N, F32D128::BR) ? F32D128::BR : F32D128Tiny::BR;
  return 0;
}

const char* hfa_status_str(hfa_status s) {
  switch (s) {
    case HFA_OK: return "ok";
    case HFA_ERR_NULL: return "a required pointer is NULL";
    case HFA_ERR_SHAPE: return "invalid shape: B, H, N must be >= 1 and N*d < 2^31";
    case HFA_ERR_UNSUPPORTED: return "unsupported head dim (64 or 128) or dtype";
    case HFA_ERR_SCALE: return "scale must be finite";
    case HFA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case HFA_ERR_ALIAS: return "o or lse overlaps an input or each other";
    case HFA_ERR_NO_DEVICE: return "no current gfx950 HIP device";
    case HFA_ERR_LAUNCH: return "kernel launch failed";
    case HFA_ERR_EPS: return "eps must be finite and > 0";
    case HFA_ERR_WORKSPACE: return "workspace smaller than the key split needs";
    default: break;
  }
  return "unknown status";
}

hfa_status hfa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                        int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype, void* stream) {
  const hfa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype);
  if (st != HFA_OK) return st;
  const hfa_status dev = check_device();
  if (dev != HFA_OK) return dev;
  return dispatch(q, k, v, o, lse, B * H, N, d, scale, dtype, static_cast<hipStream_t>(stream), true);
}

int64_t hfa_key_splits(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d) {
  if ((dtype != HFA_F32 && dtype != HFA_BF16) || (d != 64 && d != 128)) return 0;
  if (B < 1 || H < 1 || N < 1 || B > INT64_MAX / H || N > INT_MAX / d) return 0;
  return auto_splits(dtype, B * H, N, d);
}

int64_t hfa_attn_fwd_workspace_size(hfa_dtype dtype, int64_t B, int64_t H, int64_t N, int64_t d, int64_t splits) {
  if ((dtype != HFA_F32 && dtype != HFA_BF16) || (d != 64 && d != 128)) return -1;
  if (B < 1 || H < 1 || N < 1 || B > INT64_MAX / H || N > INT_MAX / d || splits < 0) return -1;
  if (B * H > INT_MAX / N) return -1;
  const bool library_choice = splits == 0;
  if (splits == 0) splits = auto_splits(dtype, B * H, N, d);
  if (dtype != HFA_BF16 && splits > 1) return -1;
  if (dtype == HFA_F32) {
    // 0: the library's choice (no workspace where packing would not pay);
    // 1: the packed path's workspace in any case
    if (library_choice && !f32_pack_pays(B * H, N, d)) return 0;
    return f32_workspace_bytes(B * H, N, d);
  }
  return split_workspace_bytes(make_split(N, d, splits).nsplit, B * H, N, d);
}

hfa_status hfa_attn_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                              int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype, int64_t splits,
                              void* workspace, int64_t workspace_bytes, void* stream) {
  const hfa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype);
  if (st != HFA_OK) return st;
  if (splits < 0) return HFA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > INT_MAX / N) return HFA_ERR_SHAPE;
  if (splits == 0) splits = auto_splits(dtype, BH, N, d);
  if (dtype != HFA_BF16 && splits > 1) return HFA_ERR_UNSUPPORTED;
  const KeySplit ks = make_split(N, d, splits);
  // bf16: a workspace only for a split; fp32: optional, the packed path
  // when one is given
  const bool use_ws = dtype == HFA_F32 ? workspace != nullptr : ks.nsplit > 1;
  if (use_ws) {
    const int64_t need =
        dtype == HFA_F32 ? f32_workspace_bytes(BH, N, d) : split_workspace_bytes(ks.nsplit, BH, N, d);
    if (!workspace) return HFA_ERR_NULL;
    if (misaligned(workspace, 16)) return HFA_ERR_ALIGN;
    if (workspace_bytes < need) return HFA_ERR_WORKSPACE;
    const size_t elt = dtype == HFA_F32 ? 4 : 2;
    const size_t bytes = static_cast<size_t>(BH) * static_cast<size_t>(N) * static_cast<size_t>(d) * elt;
    const size_t lse_bytes = static_cast<size_t>(BH) * static_cast<size_t>(N) * 4;
    const size_t wb = static_cast<size_t>(need);
    if (overlaps(workspace, wb, q, bytes) || overlaps(workspace, wb, k, bytes) || overlaps(workspace, wb, v, bytes) ||
        overlaps(workspace, wb, o, bytes) || overlaps(workspace, wb, lse, lse_bytes))
      return HFA_ERR_ALIAS;
  }
  const hfa_status dev = check_device();
  if (dev != HFA_OK) return dev;
  return dispatch(q, k, v, o, lse, BH, N, d, scale, dtype, static_cast<hipStream_t>(stream), true, ks,
                  use_ws ? workspace : nullptr);
}

hfa_status hfa_attn_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                                      int64_t B, int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype,
                                      int64_t splits, void* stream) {
  const hfa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype);
  if (st != HFA_OK) return st;
  if (splits < 0) return HFA_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > INT_MAX / N) return HFA_ERR_SHAPE;
  if (splits == 0) splits = auto_splits(dtype, BH, N, d);
  if (dtype != HFA_BF16 && splits > 1) return HFA_ERR_UNSUPPORTED;
  const KeySplit ks = make_split(N, d, splits);
  if (split_workspace_bytes(ks.nsplit, BH, N, d) > kScratchBytes) return HFA_ERR_WORKSPACE;
  const hfa_status devst = check_device();
  if (devst != HFA_OK) return devst;
  void* work = nullptr;
  if (ks.nsplit > 1) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
      (void)hipGetLastError();
      return HFA_ERR_NO_DEVICE;
    }
    work = scratch_address(dev);
    if (!work) return HFA_ERR_LAUNCH;
  }
  return dispatch(q, k, v, o, lse, BH, N, d, scale, dtype, static_cast<hipStream_t>(stream), true, ks, work);
}

hfa_status hfa_attn_fwd_graph_create(const void* q, const void* k, const void* v, void* o, float* lse,
                                     int64_t B, int64_t H, int64_t N, int64_t d, float scale, hfa_dtype dtype,
                                     int64_t count, hfa_graph* out) {
  if (!out) return HFA_ERR_NULL;
  *out = nullptr;
  const hfa_status st = validate(q, k, v, o, lse, B, H, N, d, scale, dtype);
  if (st != HFA_OK) return st;
  if (count < 1 || count > (1 << 20)) return HFA_ERR_SHAPE;
  const hfa_status dev = check_device();
  if (dev != HFA_OK) return dev;
  const int64_t BH = B * H;
  if (dispatch(q, k, v, o, lse, BH, N, d, scale, dtype, nullptr, false) != HFA_OK) return HFA_ERR_LAUNCH;

  hipStream_t s = nullptr;
  if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) {
    (void)hipGetLastError();
    return HFA_ERR_LAUNCH;
  }
  hfa_status result = HFA_OK;
  hipGraph_t graph = nullptr;
  if (hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    result = HFA_ERR_LAUNCH;
  } else {
    for (int64_t i = 0; i < count && result == HFA_OK; ++i)
      result = dispatch(q, k, v, o, lse, BH, N, d, scale, dtype, s, true);
    if (hipStreamEndCapture(s, &graph) != hipSuccess && result == HFA_OK) result = HFA_ERR_LAUNCH;
  }
  hipGraphExec_t exec = nullptr;
  if (result == HFA_OK && hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess)
    result = HFA_ERR_LAUNCH;
  (void)hipStreamDestroy(s);
  if (result != HFA_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    (void)hipGetLastError();
    return result;
  }
  hfa_graph g = new (std::nothrow) hfa_graph_s;
  if (!g) {
    (void)hipGraphExecDestroy(exec);
    (void)hipGraphDestroy(graph);
    return HFA_ERR_LAUNCH;
  }
  g->graph = graph;
  g->exec = exec;
  *out = g;
  return HFA_OK;
}

hfa_status hfa_graph_launch(hfa_graph g, void* stream) {
  if (!g) return HFA_ERR_NULL;
  if (hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream)) != hipSuccess) {
    (void)hipGetLastError();
    return HFA_ERR_LAUNCH;
  }
  return HFA_OK;
}

void hfa_graph_destroy(hfa_graph g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
