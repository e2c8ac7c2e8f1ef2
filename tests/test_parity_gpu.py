"""GPU parity: the HIP kernels (through the C ABI) against the fp64 CPU oracle.

Tolerances:
  fp32 -- max |gpu - oracle| <= 1e-5 on O and on LSE (the TritonForge page's
          parity bound, atol = 1e-5, taken against the exact fp64 result).
          Where half an fp32 ulp of the exact value exceeds 1e-5 (|LSE| >= 256,
          reached only by the extra peaked case, never by the five evaluation
          shapes) no fp32 output can meet 1e-5; there the bound is half an
          ulp + 1e-6, i.e. correct rounding up to 1e-6 of computation error;
  bf16 -- |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| element-wise on O and LSE.
The oracle reads the very host bytes that are copied to the device.
"""

import math

import numpy as np
import pytest
import torch

import fa2_fwd_amd as hfa
import oracle
from fa2_fwd_amd import workloads as W

from parity_util import (BF16_ATOL, BF16_RTOL, F32_ATOL, _log, assert_close, check_case, f32_tolerance,  # noqa: F401
                         run_gpu, run_gpu_direct, run_oracle)

pytestmark = pytest.mark.gpu


# ---- the five evaluation shapes --------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_fp32_configs_full(cfg):
    w = W.CONFIGS[cfg]
    q, k, v = W.workload_inputs(w)
    check_case(w.describe(), q, k, v, w.scale, w.dtype)


def test_bf16_config4_full():
    # B=2 H=32 N=4096 d=128: every query row of every head (the oracle needs ~20 s).
    w = W.CONFIGS[4]
    q, k, v = W.workload_inputs(w)
    check_case(w.describe(), q, k, v, w.scale, w.dtype)


def test_bf16_config5_whole_tiles():
    # B=1 H=16 N=16384 d=128, the same launch as the benchmark.  The oracle checks
    # three whole 256-row query tiles of every head (the first, one in the middle
    # and the last: every wave of the workgroup, every lane) plus seeded random
    # rows, ~5 % of the rows.
    w = W.CONFIGS[5]
    br = hfa.hfa_block_rows(hfa.HFA_BF16, w.B, w.H, w.N, w.d)
    q, k, v = W.workload_inputs(w)
    tiles = [0, (w.N // br) // 2, w.N // br - 1]
    whole = np.concatenate([np.arange(t * br, (t + 1) * br) for t in tiles])
    rows = np.unique(np.r_[whole, W.sample_rows(w.N, 64, seed=1005)]).astype(np.int64)
    check_case(w.describe() + f" ({len(rows)} rows/head, tiles {tiles} of {br} rows whole)", q, k, v, w.scale,
               w.dtype, rows=rows)


# ---- awkward shapes: ragged tails, one row, tiny and odd N ------------------

AWKWARD_N = [1, 2, 17, 63, 64, 65, 127, 129, 1000]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", AWKWARD_N)
def test_awkward_shapes(dtype, d, N):
    B, H = (1, 3) if N % 2 else (3, 1)
    q, k, v = W.make_inputs(B, H, N, d, dtype, seed=N * 7 + d)
    check_case(f"awkward {dtype} B={B} H={H} N={N} d={d}", q, k, v, 1.0 / math.sqrt(d), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_long_ragged_sequence(dtype, d):
    N = 4097
    q, k, v = W.make_inputs(1, 2, N, d, dtype, seed=4097 + d, qk_mult=2.0 if dtype == "f32" else 1.0)
    rows = W.sample_rows(N, 40, seed=d)
    check_case(f"ragged {dtype} N={N} d={d}", q, k, v, 1.0 / math.sqrt(d), dtype, rows=rows)


@pytest.mark.parametrize("B,H,N", [(1, 16, 4095), (1, 16, 4096), (1, 16, 5000), (2, 8, 8192), (1, 2, 8192)])
def test_bf16_d64_long_key_tiles(B, H, N):
    # bf16 d=64 calls that are not split take 128-key tiles from N = 4096 on (64-key tiles
    # below, and in every split): both sides of the threshold, a ragged last tile, and a
    # shape the automatic split takes (1x2x8192).
    q, k, v = W.make_inputs(B, H, N, 64, "bf16", seed=6400 + N + H)
    rows = W.sample_rows(N, 48, seed=N)
    check_case(f"bf16 d=64 B={B} H={H} N={N}", q, k, v, 0.125, "bf16", rows=rows)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_very_long_sequence(dtype, d):
    # 2^18 + 1 keys: 4097 key tiles, one ragged; rows sampled across every query tile range.
    N = (1 << 18) + 1
    q, k, v = W.make_inputs(1, 1, N, d, dtype, seed=262145 + d)
    rows = np.unique(np.r_[0, 1, N // 2, N - 2, N - 1, W.sample_rows(N, 19, seed=d)])
    check_case(f"very long {dtype} N={N} d={d}", q, k, v, 1.0 / math.sqrt(d), dtype, rows=rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_peaked_rows(dtype):
    # Q and K x8: score standard deviation ~ 64 * scale; stresses the rescale.
    q, k, v = W.make_inputs(2, 2, 700, 64, dtype, seed=77, qk_mult=8.0)
    check_case(f"peaked {dtype}", q, k, v, 0.125, dtype)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("spread", [0, 10, 24])
def test_f32_wide_range_rows(d, spread):
    # Entries log-uniform over 2^-spread .. 2^spread (random signs), rows scaled
    # by 2^-8 .. 2^8 as well, so small entries of q meet large entries of k.
    # Where the int8 slices of such rows cannot hold the scores to the fp32
    # budget, the kernel's check recomputes them exactly; either way the
    # plain fp32 tolerance holds.
    B, H, N = 1, 2, 300
    g = torch.Generator("cpu").manual_seed(4000 + 10 * d + spread)

    def wide(n):
        mag = torch.exp2((torch.rand(B, H, n, d, generator=g) * 2 - 1) * spread)
        sign = torch.where(torch.rand(B, H, n, d, generator=g) < 0.5, -1.0, 1.0)
        rows = torch.exp2(torch.randint(-8, 9, (B, H, n, 1), generator=g).float())
        return (mag * sign * rows / 2.0 ** (spread / 2)).float().contiguous()

    q, k = wide(N), wide(N)
    v = torch.randn(B, H, N, d, generator=g)
    scale = 1.0 / math.sqrt(d)
    # keep scores finite and moderate: normalise so the largest |s| is ~ 60
    qk = (q.double() @ k.double().transpose(-1, -2)).abs().amax()
    q = (q * float(60.0 / (float(qk) * scale))).float().contiguous()
    check_case(f"f32 wide range d={d} spread=2^{spread}", q, k, v, scale, "f32")


def outlier_inputs(B, H, N, d, seed, heads=None, rows=None):
    """Entries ~1e-3 with one outlier channel per row (q: ~1e3 on channel 5, k: ~1e4 on
    channel 11), in the heads `heads` (all when None) and query rows `rows` (all when None).
    The small q entry on k's outlier channel is held by the int8 slices to 2^(10-35)
    only: those scores miss by ~4e-4, far outside the fp32 budget."""
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn(B, H, N, d, generator=g) * 1e-3
    k = torch.randn(B, H, N, d, generator=g) * 1e-3
    v = torch.randn(B, H, N, d, generator=g)

    def big(mag):
        return mag * torch.where(torch.rand(B, H, N, generator=g) < 0.5, -1.0, 1.0) * (1 + torch.rand(B, H, N, generator=g))

    qo, ko = big(1e3), big(1e4)
    hsel = torch.zeros(H, dtype=torch.bool)
    hsel[list(range(H)) if heads is None else heads] = True
    rsel = torch.zeros(N, dtype=torch.bool)
    rsel[list(range(N)) if rows is None else rows] = True
    qmask = hsel.view(1, H, 1) & rsel.view(1, 1, N)
    q[..., 5] = torch.where(qmask, qo, q[..., 5])
    k[..., 11] = torch.where(hsel.view(1, H, 1), ko, k[..., 11])
    return q.contiguous(), k.contiguous(), v.contiguous()


@pytest.mark.parametrize("B,H,N,d", [(1, 256, 200, 64), (2, 64, 300, 64), (1, 255, 256, 64), (1, 4, 777, 64),
                                     (1, 1, 65, 64), (1, 3, 333, 128), (1, 2, 1000, 128)])
def test_f32_outlier_channels(B, H, N, d):
    # Every fp32 tiling (256-, 128- and 64-row workgroups at d=64, d=128) with
    # ragged N; every other head carries the outliers, so workgroups on the
    # exact scores and on the int8 products run side by side.
    q, k, v = outlier_inputs(B, H, N, d, seed=7000 + B * H + N + d, heads=list(range(0, H, 2)))
    rows = None if B * H * N <= 20000 else W.sample_rows(N, 24, seed=N)
    br = hfa.hfa_block_rows(hfa.HFA_F32, B, H, N, d)
    check_case(f"f32 outlier channels B={B} H={H} N={N} d={d} (B_r={br})", q, k, v, 1.0 / math.sqrt(d), "f32",
               rows=rows)


def test_f32_outlier_rows_in_one_tile():
    # Outlier channels in three query rows of one 256-row tile only: that
    # workgroup alone recomputes exactly.
    q, k, v = outlier_inputs(1, 256, 512, 64, seed=7100, heads=[3], rows=[260, 300, 511])
    check_case("f32 outliers in three rows of one tile", q, k, v, 0.125, "f32",
               rows=np.r_[0, 1, 255, 256, 260, 300, 511])


@pytest.mark.parametrize("N", [1, 64, 65, 128, 129, 192, 257, 320, 333, 449])
def test_f32_d64_few_key_tiles(N):
    # 256 heads with 1 to 8 key tiles of 64: the first tiles, the ragged last
    # one and the switch from steady two-tile trips to single steps.  The
    # library's tiling: 64-row tiles up to N = 64, 128-row ones up to 128 and
    # where 256-row ones would take a second, mostly empty round (N = 257 to
    # 384), else 256-row ones (N = 129 to 256 in one round, N = 449 in two
    # rounds against four).
    B, H = 1, 256
    br = hfa.hfa_block_rows(hfa.HFA_F32, B, H, N, 64)
    assert br == (64 if N <= 64 else 128 if N <= 128 or 256 < N <= 384 else 256)
    q, k, v = W.make_inputs(B, H, N, 64, "f32", seed=5000 + N, qk_mult=2.0)
    rows = W.sample_rows(N, 6, seed=N + 1)
    check_case(f"f32 d=64 B=1 H=256 N={N} (few key tiles, B_r={br})", q, k, v, 0.125, "f32", rows=rows)


@pytest.mark.parametrize("B,H,N", [(1, 256, 200), (2, 64, 300), (1, 255, 256), (1, 4, 777), (1, 8, 4000),
                                   (1, 16, 1000), (1, 1, 65)])
def test_f32_d64_all_tilings(B, H, N):
    # fp32 d=64 chooses among 256-, 128- and 64-row workgroups by shape (the
    # least rounds of workgroups times rows over the tiling's throughput): all
    # three here (256: the first three, 128: H=8 N=4000, 64: the rest), ragged N.
    br = hfa.hfa_block_rows(hfa.HFA_F32, B, H, N, 64)
    q, k, v = W.make_inputs(B, H, N, 64, "f32", seed=B * 1000 + H + N, qk_mult=2.0)
    rows = W.sample_rows(N, 24, seed=N)
    check_case(f"f32 d=64 B={B} H={H} N={N} (B_r={br})", q, k, v, 0.125, "f32", rows=rows)


@pytest.mark.parametrize("B,H,N,d", [(1, 16, 1024, 128), (1, 1, 1, 128), (1, 1, 65, 128), (1, 5, 1000, 128),
                                     (2, 3, 333, 64), (4, 8, 1024, 64), (1, 2, 3000, 64), (1, 2, 1537, 64),
                                     (1, 8, 2048, 128)])
def test_bf16_small_grid_kernel(B, H, N, d):
    # The 128-row 4-wave kernel (no ping-pong; every wave streams its quarter
    # of both K and V through 3-deep rings): one key tile, a ragged first or
    # last tile, many tiles, both head dims.
    assert hfa.hfa_block_rows(hfa.HFA_BF16, B, H, N, d) == 128
    q, k, v = W.make_inputs(B, H, N, d, "bf16", seed=B * 100 + H * 10 + N + d)
    rows = None if N <= 1100 else W.sample_rows(N, 48, seed=N + d)
    check_case(f"bf16 4-wave B={B} H={H} N={N} d={d}", q, k, v, 1.0 / math.sqrt(d), "bf16", rows=rows)


@pytest.mark.parametrize("B,H,N", [(1, 4, 4096), (1, 16, 1024), (2, 2, 1500), (1, 1, 33), (2, 8, 2048),
                                   (1, 16, 2047)])
def test_f32_d128_both_tilings(B, H, N):
    # fp32 d=128 takes 128-row workgroups when B*H*ceil(N/128) >= 256, else 64-row
    # ones (4 waves); both, ragged N (check_case runs the packed path too).
    br = hfa.hfa_block_rows(hfa.HFA_F32, B, H, N, 128)
    assert br == (128 if B * H * -(-N // 128) >= 256 else 64)
    q, k, v = W.make_inputs(B, H, N, 128, "f32", seed=B * 1000 + H + N + 128, qk_mult=2.0)
    rows = W.sample_rows(N, 24, seed=N)
    check_case(f"f32 d=128 B={B} H={H} N={N} (B_r={br})", q, k, v, 1.0 / math.sqrt(128), "f32", rows=rows)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_rising_scores(dtype, d):
    # Scores drift linearly along the keys, with a slope that differs per
    # query row (some rows fall, most rise by up to ~15 log2 units per
    # 64-key tile): the running max moves on most tiles, by amounts on both sides of
    # every rescale threshold.
    N = 1000
    g = torch.Generator("cpu").manual_seed(900 + d)
    e = torch.ones(d) / math.sqrt(d)
    slope = torch.linspace(-0.2, 1.0, N).view(N, 1)          # per query row
    ramp = torch.linspace(0.0, 1.0, N).view(N, 1)            # per key
    q = torch.randn(1, 2, N, d, generator=g) + 8.0 * slope * e
    k = torch.randn(1, 2, N, d, generator=g) + 20.75 * math.sqrt(d) * ramp * e
    v = torch.randn(1, 2, N, d, generator=g)
    td = W.torch_dtype(dtype)
    q, k, v = (t.to(td).contiguous() for t in (q, k, v))
    check_case(f"rising {dtype} d={d}", q, k, v, 1.0 / math.sqrt(d), dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.01, 1.0])
def test_other_scales(dtype, scale):
    q, k, v = W.make_inputs(1, 2, 300, 64, dtype, seed=int(abs(scale) * 1000) + 5)
    check_case(f"scale={scale} {dtype}", q, k, v, scale, dtype)


# ---- invariants on device output --------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_invariants_on_device(dtype, d):
    B, H, N = 1, 2, 333
    q, k, v = W.make_inputs(B, H, N, d, dtype, seed=5, qk_mult=4.0)
    tol = 1e-5 if dtype == "f32" else 2e-2
    # constant V -> that constant
    c = v[:, :, :1].expand(B, H, N, d).contiguous()
    o, _ = run_gpu(q, k, c, 1.0 / math.sqrt(d))
    assert np.abs(o - c.double().numpy()).max() <= tol
    # identical keys -> mean of V, LSE = scale q.k + ln N
    kk = k[:, :, :1].expand(B, H, N, d).contiguous()
    o, lse = run_gpu(q, kk, v, 0.125)
    mean_v = v.double().mean(dim=2, keepdim=True).expand(B, H, N, d).numpy()
    assert np.abs(o - mean_v).max() <= tol
    qk = torch.einsum("bhnd,bhd->bhn", q.double(), kk[:, :, 0].double()).numpy()
    ref_lse = 0.125 * qk + math.log(N)
    lse_tol = f32_tolerance(ref_lse) if dtype == "f32" else BF16_ATOL + BF16_RTOL * np.abs(ref_lse)
    assert np.all(np.abs(lse - ref_lse) <= lse_tol)
    # scale 0 -> mean of V, LSE = ln N
    o, lse = run_gpu(q, k, v, 0.0)
    assert np.abs(o - mean_v).max() <= tol
    assert np.abs(lse - math.log(N)).max() <= 1e-5


# ---- engineering checks -----------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bitwise_deterministic(dtype):
    q, k, v = W.make_inputs(2, 4, 1500, 128 if dtype == "bf16" else 64, dtype, seed=9)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o1, l1 = hfa.attn_fwd(qd, kd, vd)
    o2, l2 = hfa.attn_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("B,H,N,d", [(4, 8, 2048, 64), (1, 8, 4096, 64), (1, 4, 4096, 128)])
def test_f32_long_runs_bitwise_repeatable(B, H, N, d):
    # the fp32 kernels' double-buffered LDS tiles, on every fp32 tiling
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(B, H, N, d, "f32", seed=78, qk_mult=4.0))
    o0, l0 = hfa.attn_fwd(q, k, v)
    for _ in range(2):
        o, l = hfa.attn_fwd(q, k, v)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0)


@pytest.mark.parametrize("B,H,N,d", [(1, 8, 4096, 128), (2, 16, 8192, 64), (2, 32, 4096, 128)])
def test_bf16_long_runs_bitwise_repeatable(B, H, N, d):
    # Three runs of long bf16 sequences (64 key tiles and more; a grid of half the CUs, the
    # 128-key tiles of d=64, the #4 workload) must agree bit for bit.  A K/V tile read while
    # its ring slot is being refilled changes some outputs by ~1e-2, which the tolerance
    # against the oracle can miss but repetition does not: the copy and the reads race.
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(B, H, N, d, "bf16", seed=77))
    o0, l0 = hfa.attn_fwd(q, k, v, splits=1)
    for _ in range(2):
        o, l = hfa.attn_fwd(q, k, v, splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o, o0) and torch.equal(l, l0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_writes_stay_in_bounds(dtype):
    # O and LSE live inside larger guard buffers; nothing outside may change.
    B, H, N, d = 1, 3, 130, 64
    q, k, v = W.make_inputs(B, H, N, d, dtype, seed=11)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    n = B * H * N * d
    guard = 4096
    obuf = torch.full((n + 2 * guard,), 7.0, dtype=qd.dtype, device=dev)
    lbuf = torch.full((B * H * N + 2 * guard,), 7.0, dtype=torch.float32, device=dev)
    o = obuf[guard:guard + n].view(B, H, N, d)
    lse = lbuf[guard:guard + B * H * N].view(B, H, N)
    hfa.attn_fwd(qd, kd, vd, out=o, lse=lse)
    torch.cuda.synchronize()
    for buf in (obuf, lbuf):
        assert torch.all(buf[:guard] == 7.0) and torch.all(buf[-guard:] == 7.0)
    ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(d))
    assert_close("guarded", o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, dtype)


def test_side_stream():
    q, k, v = W.make_inputs(1, 2, 256, 128, "bf16", seed=12)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = hfa.attn_fwd(qd, kd, vd)
    s.synchronize()
    ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(128))
    assert_close("side stream", o.float().cpu().double().numpy(), lse.cpu().double().numpy(), ro, rl, "bf16")


def test_status_on_device():
    # a validation error on a real device still returns before launching
    q = torch.zeros(1, 1, 16, 96, device="cuda:0")
    with pytest.raises(hfa.HfaError) as ei:
        hfa.attn_fwd(q, q, q)
    assert ei.value.status == hfa.HFA_ERR_UNSUPPORTED


def _views_with_high_low_word(shapes, dtype, dev):
    """Tensors placed at device addresses whose low 32-bit word has bit 31 set.

    The kernels split 64-bit source addresses into 32-bit halves; this pins
    that the low half is widened without sign extension.
    """
    elt = torch.empty((), dtype=dtype).element_size()
    sizes = [math.prod(s) * elt for s in shapes]
    pool = torch.empty(4 * 2**30 + sum(sizes) + 4096 * len(shapes), dtype=torch.uint8, device=dev)
    base = pool.data_ptr()
    # first 256-byte aligned address >= base whose bit 31 is set
    cand = (base | 0x80000000) if (base & 0x80000000) == 0 else base
    cand = (cand + 255) & ~255
    if cand < base:
        cand += 2**32
    off = cand - base
    views = []
    for s, nbytes in zip(shapes, sizes):
        assert ((base + off) & 0x80000000) != 0
        views.append(pool[off:off + nbytes].view(dtype).view(s))
        off += (nbytes + 4095) // 4096 * 4096
    return pool, views


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 300])
def test_addresses_with_bit31_set(dtype, d, N):
    B, H = 1, 2
    q, k, v = W.make_inputs(B, H, N, d, dtype, seed=31 + N + d)
    dev = torch.device("cuda:0")
    td = W.torch_dtype(dtype)
    pool, (qd, kd, vd, od) = _views_with_high_low_word([(B, H, N, d)] * 4, td, dev)
    pool2, (ld,) = _views_with_high_low_word([(B, H, N)], torch.float32, dev)
    qd.copy_(q.to(dev)); kd.copy_(k.to(dev)); vd.copy_(v.to(dev))
    hfa.attn_fwd(qd, kd, vd, 1.0 / math.sqrt(d), out=od, lse=ld)
    torch.cuda.synchronize()
    ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(d))
    assert_close(f"bit31 {dtype} N={N} d={d}", od.float().cpu().double().numpy(), ld.cpu().double().numpy(),
                 ro, rl, dtype)
    del pool, pool2


# ---- key split (hfa_attn_fwd_split) -----------------------------------------

def run_gpu_split(q, k, v, scale, splits):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o, lse = hfa.attn_fwd(qd, kd, vd, scale, splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,H,N,splits", [(1, 2, 1000, 0), (1, 2, 1000, 2), (1, 3, 777, 3), (2, 1, 4097, 7),
                                          (1, 16, 1024, 0), (1, 1, 65, 2), (1, 1, 300, 32), (1, 4, 2048, 5)])
def test_bf16_key_split(d, B, H, N, splits):
    # Ranges of whole 64-key tiles, the last one ragged where N is; 0 = the
    # library's choice.  Checked on every row against the oracle.
    q, k, v = W.make_inputs(B, H, N, d, "bf16", seed=8000 + N + d + splits)
    name = f"bf16 split={splits} (auto {hfa.hfa_key_splits(hfa.HFA_BF16, B, H, N, d)}) B={B} H={H} N={N} d={d}"
    _log(f"[parity] {name}")
    go, gl = run_gpu_split(q, k, v, 1.0 / math.sqrt(d), splits)
    ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(d))
    assert_close(name, go, gl, ro, rl, "bf16")


def test_bf16_key_split_rising_scores():
    # The running max moves on most tiles (see test_rising_scores), and each key
    # range starts from its own first tile: the merge must rescale ranges whose
    # maxima differ by tens of log2 units.
    N, d = 1000, 128
    g = torch.Generator("cpu").manual_seed(902)
    e = torch.ones(d) / math.sqrt(d)
    slope = torch.linspace(-0.2, 1.0, N).view(N, 1)
    ramp = torch.linspace(0.0, 1.0, N).view(N, 1)
    q = (torch.randn(1, 2, N, d, generator=g) + 8.0 * slope * e).to(torch.bfloat16).contiguous()
    k = (torch.randn(1, 2, N, d, generator=g) + 20.75 * math.sqrt(d) * ramp * e).to(torch.bfloat16).contiguous()
    v = torch.randn(1, 2, N, d, generator=g).to(torch.bfloat16).contiguous()
    go, gl = run_gpu_split(q, k, v, 1.0 / math.sqrt(d), 4)
    ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(d))
    assert_close("bf16 split=4 rising", go, gl, ro, rl, "bf16")


def test_split_with_caller_workspace_and_repeat():
    # A caller workspace (leftover contents from an earlier call of another
    # shape) and two calls in a row give the same bits.
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in W.make_inputs(1, 4, 1500, 128, "bf16", seed=8100))
    need = hfa.hfa_attn_fwd_workspace_size(hfa.HFA_BF16, 1, 4, 1500, 128, 6)
    ws = torch.full((need + 4096,), 0x7f, dtype=torch.uint8, device=dev)
    o1, l1 = hfa.attn_fwd(q, k, v, splits=6, workspace=ws)
    o2, l2 = hfa.attn_fwd(q, k, v, splits=6, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = hfa.attn_fwd(q, k, v, splits=1)
    torch.cuda.synchronize()
    assert (o1.float() - o3.float()).abs().max().item() <= 2e-2
    assert (l1 - l3).abs().max().item() <= 1e-3


# ---- fp32 packed K/V (hfa_attn_fwd_split with a workspace) -----------------

def test_f32_packed_workspace_reuse():
    # One workspace, filled with junk, then used by a larger call and a smaller
    # one of another head dim (leftover tiles of the first stay behind it): each
    # call equals hfa_attn_fwd bit for bit, and the oracle.
    dev = torch.device("cuda:0")
    need = hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, 2, 8, 1500, 64, 1)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device=dev)
    for (B, H, N, d, seed) in [(2, 8, 1500, 64, 8200), (1, 3, 333, 128, 8201), (1, 1, 70, 64, 8202)]:
        assert hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, B, H, N, d, 1) <= need
        q, k, v = W.make_inputs(B, H, N, d, "f32", seed=seed, qk_mult=2.0)
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        o1, l1 = hfa.attn_fwd(qd, kd, vd, splits=1, workspace=ws)
        torch.cuda.synchronize()
        do, dl = run_gpu_direct(q, k, v, 1.0 / math.sqrt(d))
        go, gl = o1.cpu().double().numpy(), l1.cpu().double().numpy()
        assert np.array_equal(go, do) and np.array_equal(gl, dl), (B, H, N, d)
        rows = W.sample_rows(N, 24, seed=seed)
        ro, rl = run_oracle(q, k, v, 1.0 / math.sqrt(d), rows)
        assert_close(f"f32 packed reuse B={B} H={H} N={N} d={d}", go[:, :, rows], gl[:, :, rows], ro, rl, "f32")


def test_f32_default_call_packs_where_it_pays():
    # The Python entry point's default takes the library's choice: a workspace
    # (packed path) for B*H=32 N=2048 d=64, none for B*H=256 N=200; both give
    # hfa_attn_fwd's bits.
    for (B, H, N, seed) in [(4, 8, 2048, 8300), (1, 256, 200, 8301)]:
        q, k, v = W.make_inputs(B, H, N, 64, "f32", seed=seed)
        packs = hfa.hfa_attn_fwd_workspace_size(hfa.HFA_F32, B, H, N, 64, 0) > 0
        assert packs == (N == 2048)
        go, gl = run_gpu(q, k, v, 0.125)
        do, dl = run_gpu_direct(q, k, v, 0.125)
        assert np.array_equal(go, do) and np.array_equal(gl, dl)
