"""Checks that pin the CPU oracle against facts fixed outside the oracle itself.

The pages give the definition of attention (neuralmasteryai "Hardware
Acceleration & Custom Kernels", section 2), the stable row softmax (book
chapter "Triton and kernel fusion", section "Fusion") and the online
normalisation identity (same section 2, step 2).  They print no worked numeric
example (the "Python Simulation" of section 5 is cut off), so the oracle is
pinned by closed forms, invariants, exact-rational brute force and an
independent library routine (torch fp64 softmax / logsumexp, the pages' own
parity baseline being PyTorch eager).
"""

from fractions import Fraction
import math

import numpy as np
import pytest
import torch

from fa2_fwd_amd import workloads

TIGHT = 1e-12


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _torch_ref(q, k, v, scale, rows=None):
    """Independent library routine: torch fp64 softmax(q k^T * scale) v and logsumexp."""
    q64, k64, v64 = (torch.from_numpy(np.asarray(a, dtype=np.float64)) for a in (q, k, v))
    if rows is not None:
        q64 = q64[:, :, torch.as_tensor(rows)]
    s = torch.matmul(q64, k64.transpose(-1, -2).contiguous()) * scale
    o = torch.matmul(torch.softmax(s, dim=-1), v64)
    return o.numpy(), torch.logsumexp(s, dim=-1).numpy()


def _widen_bf16(a_u16):
    return (a_u16.astype(np.uint32) << 16).view(np.float32)


# P1 -- softmax rows are stochastic: with V = identity, O is the probability matrix.
def check_p1_rows_sum_to_one(orc):
    N = d = 64
    q = _rand((1, 2, N, d), 1, 4.0)
    k = _rand((1, 2, N, d), 2, 4.0)
    v = np.broadcast_to(np.eye(N, d, dtype=np.float32), (1, 2, N, d)).copy()
    o, _ = orc.attn_fwd(q, k, v, 0.125)
    assert np.all(o >= 0.0) and np.all(o <= 1.0)
    np.testing.assert_allclose(o.sum(axis=-1), 1.0, rtol=0, atol=TIGHT)


# P2 -- identical keys: every score in a row is equal, so O is the mean of V
# and LSE = scale * q.k + ln N.
def check_p2_identical_keys(orc):
    B, H, N, d = 2, 3, 77, 16
    q = _rand((B, H, N, d), 3)
    krow = _rand((B, H, 1, d), 4)
    k = np.broadcast_to(krow, (B, H, N, d)).copy()
    v = _rand((B, H, N, d), 5)
    scale = 0.25
    o, lse = orc.attn_fwd(q, k, v, scale)
    np.testing.assert_allclose(o, np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), o.shape),
                               rtol=0, atol=TIGHT)
    qk = np.einsum("bhnd,bhd->bhn", q.astype(np.float64), krow[:, :, 0].astype(np.float64))
    np.testing.assert_allclose(lse, scale * qk + math.log(N), rtol=0, atol=1e-11)


# P3 -- constant V gives that constant for any Q, K, including peaked rows.
def check_p3_constant_v(orc):
    B, H, N, d = 1, 2, 129, 64
    q = _rand((B, H, N, d), 6, 8.0)
    k = _rand((B, H, N, d), 7, 8.0)
    c = _rand((1, 1, 1, d), 8)
    v = np.broadcast_to(c, (B, H, N, d)).copy()
    o, _ = orc.attn_fwd(q, k, v, 0.125)
    np.testing.assert_allclose(o, np.broadcast_to(c.astype(np.float64), o.shape), rtol=0, atol=TIGHT)


# P4 -- the online identity: any tiling of the keys (tile 1 is the scalar
# recurrence as stated; tiles >= N/2 are exactly two tiles split at `tile`)
# equals the one-pass definition.
def check_p4_online_equals_direct_every_split(orc):
    B, H, N, d = 1, 2, 40, 8
    q = _rand((B, H, N, d), 9, 3.0)
    k = _rand((B, H, N, d), 10, 3.0)
    v = _rand((B, H, N, d), 11)
    o_ref, lse_ref = orc.attn_fwd(q, k, v, 0.5)
    for tile in range(1, N + 1):
        o, lse = orc.attn_fwd_online(q, k, v, 0.5, tile)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=TIGHT, err_msg=f"tile={tile}")
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=TIGHT, err_msg=f"tile={tile}")


def check_p4_online_kernel_tiles_peaked(orc):
    # Peaked rows like the N=2048 workload, with the tile widths the kernels use.
    B, H, N, d = 1, 1, 300, 64
    q = _rand((B, H, N, d), 12, 4.0)
    k = _rand((B, H, N, d), 13, 4.0)
    v = _rand((B, H, N, d), 14)
    o_ref, lse_ref = orc.attn_fwd(q, k, v, 0.125)
    for tile in (16, 32, 64, 128):
        o, lse = orc.attn_fwd_online(q, k, v, 0.125, tile)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-11)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-11)


# P5 -- brute force on tiny inputs.
def check_p5_single_key(orc):
    q = _rand((1, 1, 1, 8), 15)
    k = _rand((1, 1, 1, 8), 16)
    v = _rand((1, 1, 1, 8), 17)
    o, lse = orc.attn_fwd(q, k, v, 0.3)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 0, 0].astype(np.float64))
    s = 0.3 * float(np.dot(q[0, 0, 0].astype(np.float64), k[0, 0, 0].astype(np.float64)))
    assert abs(lse[0, 0, 0] - s) < TIGHT


def check_p5_two_keys_logistic(orc):
    q = _rand((1, 1, 2, 4), 18)
    k = _rand((1, 1, 2, 4), 19)
    v = _rand((1, 1, 2, 4), 20)
    scale = 0.7
    o, lse = orc.attn_fwd(q, k, v, scale)
    q64, k64, v64 = (a[0, 0].astype(np.float64) for a in (q, k, v))
    for i in range(2):
        s0, s1 = scale * q64[i] @ k64[0], scale * q64[i] @ k64[1]
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))  # logistic closed form
        np.testing.assert_allclose(o[0, 0, i], p0 * v64[0] + (1 - p0) * v64[1], rtol=0, atol=TIGHT)
        assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) < TIGHT


def check_p5_exact_rational(orc):
    # d = 1, q = 1, integer keys, scale = ln 2: p_j is proportional to 2^k_j,
    # so O = sum 2^k_j v_j / sum 2^k_j is an exact rational for dyadic v.
    keys = [-7, 3, 0, 12, 12, -20, 5, 1, 9]
    vals = [Fraction(n, 8) for n in (3, -5, 11, 1, -2, 7, 0, 13, -9)]
    N = len(keys)
    q = np.ones((1, 1, N, 1), np.float32)
    k = np.asarray(keys, np.float32).reshape(1, 1, N, 1)
    v = np.asarray([float(x) for x in vals], np.float32).reshape(1, 1, N, 1)
    o, lse = orc.attn_fwd(q, k, v, math.log(2.0))
    den = sum(Fraction(2) ** kj for kj in keys)
    num = sum(Fraction(2) ** kj * vj for kj, vj in zip(keys, vals))
    exact_o = float(num / den)
    exact_lse = math.log(2.0) * math.log2(float(den))
    np.testing.assert_allclose(o[0, 0, :, 0], exact_o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], exact_lse, rtol=0, atol=1e-12)


# P6 -- scale 0: uniform weights, O = mean V, LSE = ln N.
def check_p6_zero_scale(orc):
    B, H, N, d = 1, 2, 50, 16
    q, k, v = _rand((B, H, N, d), 21), _rand((B, H, N, d), 22), _rand((B, H, N, d), 23)
    o, lse = orc.attn_fwd(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.astype(np.float64).mean(axis=2, keepdims=True), o.shape),
                               rtol=0, atol=TIGHT)
    np.testing.assert_allclose(lse, math.log(N), rtol=0, atol=TIGHT)


# P7 -- adding one vector c to every key shifts every score of row i by
# scale * q_i.c: O is unchanged and LSE moves by exactly that amount.
def check_p7_key_shift(orc):
    rng = np.random.default_rng(24)
    B, H, N, d = 1, 1, 64, 16
    q = rng.integers(-3, 4, (B, H, N, d)).astype(np.float32)
    k = rng.integers(-3, 4, (B, H, N, d)).astype(np.float32)
    v = _rand((B, H, N, d), 25)
    c = rng.integers(-5, 6, (1, 1, 1, d)).astype(np.float32)
    scale = 0.25
    o0, lse0 = orc.attn_fwd(q, k, v, scale)
    o1, lse1 = orc.attn_fwd(q, k + c, v, scale)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=TIGHT)
    shift = scale * np.einsum("bhnd,d->bhn", q.astype(np.float64), c[0, 0, 0].astype(np.float64))
    np.testing.assert_allclose(lse1, lse0 + shift, rtol=0, atol=1e-11)


# P8 -- a joint permutation of the keys and values changes nothing; a
# permutation of the queries permutes the output rows.
def check_p8_permutations(orc):
    B, H, N, d = 1, 2, 70, 16
    q, k, v = _rand((B, H, N, d), 26, 2.0), _rand((B, H, N, d), 27, 2.0), _rand((B, H, N, d), 28)
    o, lse = orc.attn_fwd(q, k, v, 0.25)
    perm = np.random.default_rng(29).permutation(N)
    o_kv, lse_kv = orc.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.25)
    np.testing.assert_allclose(o_kv, o, rtol=0, atol=TIGHT)
    np.testing.assert_allclose(lse_kv, lse, rtol=0, atol=TIGHT)
    o_q, lse_q = orc.attn_fwd(q[:, :, perm], k, v, 0.25)
    np.testing.assert_allclose(o_q, o[:, :, perm], rtol=0, atol=TIGHT)
    np.testing.assert_allclose(lse_q, lse[:, :, perm], rtol=0, atol=TIGHT)


# P9 -- cross-check against torch's fp64 softmax / logsumexp on the five
# evaluation shapes (whole for the two small ones, sampled rows otherwise).
def check_p9_library_crosscheck(orc, cfg):
    w = workloads.CONFIGS[cfg]
    q, k, v = workloads.workload_inputs(w)
    qa, ka, va = (workloads.to_oracle_array(t) for t in (q, k, v))
    rows = None if cfg <= 2 else workloads.sample_rows(w.N, 8, seed=100 + cfg)
    o, lse = orc.attn_fwd(qa, ka, va, w.scale, rows=rows)
    if w.dtype == "bf16":
        qa, ka, va = (_widen_bf16(a) for a in (qa, ka, va))
    o_t, lse_t = _torch_ref(qa, ka, va, w.scale, rows)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-11)


# P10 -- one key leading every other score by > 40: O is that key's value row
# to within e^-40 relative weight.
def check_p10_peaked_limit(orc):
    B, H, N, d = 1, 1, 33, 16
    rng = np.random.default_rng(30)
    q = np.zeros((B, H, N, d), np.float32)
    q[..., 0] = 20.0
    k = (rng.standard_normal((B, H, N, d)) * 0.1).astype(np.float32)
    k[0, 0, 17, 0] = 20.0
    v = _rand((B, H, N, d), 31)
    o, lse = orc.attn_fwd(q, k, v, 0.25)
    bound = N * math.exp(-40.0) * float(np.abs(v).max())
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, 17].astype(np.float64), (N, d)),
                               rtol=0, atol=bound)


def check_rejects_bad_arguments(orc):
    q = _rand((1, 1, 4, 4), 32)
    with pytest.raises(ValueError):
        orc.attn_fwd(q, q, q, float("nan"))
    with pytest.raises(ValueError):
        orc.attn_fwd(q, q, q, 1.0, rows=[0, 4])
    with pytest.raises(ValueError):
        orc.attn_fwd_online(q, q, q, 1.0, 0)
    with pytest.raises(ValueError):
        orc.attn_fwd(q.astype(np.float64), q, q, 1.0)


def check_bf16_widening_is_exact(orc):
    # bf16 inputs reach the oracle as bit patterns; check the widened values
    # against torch's own bf16 -> fp64 conversion.
    q, k, v = workloads.make_inputs(1, 1, 64, 16, "bf16", 33)
    qa, ka, va = (workloads.to_oracle_array(t) for t in (q, k, v))
    o, lse = orc.attn_fwd(qa, ka, va, 0.25)
    o_t, lse_t = _torch_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.25)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-13)


def check_p9_small_sampled(orc):
    # Same library cross-check on a small bf16 problem with a row sample, so
    # that the row-selection bookkeeping is exercised quickly.
    q, k, v = workloads.make_inputs(1, 2, 200, 32, "bf16", 34)
    qa, ka, va = (workloads.to_oracle_array(t) for t in (q, k, v))
    rows = np.asarray([0, 5, 63, 64, 150, 199], np.int64)
    o, lse = orc.attn_fwd(qa, ka, va, 0.2, rows=rows)
    o_t, lse_t = _torch_ref(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.2, rows)
    np.testing.assert_allclose(o, o_t, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_t, rtol=0, atol=1e-12)


ALL_CHECKS = [
    check_p1_rows_sum_to_one,
    check_p2_identical_keys,
    check_p3_constant_v,
    check_p4_online_equals_direct_every_split,
    check_p4_online_kernel_tiles_peaked,
    check_p5_single_key,
    check_p5_two_keys_logistic,
    check_p5_exact_rational,
    check_p6_zero_scale,
    check_p7_key_shift,
    check_p8_permutations,
    check_p10_peaked_limit,
    check_rejects_bad_arguments,
    check_bf16_widening_is_exact,
    check_p9_small_sampled,
    lambda orc: check_p9_library_crosscheck(orc, 1),
]


def check_golden_exact_rational(orc):
    # Stored hand derivation (tests/golden/exact_rational.txt).
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "exact_rational.txt")
    fields = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            fields[key] = [float(x) for x in vals]
    keys, vals = fields["keys"], fields["values"]
    N = len(keys)
    q = np.ones((1, 1, N, 1), np.float32)
    k = np.asarray(keys, np.float32).reshape(1, 1, N, 1)
    v = np.asarray(vals, np.float32).reshape(1, 1, N, 1)
    o, lse = orc.attn_fwd(q, k, v, math.log(2.0))
    exact_o = fields["o_num"][0] / fields["o_den"][0]
    exact_lse = math.log(fields["lse_arg_num"][0] / fields["lse_arg_den"][0])
    np.testing.assert_allclose(o[0, 0, :, 0], exact_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], exact_lse, rtol=0, atol=1e-14)


ALL_CHECKS.append(check_golden_exact_rational)


# ---- standalone row softmax (book chapter "Triton and kernel fusion",
# section "Fusion": subtract the row max, exponentiate, sum, divide; stretch
# exercise: rows wider than one block by a running max and sum).

def _srand(shape, seed, scale=1.0):
    return _rand(shape, seed, scale)


# S1 -- every row is a probability vector.
def check_s1_softmax_rows_stochastic(orc):
    x = _srand((6, 1000), 21, 10.0)
    y = orc.softmax_rows(x)
    assert np.all(y >= 0) and np.all(y <= 1)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-13)


# S2 -- a constant row gives the uniform distribution.
def check_s2_softmax_constant_row(orc):
    x = np.full((3, 777), 3.25, np.float32)
    x[1] = -40.0
    np.testing.assert_allclose(orc.softmax_rows(x), 1.0 / 777, rtol=1e-14, atol=0)


# S3 -- two distinct values: C-1 copies of a and one b, closed form
# y_b = 1 / (1 + (C-1) e^(a-b)), y_a = e^(a-b) y_b.
def check_s3_softmax_two_values(orc):
    C, a, b, pos = 301, 1.5, 4.0, 137
    x = np.full((1, C), a, np.float32)
    x[0, pos] = b
    y = orc.softmax_rows(x)[0]
    yb = 1.0 / (1.0 + (C - 1) * math.exp(a - b))
    np.testing.assert_allclose(y[pos], yb, rtol=1e-14)
    np.testing.assert_allclose(np.delete(y, pos), math.exp(a - b) * yb, rtol=1e-14)


# S4 -- shifting a row by a constant changes nothing (exact fp32 shift).
def check_s4_softmax_shift_invariance(orc):
    rng = np.random.default_rng(24)
    x = (rng.integers(-80, 80, size=(4, 513)) / 8.0).astype(np.float32)
    y0 = orc.softmax_rows(x)
    y1 = orc.softmax_rows((x + np.float32(37.0)).astype(np.float32))
    np.testing.assert_allclose(y1, y0, rtol=0, atol=1e-15)


# S5 -- magnitudes where exp overflows without the max subtraction.
def check_s5_softmax_large_magnitudes(orc):
    x = (_srand((3, 400), 25, 30.0) + np.float32(750.0)).astype(np.float32)
    y = orc.softmax_rows(x)
    assert np.all(np.isfinite(y))
    from scipy.special import softmax as sp_softmax
    np.testing.assert_allclose(y, sp_softmax(x.astype(np.float64), axis=1), rtol=0, atol=1e-14)


# S6 -- independent library routine, rows of the chapter's width (32000) and
# wider than its one-block limit (65536).  The fp64 row sums of C terms carry
# up to about C * 2^-53 relative rounding in either routine: rtol 5e-13.
def check_s6_softmax_library_crosscheck(orc):
    from scipy.special import softmax as sp_softmax
    for shape, seed in (((3, 32000), 26), ((2, 70001), 27)):
        x = _srand(shape, seed, 6.0)
        np.testing.assert_allclose(orc.softmax_rows(x), sp_softmax(x.astype(np.float64), axis=1),
                                   rtol=5e-13, atol=0)


# S7 -- the running (max, sum) identity over any chunking equals the definition.
def check_s7_softmax_online_equals_direct(orc):
    x = _srand((3, 1000), 28, 12.0)
    y = orc.softmax_rows(x)
    for chunk in (1, 5, 64, 999, 1000, 4096):
        # the rescale factors add a few roundings: agreement to 1e-13 relative
        np.testing.assert_allclose(orc.softmax_rows_online(x, chunk), y, rtol=1e-13, atol=0)


# S8 -- a row sample gives exactly those rows of the full result.
def check_s8_softmax_sampled_rows(orc):
    x = _srand((9, 300), 29, 5.0)
    full = orc.softmax_rows(x)
    rows = [7, 0, 8, 3]
    np.testing.assert_array_equal(orc.softmax_rows(x, rows=rows), full[rows])


# S9 -- one element g ~ 60 above the rest (g the gap in the fp32 data):
# one-hot within (C-1) e^-g, every other weight <= e^-g.
def check_s9_softmax_dominance(orc):
    C = 1000
    x = _srand((1, C), 30, 1.0)
    x[0, 321] = x[0].max() + 60.0
    gap = float(x[0, 321]) - float(np.delete(x[0], 321).max())
    y = orc.softmax_rows(x)[0]
    assert abs(y[321] - 1.0) <= (C - 1) * math.exp(-gap)
    assert np.delete(y, 321).max() <= math.exp(-gap) * (1 + 1e-12)


def check_s10_softmax_rejects_bad_arguments(orc):
    x = _srand((2, 10), 31)
    bad = x.copy()
    bad[1, 3] = np.nan
    with pytest.raises(ValueError):
        orc.softmax_rows(bad)
    with pytest.raises(ValueError):
        orc.softmax_rows(x, rows=[0, 2])
    with pytest.raises(ValueError):
        orc.softmax_rows_online(x, 0)


SOFTMAX_CHECKS = [
    check_s1_softmax_rows_stochastic,
    check_s2_softmax_constant_row,
    check_s3_softmax_two_values,
    check_s4_softmax_shift_invariance,
    check_s5_softmax_large_magnitudes,
    check_s6_softmax_library_crosscheck,
    check_s7_softmax_online_equals_direct,
    check_s8_softmax_sampled_rows,
    check_s9_softmax_dominance,
    check_s10_softmax_rejects_bad_arguments,
]
ALL_CHECKS.extend(SOFTMAX_CHECKS)


# ---- RMS normalisation (TritonForge "Fused RMSNorm" card: RMSNorm(x) = x /
# sqrt(sum_i x_i^2 / d + eps) * gamma; book chapter "Triton and kernel
# fusion", section "Fused residual add + RMSNorm": s = x + residual, added
# in fp32 by that section's kernel, is normalised and returned as well).

def _golden_rmsnorm():
    import os

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rmsnorm_exact.txt")
    fields = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            key, *vals = line.split()
            fields[key] = [float(v) for v in vals]
    return fields


def _row(vals):
    return np.asarray(vals, np.float32).reshape(1, -1)


# R1 -- the hand-derived rows of tests/golden/rmsnorm_exact.txt.
def check_r1_rmsnorm_golden(orc):
    g = _golden_rmsnorm()
    y, s = orc.rmsnorm(_row(g["a_x"]), np.asarray(g["a_w"], np.float32), g["a_eps"][0])
    np.testing.assert_allclose(y[0], np.asarray(g["a_y_over_sqrt2"]) * math.sqrt(2.0), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(s[0], g["a_x"])
    y, _ = orc.rmsnorm(_row(g["b_x"]), np.asarray(g["b_w"], np.float32), g["b_eps"][0])
    np.testing.assert_allclose(y[0], g["b_y"], rtol=1e-15, atol=0)
    y, s = orc.rmsnorm(_row(g["c_x"]), np.asarray(g["c_w"], np.float32), g["c_eps"][0], residual=_row(g["c_r"]))
    np.testing.assert_array_equal(s[0], g["c_s"])
    rms = math.sqrt(g["c_rms_sq_num"][0] / g["c_rms_sq_den"][0])
    np.testing.assert_allclose(y[0], np.asarray(g["c_s"]) / rms, rtol=1e-15, atol=0)


# R2 -- with unit weight the output's mean square is ms / (ms + eps), ms the
# input's mean square (computed here by numpy): pins the 1/d, eps inside the root.
def check_r2_rmsnorm_output_mean_square(orc):
    for C, eps in ((1, 0.25), (7, 0.5), (512, 0.5), (4097, 2.0)):
        x = _rand((5, C), 40 + C, 1.0)
        y, _ = orc.rmsnorm(x, np.ones(C, np.float32), eps)
        ms = np.mean(x.astype(np.float64) ** 2, axis=1)
        np.testing.assert_allclose(np.mean(y ** 2, axis=1), ms / (ms + eps), rtol=1e-13, atol=0)


# R3 -- homogeneity: y(a x; a^2 eps) = y(x; eps), and with eps = 0 the output is
# invariant to scaling the row (a a power of two, so a x is exact in fp32).
def check_r3_rmsnorm_homogeneity(orc):
    x = _rand((4, 300), 43, 1.0)
    w = _rand((300,), 44, 1.0)
    for a in (4.0, 0.125):
        y1, _ = orc.rmsnorm(x, w, 0.3)
        y2, _ = orc.rmsnorm((x * a).astype(np.float32), w, 0.3 * a * a)
        np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-15)
        y1, _ = orc.rmsnorm(x, w, 0.0)
        y2, _ = orc.rmsnorm((x * a).astype(np.float32), w, 0.0)
        np.testing.assert_allclose(y2, y1, rtol=1e-13, atol=1e-15)


# R4 -- independent library routine: torch's fp64 rms_norm (the pages' parity
# baseline being PyTorch eager), over several widths.
def check_r4_rmsnorm_library_crosscheck(orc):
    import torch.nn.functional as F

    for C in (1, 7, 512, 2048, 4097):
        x = _rand((6, C), 50 + C, 3.0)
        w = (1.0 + 0.1 * _rand((C,), 60 + C)).astype(np.float32)
        y, _ = orc.rmsnorm(x, w, 1e-6)
        ref = F.rms_norm(torch.from_numpy(x.astype(np.float64)), (C,), torch.from_numpy(w.astype(np.float64)),
                         eps=1e-6).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


# R5 -- the weight multiplies column by column: y(w) = y(1) * w, and permuting
# the columns of x and w permutes the output's columns.
def check_r5_rmsnorm_weight_columns(orc):
    C = 257
    x = _rand((3, C), 61, 2.0)
    w = _rand((C,), 62, 1.0)
    y1, _ = orc.rmsnorm(x, np.ones(C, np.float32), 1e-3)
    yw, _ = orc.rmsnorm(x, w, 1e-3)
    np.testing.assert_allclose(yw, y1 * w.astype(np.float64), rtol=1e-14, atol=1e-15)
    perm = np.random.default_rng(63).permutation(C)
    yp, _ = orc.rmsnorm(np.ascontiguousarray(x[:, perm]), np.ascontiguousarray(w[perm]), 1e-3)
    np.testing.assert_allclose(yp, yw[:, perm], rtol=1e-14, atol=1e-15)


# R6 -- the residual is added in fp32 (numpy float32 addition, IEEE round to
# nearest even), and the output is the normalisation of that sum.
def check_r6_rmsnorm_residual_fp32_sum(orc):
    x = _rand((4, 1000), 64, 1.0)
    r = _rand((4, 1000), 65, 1e-3)
    w = _rand((1000,), 66, 1.0)
    s32 = x + r  # float32 + float32 in numpy is one fp32 add
    assert s32.dtype == np.float32
    y, s = orc.rmsnorm(x, w, 1e-6, residual=r)
    np.testing.assert_array_equal(s, s32.astype(np.float64))
    assert np.any(s32.astype(np.float64) != x.astype(np.float64) + r.astype(np.float64))
    y_ref, s_ref = orc.rmsnorm(s32, w, 1e-6)
    np.testing.assert_array_equal(y, y_ref)
    np.testing.assert_array_equal(s_ref, s)


# R7 -- bf16 inputs are widened exactly: the result equals that of the widened
# fp32 values (residual included).
def check_r7_rmsnorm_bf16_widening(orc):
    rng = np.random.default_rng(67)
    xb = rng.integers(0x3c00, 0x4100, size=(3, 129)).astype(np.uint16)
    xb[:, ::2] |= 0x8000
    rb = rng.integers(0x3a00, 0x4000, size=(3, 129)).astype(np.uint16)
    wb = rng.integers(0x3f00, 0x3fa0, size=(129,)).astype(np.uint16)
    y, s = orc.rmsnorm(xb, wb, 1e-5, residual=rb)
    y32, s32 = orc.rmsnorm(_widen_bf16(xb), _widen_bf16(wb), 1e-5, residual=_widen_bf16(rb))
    np.testing.assert_array_equal(y, y32)
    np.testing.assert_array_equal(s, s32)


# R8 -- a row subset equals the same rows of the full result.
def check_r8_rmsnorm_sampled_rows(orc):
    x = _rand((9, 100), 68, 1.0)
    r = _rand((9, 100), 69, 1.0)
    w = _rand((100,), 70, 1.0)
    y, s = orc.rmsnorm(x, w, 1e-6, residual=r)
    rows = [8, 0, 5]
    ys, ss = orc.rmsnorm(x, w, 1e-6, residual=r, rows=rows)
    np.testing.assert_array_equal(ys, y[rows])
    np.testing.assert_array_equal(ss, s[rows])


# R9 -- one column: y = s / sqrt(s^2 + eps) * w, and sign(s) * w when eps = 0.
def check_r9_rmsnorm_single_column(orc):
    x = np.asarray([[3.0], [-0.5], [1e-3]], np.float32)
    w = np.asarray([2.0], np.float32)
    y, _ = orc.rmsnorm(x, w, 0.0)
    np.testing.assert_allclose(y[:, 0], [2.0, -2.0, 2.0], rtol=1e-15, atol=0)
    y, _ = orc.rmsnorm(x, w, 1.0)
    xd = x[:, 0].astype(np.float64)
    np.testing.assert_allclose(y[:, 0], 2.0 * xd / np.sqrt(xd * xd + 1.0), rtol=1e-15, atol=0)


# R10 -- invalid arguments are rejected.
def check_r10_rmsnorm_rejects_bad_arguments(orc):
    x = _rand((2, 10), 71)
    w = np.ones(10, np.float32)
    bad = x.copy()
    bad[1, 3] = np.inf
    with pytest.raises(ValueError):
        orc.rmsnorm(bad, w, 1e-6)
    with pytest.raises(ValueError):
        orc.rmsnorm(x, w, -1e-6)
    with pytest.raises(ValueError):
        orc.rmsnorm(np.zeros((2, 10), np.float32), w, 0.0)
    with pytest.raises(ValueError):
        orc.rmsnorm(x, w, 1e-6, rows=[0, 2])


RMSNORM_CHECKS = [
    check_r1_rmsnorm_golden,
    check_r2_rmsnorm_output_mean_square,
    check_r3_rmsnorm_homogeneity,
    check_r4_rmsnorm_library_crosscheck,
    check_r5_rmsnorm_weight_columns,
    check_r6_rmsnorm_residual_fp32_sum,
    check_r7_rmsnorm_bf16_widening,
    check_r8_rmsnorm_sampled_rows,
    check_r9_rmsnorm_single_column,
    check_r10_rmsnorm_rejects_bad_arguments,
]
ALL_CHECKS.extend(RMSNORM_CHECKS)
