"""CPU checks of the arithmetic identities the fp32 attention kernel relies on.

The kernel forms S = Q K^T from int8 slices of each fp32 row and P V from
three-piece bf16 splits of P and V.  These tests replay the same steps in IEEE
fp32 (numpy, round to nearest even, as the vector unit does) and check the
claims the kernel's design rests on: slice ranges, exactness, the residual
bound, int32 headroom, and the resulting score bound.  They test the method's
numerics on the host; the GPU parity tests check the kernel itself.
"""

from __future__ import annotations

import numpy as np
import pytest

F = np.float32


def row_exponent(m: np.ndarray) -> np.ndarray:
    """e with |x| < 2^e for the row maximum m (0 for an all-zero row)."""
    _, e = np.frexp(m.astype(np.float32))
    return np.where(m == 0, 0, e).astype(np.int64)


def slice5(x: np.ndarray, e: np.ndarray):
    """The kernel's slicing of fp32 values x (rows of length d) under row exponents e.

    Returns int slices s[a] (a < 5) and the fp32 remainder after the last slice."""
    r = np.ldexp(x.astype(F), (6 - e)[..., None]).astype(F)
    out = []
    for a in range(5):
        M = F(12582912.0 / (1 << (7 * a)))
        f = (r + M).astype(F)
        byte = (f.view(np.uint32) & 0xFF).astype(np.int64)
        out.append(np.where(byte >= 128, byte - 256, byte))
        r = (r - (f - M).astype(F)).astype(F)
    return np.stack(out), r


def random_rows(rng, n, d, spread):
    mag = np.exp2(rng.uniform(-spread, spread, (n, d)))
    sign = np.where(rng.random((n, d)) < 0.5, -1.0, 1.0)
    rows = np.exp2(rng.integers(-20, 21, (n, 1)).astype(np.float64))
    return (mag * sign * rows).astype(F)


@pytest.mark.parametrize("spread", [0, 6, 11, 30])
def test_slices_in_range_and_residual_bound(spread):
    rng = np.random.default_rng(100 + spread)
    x = random_rows(rng, 400, 64, spread)
    x[0] = 0.0                                   # an all-zero row
    x[1, :] = np.float32(2.0 ** 20)              # a power-of-two row maximum
    x[2, 5] = np.float32(-(2.0 ** 24 - 1))       # a full 24-bit mantissa
    e = row_exponent(np.abs(x).max(axis=1))
    s, _ = slice5(x, e)
    assert np.abs(s).max() <= 64
    recon = np.ldexp(sum(s[a].astype(np.float64) * 2.0 ** (-7 * a) for a in range(5)), (e - 6)[:, None])
    resid = np.abs(x.astype(np.float64) - recon)
    assert np.all(resid <= np.ldexp(1.0, e - 35)[:, None])
    # every entry within 2^-11 of its row maximum is represented exactly
    near = np.abs(x) >= np.ldexp(1.0, e - 11)[:, None]
    assert np.all(resid[near] == 0.0)


def test_slices_exact_for_comparable_rows():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((512, 128)) * 4).astype(F)      # the N=2048 workload's Q, K scale
    e = row_exponent(np.abs(x).max(axis=1))
    s, _ = slice5(x, e)
    recon = np.ldexp(sum(s[a].astype(np.float64) * 2.0 ** (-7 * a) for a in range(5)), (e - 6)[:, None])
    small = np.abs(x) < np.ldexp(1.0, e - 11)[:, None]
    resid = np.abs(x.astype(np.float64) - recon)
    assert np.all(resid[~small] == 0.0)
    assert np.all(resid <= np.ldexp(1.0, e - 35)[:, None])


@pytest.mark.parametrize("d", [64, 128])
def test_int32_headroom(d):
    # Worst case: every slice at +-64.  acc_t sums the pairs with a + b = t
    # (a, b < 5, t <= 5) over d columns; acc01 = 2^7 acc_0 + acc_1 etc. must fit
    # in int32, and the fp64 combination 2^28 acc01 + 2^14 acc23 + acc45 must
    # carry at most one rounding.
    pairs = {t: sum(1 for a in range(5) for b in range(5) if a + b == t) for t in range(6)}
    acc = {t: pairs[t] * 64 * 64 * d for t in range(6)}
    assert max(acc.values()) < 2 ** 22
    for hi, lo in ((0, 1), (2, 3), (4, 5)):
        assert acc[hi] * 128 + acc[lo] < 2 ** 31
    assert (acc[2] * 128 + acc[3]) * 2 ** 14 + (acc[4] * 128 + acc[5]) < 2 ** 53


@pytest.mark.parametrize("spread", [0, 10, 24])
@pytest.mark.parametrize("d", [64, 128])
def test_score_bound(spread, d):
    # The kernel's score from the 19 slice products (a + b <= 5) against the
    # exact dot product: |ds| <= d 2^-32 max|q| max|k|.
    rng = np.random.default_rng(1000 * d + spread)
    q = random_rows(rng, 64, d, spread)
    k = random_rows(rng, 64, d, spread)
    eq = row_exponent(np.abs(q).max(axis=1))
    ek = row_exponent(np.abs(k).max(axis=1))
    sq, _ = slice5(q, eq)
    sk, _ = slice5(k, ek)
    acc = [sum(sq[a] @ sk[b].T for a in range(5) for b in range(5) if a + b == t) for t in range(6)]
    assert all(np.abs(a_).max() < 2 ** 22 for a_ in acc)
    comb = sum(a_.astype(np.float64) * 2.0 ** (-7 * t) for t, a_ in enumerate(acc))
    s = np.ldexp(comb, eq[:, None] + ek[None, :] - 12)
    exact = q.astype(np.float64) @ k.astype(np.float64).T
    bound = d * 2.0 ** -32 * np.abs(q).max(axis=1)[:, None].astype(np.float64) * np.abs(k).max(axis=1)[None, :]
    assert np.all(np.abs(s - exact) <= bound)


def bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as the fp32 value it represents."""
    u = x.astype(F).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(F)


def trunc16(x: np.ndarray) -> np.ndarray:
    return (x.astype(F).view(np.uint32) & np.uint32(0xFFFF0000)).view(F)


def test_three_piece_splits_exact():
    rng = np.random.default_rng(11)
    # V: any finite fp32, split by truncation
    v = (rng.standard_normal(200000) * np.exp2(rng.uniform(-60, 60, 200000))).astype(F)
    v = np.concatenate([v, np.array([np.finfo(F).max, -np.finfo(F).max, 1.0, -0.0], dtype=F)])
    v1 = trunc16(v)
    r = (v - v1).astype(F)
    v2 = trunc16(r)
    v3 = (r - v2).astype(F)
    assert np.array_equal(trunc16(v3), v3)               # the last piece is a bf16 value
    assert np.all(v1.astype(np.float64) + v2 + v3 == v.astype(np.float64))
    assert np.all(np.abs(v2) <= 2.0 ** -7 * np.abs(v.astype(np.float64)))
    assert np.all(np.abs(v3) <= 2.0 ** -14 * np.abs(v.astype(np.float64)))
    # P: weights in (0, 1], split by round to nearest even
    p = np.exp2(-rng.uniform(0, 40, 200000)).astype(F)
    p1 = bf16_bits_rne(p)
    r = (p - p1).astype(F)
    p2 = bf16_bits_rne(r)
    p3 = (r - p2).astype(F)
    assert np.array_equal(bf16_bits_rne(p3), p3)
    assert np.all(p1.astype(np.float64) + p2 + p3 == p.astype(np.float64))
    # the three dropped products are below 2^-21 of |p v|
    pp = rng.choice(p, 5000)
    vv = rng.choice(v[np.isfinite(v) & (np.abs(v) < 1e30)], 5000)
    P = [bf16_bits_rne(pp)]
    P.append(bf16_bits_rne((pp - P[0]).astype(F)))
    P.append((pp - P[0] - P[1]).astype(F))
    Vt = [trunc16(vv)]
    Vt.append(trunc16((vv - Vt[0]).astype(F)))
    Vt.append((vv - Vt[0] - Vt[1]).astype(F))
    dropped = sum(P[a].astype(np.float64) * Vt[b] for a in range(3) for b in range(3) if a + b >= 3)
    assert np.all(np.abs(dropped) <= 2.0 ** -21 * np.abs(pp.astype(np.float64) * vv))


# ---- the exactness check that sends a workgroup to exact fp64 scores --------

EXACT_SCORE_BOUND = 2.0 ** -22  # largest slice-score error bound kept on the int8 path


def slice_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """The int8-slice scores q . k^T the kernel forms (19 slice products, fp64 combination)."""
    eq = row_exponent(np.abs(q).max(axis=1))
    ek = row_exponent(np.abs(k).max(axis=1))
    sq, _ = slice5(q, eq)
    sk, _ = slice5(k, ek)
    acc = [sum(sq[a] @ sk[b].T for a in range(5) for b in range(5) if a + b == t) for t in range(6)]
    comb = sum(a_.astype(np.float64) * 2.0 ** (-7 * t) for t, a_ in enumerate(acc))
    return np.ldexp(comb, eq[:, None] + ek[None, :] - 12)


def pair_bound(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """|ds| <= 2^-35 (2^e_k A_q + 2^e_q A_k) + d 2^-40 2^(e_q + e_k) per (query, key), A = L1 norm."""
    d = q.shape[1]
    bq = np.where(np.abs(q).max(axis=1) > 0, np.ldexp(1.0, row_exponent(np.abs(q).max(axis=1))), 0.0)
    bk = np.ldexp(1.0, row_exponent(np.abs(k).max(axis=1)))
    aq = np.abs(q.astype(np.float64)).sum(axis=1)
    ak = np.abs(k.astype(np.float64)).sum(axis=1)
    return 2.0 ** -35 * (bk[None, :] * aq[:, None] + bq[:, None] * ak[None, :]) + d * 2.0 ** -40 * np.outer(bq, bk)


def wave_flag(q: np.ndarray, k: np.ndarray, scale: float) -> bool:
    """The kernel's check for one wave (its query rows q) after the key loop: the largest
    L1 norm and 2^e over the wave's query rows, the largest 2^e over every key row of the
    head (the workgroup stages them all), and for the keys' L1 norm the sum over the
    4-column chunks of each chunk's largest L1 norm; combined into one bound."""
    d = q.shape[1]
    mq = np.abs(q).max(axis=1)
    bq = float(np.max(np.where(mq > 0, np.ldexp(1.0, row_exponent(mq)), 0.0)))
    aq = float(np.abs(q.astype(np.float64)).sum(axis=1).max())
    bk = float(np.ldexp(1.0, row_exponent(np.abs(k).max(axis=1)).max()))
    ak = float(np.abs(k.astype(np.float64)).reshape(k.shape[0], d // 4, 4).sum(axis=2).max(axis=0).sum())
    assert ak >= np.abs(k.astype(np.float64)).sum(axis=1).max()
    bound = abs(scale) * (2.0 ** -35 * (bk * aq + bq * ak) + d * 2.0 ** -40 * bq * bk)
    return bound > EXACT_SCORE_BOUND


def outlier_rows(rng, n, d, small, big, channel):
    """Rows of N(0, small^2) entries with one outlier channel of magnitude ~big."""
    x = rng.standard_normal((n, d)) * small
    x[:, channel] = big * np.where(rng.random(n) < 0.5, -1.0, 1.0) * (1 + rng.random(n))
    return x.astype(F)


@pytest.mark.parametrize("spread", [0, 10, 24])
@pytest.mark.parametrize("d", [64, 128])
def test_pair_bound_covers_the_slice_error(spread, d):
    rng = np.random.default_rng(2000 * d + spread)
    q = random_rows(rng, 64, d, spread)
    k = random_rows(rng, 64, d, spread)
    k[:8] = outlier_rows(rng, 8, d, 1e-3, 1e4, 3)
    q[:8] = outlier_rows(rng, 8, d, 1e-3, 1e3, 7)
    err = np.abs(slice_scores(q, k) - q.astype(np.float64) @ k.astype(np.float64).T)
    assert np.all(err <= pair_bound(q, k))


@pytest.mark.parametrize("d", [64, 128])
def test_outlier_channels_take_the_exact_path(d):
    # q rows: entries ~1e-3 with an outlier channel ~1e3; k rows: entries ~1e-3
    # with another outlier channel ~1e4.  The small q entry on k's outlier
    # channel is held to 2^(10-35) only, so the slice scores miss by far more
    # than the 1e-5 budget allows -- and the check sends the workgroup to the
    # exact scores.
    rng = np.random.default_rng(d)
    scale = 1.0 / np.sqrt(d)
    q = outlier_rows(rng, 256, d, 1e-3, 1e3, 5)
    k = outlier_rows(rng, 256, d, 1e-3, 1e4, 11)
    err = scale * np.abs(slice_scores(q, k) - q.astype(np.float64) @ k.astype(np.float64).T)
    assert err.max() > 2e-5
    assert wave_flag(q, k, scale)
    # plain sequential fp32 dot products stay far below it on the same rows
    fp32 = np.zeros((q.shape[0], k.shape[0]), dtype=F)
    for c in range(d):
        fp32 = (fp32 + (q[:, c:c + 1] * k[None, :, c]).astype(F)).astype(F)
    assert scale * np.abs(fp32 - q.astype(np.float64) @ k.astype(np.float64).T).max() < 2e-5


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_evaluation_workloads_stay_on_the_int8_path(cfg):
    # With the head-wide maxima of the query statistics (at least those of any
    # wave), the fp32 evaluation workloads stay below the bound: every wave
    # keeps the int8 products.
    from fa2_fwd_amd import workloads as W

    w = W.CONFIGS[cfg]
    q, k, _ = (t.numpy() for t in W.workload_inputs(w))
    for b in range(w.B):
        for h in range(w.H):
            assert not wave_flag(q[b, h], k[b, h], w.scale), (b, h)
