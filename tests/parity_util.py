"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 CPU oracle on the same host bytes, and compare within the stated tolerances.

Tolerances:
  fp32 -- max |gpu - oracle| <= 1e-5 on O and on LSE (the TritonForge page's
          parity bound, atol = 1e-5, taken against the exact fp64 result).
          Where half an fp32 ulp of the exact value exceeds 1e-5 (|LSE| >= 256)
          no fp32 output can meet 1e-5; there the bound is half an ulp + 1e-6,
          i.e. correct rounding up to 1e-6 of computation error;
  bf16 -- |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| element-wise on O and LSE.
"""

import numpy as np
import torch

import fa2_fwd_amd as hfa
import oracle
from fa2_fwd_amd import workloads as W

F32_ATOL = 1e-5
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def _log(msg):
    print(msg, flush=True)


def run_gpu(q, k, v, scale, splits=0):
    """The Python entry point.  fp32 with splits=1: the packed path (a workspace
    in which one kernel formats K and V once per call) whatever the shape."""
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    o, lse = hfa.attn_fwd(qd, kd, vd, scale, splits=splits)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def run_gpu_direct(q, k, v, scale):
    """hfa_attn_fwd itself through the C ABI (fp32: every workgroup formats its
    own K and V tiles, no workspace)."""
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev).contiguous() for t in (q, k, v))
    B, H, N, d = qd.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    code = hfa.HFA_F32 if qd.dtype == torch.float32 else hfa.HFA_BF16
    st = hfa.hfa_attn_fwd(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
                          float(scale), code, torch.cuda.current_stream(dev).cuda_stream)
    assert st == hfa.HFA_OK, hfa.hfa_status_str(st)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def run_oracle(q, k, v, scale, rows=None):
    # The C ABI takes the scale as fp32: the oracle gets that same value, so
    # both sides compute the same function (1/sqrt(128) moves by 1.7e-8
    # relative when rounded, 3.6e-6 on a log-sum-exp of 200).
    return oracle.attn_fwd(*(W.to_oracle_array(t) for t in (q, k, v)), float(np.float32(scale)), rows=rows)


def f32_tolerance(ref):
    """1e-5, or half an fp32 ulp of the exact value + 1e-6 where that is larger."""
    half_ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64) / 2
    return np.maximum(F32_ATOL, half_ulp + 1e-6)


def assert_close(name, got_o, got_lse, ref_o, ref_lse, dtype):
    assert np.isfinite(got_o).all(), f"{name}: non-finite O"
    assert np.isfinite(got_lse).all(), f"{name}: non-finite LSE"
    report = []
    for what, g, r in (("O", got_o, ref_o), ("LSE", got_lse, ref_lse)):
        err = np.abs(g - r)
        tol = f32_tolerance(r) if dtype == "f32" else BF16_ATOL + BF16_RTOL * np.abs(r)
        excess = err - tol
        worst = np.unravel_index(np.argmax(excess), excess.shape)
        report.append(f"max|d{what}|={err.max():.3e}")
        assert excess.max() <= 0, f"{name}: {what} off by {err[worst]:.3e} (tol {np.broadcast_to(tol, err.shape)[worst]:.3e}) at {worst}"
    _log(f"[parity] {name}: " + " ".join(report))


def check_case(name, q, k, v, scale, dtype, rows=None):
    """GPU against the oracle.  fp32 runs both paths, the packed one (Python
    entry point, with a workspace) and hfa_attn_fwd without one: each meets the
    tolerance, and the two agree bit for bit (the packing kernel leaves the same
    bytes in LDS as the in-kernel formatting)."""
    _log(f"[parity] {name}")
    go, gl = run_gpu(q, k, v, scale, splits=1 if dtype == "f32" else 0)
    ro, rl = run_oracle(q, k, v, scale, rows)
    if dtype == "f32":
        do, dl = run_gpu_direct(q, k, v, scale)
        assert np.array_equal(go, do) and np.array_equal(gl, dl), f"{name}: packed and direct fp32 paths differ"
    if rows is not None:
        go, gl = go[:, :, rows], gl[:, :, rows]
    assert_close(name, go, gl, ro, rl, dtype)
    return go, gl
