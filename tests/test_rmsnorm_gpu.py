"""GPU parity of hfa_rmsnorm against the fp64 CPU oracle.

Bars (readings of the pages):
  * the sum s = x + residual is one fp32 add on both sides, so residual_out is
    compared bit for bit (fp32), or against the oracle's sum rounded to bf16
    (nearest even, torch's conversion) for bf16;
  * fp32 y: |gpu - oracle| <= 1e-5 + 1e-5 |oracle| per element (the TritonForge
    page's parity claim, atol 1e-5, with torch.allclose's default rtol);
  * bf16 y: |gpu - oracle| <= 2^-8 |oracle| (1 + 2^-10) + 1e-6: one rounding to
    bf16 (at most half an ulp, 2^-8 relative) of an fp32 value.
Shapes cover every row-group size of the dispatch, ragged widths and row
counts, the 65536-column limit, unaligned buffers (the element-wise path),
in-place use, large and small magnitudes, several eps, and the benchmark
workloads at full size (the sum everywhere, the output on sampled rows).
"""

import numpy as np
import pytest
import torch

import fa2_fwd_amd as hfa
from fa2_fwd_amd import workloads as W
import oracle

pytestmark = pytest.mark.gpu

F32_ATOL = 1e-5
F32_RTOL = 1e-5
BF16_RTOL = 2.0 ** -8 * (1 + 2.0 ** -10)
BF16_ATOL = 1e-6


def _np(t):
    """Host numpy view for the oracle: float32, or uint16 bf16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def _inputs(rows, cols, dtype, seed, residual=True, xscale=1.0):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(rows, cols, generator=g) * xscale
    r = torch.randn(rows, cols, generator=g) * xscale if residual else None
    w = 1.0 + 0.1 * torch.randn(cols, generator=g)
    return x.to(dtype), (r.to(dtype) if residual else None), w.to(dtype)


def _check(name, x, r, w, eps, y_dev, s_dev, rows=None):
    """Compare GPU outputs (device tensors, full) with the oracle on `rows` (all if None)."""
    print(f"[rmsnorm] {name}", flush=True)
    ref_y, ref_s = oracle.rmsnorm(_np(x), _np(w), eps, residual=None if r is None else _np(r), rows=rows)
    y = y_dev.float().cpu().double().numpy()
    if rows is not None:
        y = y[rows]
    assert np.isfinite(y).all(), f"{name}: non-finite output"
    err = np.abs(y - ref_y)
    if x.dtype == torch.float32:
        bound = F32_ATOL + F32_RTOL * np.abs(ref_y)
    else:
        bound = BF16_ATOL + BF16_RTOL * np.abs(ref_y)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    print(f"[rmsnorm] {name}: max|d|={err.max():.3e}", flush=True)
    assert np.all(err <= bound), f"{name}: y off by {err[worst]:.3e} at {worst} (bound {bound[worst]:.3e})"
    if s_dev is not None:
        s = s_dev.cpu()
        if rows is not None:
            s = s[torch.as_tensor(rows)]
        expect = torch.from_numpy(ref_s).to(torch.float32).to(x.dtype)
        assert torch.equal(s.view(torch.int16) if x.dtype == torch.bfloat16 else s,
                           expect.view(torch.int16) if x.dtype == torch.bfloat16 else expect), f"{name}: sum differs"


F32_COLS = [1, 3, 4, 255, 256, 257, 512, 1000, 1023, 1024, 2048, 4095, 4096, 8192, 12289, 32768, 32771, 65536]
BF16_COLS = [1, 7, 8, 511, 512, 513, 2048, 4096, 8192, 8200, 16384, 32768, 40000, 65536]


@pytest.mark.parametrize("residual", [True, False], ids=["res", "nores"])
@pytest.mark.parametrize("dtype,cols", [(torch.float32, c) for c in F32_COLS] + [(torch.bfloat16, c) for c in BF16_COLS],
                         ids=lambda v: str(v).replace("torch.", ""))
def test_rmsnorm_widths(dtype, cols, residual):
    rows = 37 if cols <= 4096 else 5
    x, r, w = _inputs(rows, cols, dtype, seed=cols * 3 + (1 if residual else 0), residual=residual)
    xd, wd = x.cuda(), w.cuda()
    if residual:
        y, s = hfa.rmsnorm(xd, wd, 1e-6, residual=r.cuda())
    else:
        y, s = hfa.rmsnorm(xd, wd, 1e-6), None
    torch.cuda.synchronize()
    _check(f"{dtype} {rows}x{cols} res={residual}", x, r, w, 1e-6, y, s)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_rmsnorm_in_place(dtype):
    x, r, w = _inputs(9, 3000, dtype, seed=11)
    wd = w.cuda()
    # y over x, the sum over the residual
    xd, rd = x.cuda(), r.cuda()
    y, s = hfa.rmsnorm(xd, wd, 1e-6, residual=rd, out=xd, residual_out=rd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr() and s.data_ptr() == rd.data_ptr()
    _check(f"{dtype} y->x, s->residual", x, r, w, 1e-6, y, s)
    # the sum over x (the residual stream updated in place), y over the residual
    xd, rd = x.cuda(), r.cuda()
    y, s = hfa.rmsnorm(xd, wd, 1e-6, residual=rd, out=rd, residual_out=xd)
    torch.cuda.synchronize()
    _check(f"{dtype} y->residual, s->x", x, r, w, 1e-6, y, s)
    # no residual, y over x
    xd = x.cuda()
    y = hfa.rmsnorm(xd, wd, 1e-6, out=xd)
    torch.cuda.synchronize()
    _check(f"{dtype} no residual, y->x", x, None, w, 1e-6, y, None)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("cols", [512, 4096, 32768])
def test_rmsnorm_unaligned(dtype, cols):
    rows = 6
    x, r, w = _inputs(rows, cols, dtype, seed=cols + 5)
    n = rows * cols

    def shifted(t, k):
        buf = torch.zeros(t.numel() + 8, dtype=dtype, device="cuda")
        v = buf[k:k + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    xd, rd, wd = shifted(x, 1), shifted(r, 3), shifted(w, 1)
    y, s = shifted(torch.zeros(rows, cols, dtype=dtype), 1), shifted(torch.zeros(rows, cols, dtype=dtype), 2)
    assert xd.data_ptr() % 16 != 0 and n == xd.numel()
    hfa.rmsnorm(xd, wd, 1e-6, residual=rd, out=y, residual_out=s)
    torch.cuda.synchronize()
    _check(f"{dtype} unaligned {rows}x{cols}", x, r, w, 1e-6, y, s)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("xscale,eps", [(1e15, 1e-6), (1e-15, 1e-6), (1.0, 1e-2), (0.1, 10.0), (1e-3, 1e-6)])
def test_rmsnorm_magnitudes_and_eps(dtype, xscale, eps):
    x, r, w = _inputs(8, 2048, dtype, seed=17, xscale=xscale)
    y, s = hfa.rmsnorm(x.cuda(), w.cuda(), eps, residual=r.cuda())
    torch.cuda.synchronize()
    _check(f"{dtype} scale={xscale:g} eps={eps:g}", x, r, w, eps, y, s)


def test_rmsnorm_zero_rows_and_spike():
    # an all-zero row gives y = 0 (eps > 0); a single spike gives sqrt(C) * w there
    cols = 1024
    x = torch.zeros(3, cols)
    x[1, 17] = 3.0
    x[2] = torch.randn(cols, generator=torch.Generator().manual_seed(5))
    w = torch.ones(cols)
    y = hfa.rmsnorm(x.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    _check("zero row and spike", x, None, w, 1e-6, y, None)
    assert torch.count_nonzero(y[0]).item() == 0


@pytest.mark.parametrize("cfg", sorted(W.RMSNORM_CONFIGS))
def test_rmsnorm_benchmark_workloads(cfg):
    """Full-size workloads as the benchmark launches them: the sum checked on every element
    against torch's fp32 addition on the host, the output on sampled rows against the oracle."""
    wl = W.RMSNORM_CONFIGS[cfg]
    x, r, w = wl.inputs()
    print(f"[rmsnorm] {wl.describe()}", flush=True)
    y, s = hfa.rmsnorm(x.cuda(), w.cuda(), wl.eps, residual=r.cuda())
    torch.cuda.synchronize()
    s_host = (x.float() + r.float()).to(x.dtype)
    s_gpu = s.cpu()
    if x.dtype == torch.bfloat16:
        assert torch.equal(s_gpu.view(torch.int16), s_host.view(torch.int16))
    else:
        assert torch.equal(s_gpu, s_host)
    rng = np.random.default_rng(cfg)
    rows = np.unique(np.r_[0, wl.rows // 2, wl.rows - 1, rng.integers(0, wl.rows, 45)])
    _check(wl.describe(), x, r, w, wl.eps, y, None, rows=rows)


@pytest.mark.parametrize("rows,cols,dtype", [(131072, 512, torch.float32), (8192, 8192, torch.float32),
                                             (16384, 8192, torch.bfloat16)])
def test_rmsnorm_bitwise_repeatable(rows, cols, dtype):
    # three runs of the residual-add + RMSNorm kernel agree bit for bit (y and the sum)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(rows + cols)
    x = torch.randn(rows, cols, generator=g, device=dev).to(dtype)
    r = torch.randn(rows, cols, generator=g, device=dev).to(dtype)
    w = torch.randn(cols, generator=g, device=dev).to(dtype)
    y0, s0 = hfa.rmsnorm(x, w, 1e-6, residual=r)
    for _ in range(2):
        y, s = hfa.rmsnorm(x, w, 1e-6, residual=r)
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(s, s0)
