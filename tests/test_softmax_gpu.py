"""GPU parity of hfa_softmax_rows against the fp64 CPU oracle.

Tolerance: max |gpu - oracle| <= 1e-5 per element (the fp32 bound used for
attention; softmax outputs lie in [0, 1]).  Shapes cover the book chapter's
[4096, 32000] matrix, rows wider than its one-block limit (65536: up to 65536
columns in registers, wider rows partly on chip and partly read twice), widths
that are not multiples of 4 and misaligned rows (the element-wise layout),
tiny widths, in-place use, inputs near the exp overflow range and -inf
entries.
"""

import numpy as np
import pytest
import torch

import fa2_fwd_amd as hfa
import oracle

pytestmark = pytest.mark.gpu

ATOL = 1e-5


def _x(rows, cols, seed, scale=4.0, shift=0.0):
    g = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(rows, cols, generator=g) * scale + shift).contiguous()


def _check(name, x_host, y_dev, rows=None):
    print(f"[softmax] {name}", flush=True)
    y = y_dev.cpu().double().numpy()
    ref = oracle.softmax_rows(x_host.numpy(), rows=rows)
    if rows is not None:
        y = y[rows]
    assert np.isfinite(y).all(), f"{name}: non-finite output"
    err = np.abs(y - ref).max()
    print(f"[softmax] {name}: max|d|={err:.3e}", flush=True)
    assert err <= ATOL, f"{name}: off by {err:.3e}"


@pytest.mark.parametrize("rows,cols", [(4096, 32000), (64, 70001), (8, 262144), (8, 262147), (3, 32768),
                                       (5, 32769), (7, 1000), (9, 1001), (2, 1), (3, 3), (1, 5)])
def test_softmax_rows_shapes(rows, cols):
    x = _x(rows, cols, seed=rows * 7 + cols)
    y = hfa.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    sample = None if rows * cols <= 4_000_000 else np.unique(np.r_[0, 1, rows // 2, rows - 1,
                                                             np.random.default_rng(cols).integers(0, rows, 24)])
    _check(f"{rows}x{cols}", x, y, rows=sample)


def test_softmax_rows_in_place():
    x = _x(16, 5000, seed=3)
    xd = x.cuda()
    y = hfa.softmax_rows(xd, out=xd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    _check("in place", x, xd)


def test_softmax_rows_misaligned_rows():
    # a view starting one float into the buffer: 4-byte aligned only
    x = _x(6, 4000, seed=5)
    buf = torch.empty(6 * 4000 + 1, device="cuda")
    xd = buf[1:].view(6, 4000)
    xd.copy_(x.cuda())
    y = hfa.softmax_rows(xd)
    torch.cuda.synchronize()
    _check("misaligned", x, y)


def test_softmax_rows_large_magnitudes():
    x = _x(4, 40000, seed=6, scale=30.0, shift=750.0)
    y = hfa.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    _check("near exp overflow", x, y)


def test_softmax_rows_minus_inf_entries():
    x = _x(3, 2000, seed=8)
    x[:, ::7] = -float("inf")
    y = hfa.softmax_rows(x.cuda()).cpu().double().numpy()
    finite = x.clone()
    keep = ~torch.isinf(x)
    ref = np.zeros((3, 2000))
    for r in range(3):
        cols = keep[r].numpy()
        ref[r, cols] = oracle.softmax_rows(finite[r:r + 1, cols].contiguous().numpy())[0]
    assert np.all(y[:, ::7] == 0.0)
    assert np.abs(y - ref).max() <= ATOL


def test_softmax_rows_rows_sum_to_one_on_device():
    x = _x(256, 100000, seed=9, scale=10.0)
    y = hfa.softmax_rows(x.cuda())
    s = y.double().sum(dim=1)
    assert torch.all((s - 1).abs() < 1e-4)


# Rows around and past the register-resident limits (49152 and 65536 columns:
# 24 and 32 slots of 2048 columns) with 16-byte accesses, then the wide
# kernel, whose first 52 slots of 2048 columns stay in
# registers (106496 columns), the next 18 in LDS, filled 6 slots per step
# (to 143360), the rest read twice in steps of 8 slots; widths around each of
# those boundaries and far past them.
WIDE = [(3, 32772), (2, 49148), (2, 49152), (2, 49156), (2, 65532), (2, 65536), (2, 65540), (2, 72700),
        (2, 72704), (2, 90000), (2, 102400), (2, 106492), (2, 106496), (2, 106500),
        (2, 118784), (2, 118788), (2, 131076), (2, 138236), (2, 143356), (2, 143360), (2, 143364), (2, 156668),
        (2, 156672), (2, 176128), (2, 176132), (2, 300000), (1, 1 << 20)]


@pytest.mark.parametrize("rows,cols", WIDE)
def test_softmax_rows_wide(rows, cols):
    x = _x(rows, cols, seed=rows + cols)
    y = hfa.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    _check(f"wide {rows}x{cols}", x, y)


@pytest.mark.parametrize("cols", [100000, 262144])
def test_softmax_rows_wide_in_place(cols):
    # every element is read (twice) by the thread that writes it, before it writes it
    x = _x(3, cols, seed=cols + 1)
    xd = x.cuda()
    y = hfa.softmax_rows(xd, out=xd)
    torch.cuda.synchronize()
    assert y.data_ptr() == xd.data_ptr()
    _check(f"wide in place 3x{cols}", x, xd)


def test_softmax_rows_wide_large_magnitudes_and_minus_inf():
    # peaked and shifted rows (the running max moves from chunk to chunk), runs
    # of -inf entries, the largest value in the last column
    x = _x(2, 200000, seed=11, scale=30.0, shift=-500.0)
    x[:, 156000:157000] = -float("inf")
    x[:, :5] = -float("inf")
    x[0, 199999] = 400.0
    y = hfa.softmax_rows(x.cuda()).cpu().double().numpy()
    keep = ~torch.isinf(x)
    ref = np.zeros(tuple(x.shape))
    for r in range(2):
        cols = keep[r].numpy()
        ref[r, cols] = oracle.softmax_rows(x[r:r + 1, cols].contiguous().numpy())[0]
    assert np.all(y[~keep.numpy()] == 0.0)
    err = np.abs(y - ref).max()
    print(f"[softmax] wide peaked/-inf: max|d|={err:.3e}", flush=True)
    assert err <= ATOL


@pytest.mark.parametrize("rows,cols", [(4096, 32000), (256, 262144), (64, 70001)])
def test_softmax_rows_bitwise_repeatable(rows, cols):
    # the resident and the wide kernel (block reductions through LDS): three runs agree bit for bit
    dev = torch.device("cuda:0")
    x = _x(rows, cols, seed=rows + cols).to(dev)
    y0 = hfa.softmax_rows(x)
    for _ in range(2):
        y = hfa.softmax_rows(x)
        torch.cuda.synchronize()
        assert torch.equal(y, y0)


@pytest.mark.parametrize("cols", [32767, 49151, 49153, 102401, 139265, 200003])
def test_softmax_rows_wide_unaligned(cols):
    # widths that are not a multiple of 4: the element-wise layout, resident up to
    # 24 slots (49152 columns), then the wide kernel (50 register slots, to 102400;
    # LDS to 139264), with the register, LDS and twice-read parts all in use at 200003
    x = _x(2, cols, seed=cols + 7)
    y = hfa.softmax_rows(x.cuda())
    torch.cuda.synchronize()
    _check(f"wide unaligned 2x{cols}", x, y)

