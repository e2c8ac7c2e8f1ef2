"""Seeded synthetic inputs for the attention forward, the row softmax and the RMS normalisation.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic, so both the GPU path's tests and the CPU oracle can take
their inputs from it.

Recipe: ``torch.Generator('cpu').manual_seed(seed)``, then ``torch.randn`` in
fp32 for full [B, H, N, d] tensors drawn in the order Q, K, V.  Optionally Q
and K are multiplied by a power of two after drawing (exact in binary floating
point), which makes softmax rows peaked.  bf16 workloads round the fp32 draws
to bf16 with round-to-nearest-even (torch's ``.to(torch.bfloat16)``).
"""

from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" or "bf16"
    seed: int
    qk_mult: float = 1.0

    @property
    def scale(self) -> float:
        """1/sqrt(d) as the fp32 value both sides use."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> int:
        """Counted work: the two matrix products, 4*B*H*N^2*d."""
        return 4 * self.B * self.H * self.N * self.N * self.d

    def describe(self) -> str:
        extra = f" Q,K x{self.qk_mult:g}" if self.qk_mult != 1.0 else ""
        return f"attn_fwd B={self.B} H={self.H} N={self.N} d={self.d} {self.dtype}{extra} seed={self.seed}"


# The five evaluation shapes: small fp32, the two fp32 sequence lengths of the
# pages' benchmark table (N=1024, N=2048; the table does not state B, H or d),
# and two long bf16 sequences.
CONFIGS = {
    1: Workload("cfg1", 1, 1, 128, 64, "f32", 1),
    2: Workload("cfg2", 4, 8, 1024, 64, "f32", 2),
    3: Workload("cfg3", 4, 8, 2048, 64, "f32", 3, qk_mult=4.0),
    4: Workload("cfg4", 2, 32, 4096, 128, "bf16", 4),
    5: Workload("cfg5", 1, 16, 16384, 128, "bf16", 5),
}


@dataclass(frozen=True)
class SoftmaxWorkload:
    """Row softmax of a seeded N(0, scale^2) fp32 [rows, cols] matrix."""

    name: str
    rows: int
    cols: int
    seed: int
    scale: float = 4.0

    @property
    def algorithmic_bytes(self) -> int:
        """The method's minimum traffic: read x once, write y once (fp32)."""
        return 2 * self.rows * self.cols * 4

    def describe(self) -> str:
        return f"softmax_rows {self.rows}x{self.cols} f32 seed={self.seed}"

    def inputs(self) -> torch.Tensor:
        g = torch.Generator("cpu").manual_seed(int(self.seed))
        return (torch.randn(self.rows, self.cols, generator=g, dtype=torch.float32) * self.scale).contiguous()


# Row softmax workloads: the [4096, 32000] fp32 matrix of the book chapter
# "Triton and kernel fusion" (section "Fusion"), and rows four times wider
# than that chapter's one-block limit of 65536 columns.
SOFTMAX_CONFIGS = {
    1: SoftmaxWorkload("softmax1", 4096, 32000, 101),
    2: SoftmaxWorkload("softmax2", 256, 262144, 102),
}


@dataclass(frozen=True)
class RmsNormWorkload:
    """Residual add + RMS normalisation of seeded [rows, cols] rows.

    Draw order: x, residual (both N(0, 1)), then weight = 1 + 0.1 N(0, 1), all fp32,
    rounded to bf16 (nearest even) for bf16 workloads."""

    name: str
    rows: int
    cols: int
    dtype: str  # "f32" or "bf16"
    seed: int
    residual: bool = True
    eps: float = 1e-6

    @property
    def elt(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def algorithmic_bytes(self) -> int:
        """x (and the residual) read once, y (and the sum) written once, the weight read once."""
        arrays = 4 if self.residual else 2
        return (arrays * self.rows * self.cols + self.cols) * self.elt

    def describe(self) -> str:
        res = " +residual" if self.residual else ""
        return f"rmsnorm {self.rows}x{self.cols} {self.dtype}{res} seed={self.seed}"

    def inputs(self):
        """Host tensors (x, residual or None, weight) in the workload's dtype."""
        g = torch.Generator("cpu").manual_seed(int(self.seed))
        x = torch.randn(self.rows, self.cols, generator=g, dtype=torch.float32)
        r = torch.randn(self.rows, self.cols, generator=g, dtype=torch.float32) if self.residual else None
        w = 1.0 + 0.1 * torch.randn(self.cols, generator=g, dtype=torch.float32)
        dt = torch_dtype(self.dtype)
        return x.to(dt), (r.to(dt) if r is not None else None), w.to(dt)


# RMS normalisation workloads: the widths of the TritonForge benchmark table
# (N = 512, 2048, 8192, fp32; its row counts are not given), each sized to
# 2^26 elements, and a bf16 [16384, 8192] transformer residual stream.  All
# take the fused residual form of the book chapter "Triton and kernel fusion".
RMSNORM_CONFIGS = {
    1: RmsNormWorkload("rmsnorm1", 131072, 512, "f32", 201),
    2: RmsNormWorkload("rmsnorm2", 32768, 2048, "f32", 202),
    3: RmsNormWorkload("rmsnorm3", 8192, 8192, "f32", 203),
    4: RmsNormWorkload("rmsnorm4", 16384, 8192, "bf16", 204),
}


def torch_dtype(dtype: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_inputs(B: int, H: int, N: int, d: int, dtype: str, seed: int, qk_mult: float = 1.0):
    """Host (CPU) tensors q, k, v of shape [B, H, N, d] in ``dtype``, contiguous."""
    g = torch.Generator("cpu").manual_seed(int(seed))
    shape = (B, H, N, d)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if qk_mult != 1.0:
        q.mul_(qk_mult)
        k.mul_(qk_mult)
    td = torch_dtype(dtype)
    if td != torch.float32:
        q, k, v = q.to(td), k.to(td), v.to(td)
    return q.contiguous(), k.contiguous(), v.contiguous()


def workload_inputs(w: Workload):
    return make_inputs(w.B, w.H, w.N, w.d, w.dtype, w.seed, w.qk_mult)


def to_oracle_array(t: torch.Tensor) -> np.ndarray:
    """Host numpy view the oracle accepts: float32, or uint16 bit patterns for bf16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unsupported dtype {t.dtype}")


def sample_rows(N: int, n_random: int, seed: int) -> np.ndarray:
    """Deterministic query-row sample: tile edges, the middle, the end, plus seeded random rows."""
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, N // 2, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, N, size=n_random) if n_random > 0 else np.empty(0, dtype=np.int64)
    rows = sorted({int(r) for r in fixed if 0 <= r < N} | {int(r) for r in rnd})
    return np.asarray(rows, dtype=np.int64)
