"""CPU oracle for exact attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library (``fa2_fwd_amd``)
never imports, links or calls it, and the two share no code: this side is a
plain fp64 C++ implementation (``hfa_ref.cpp``) built with g++, driven through
ctypes.

What it computes (neuralmasteryai "Hardware Acceleration & Custom Kernels",
section 2, the attention definition; book chapter "Triton and kernel fusion",
section "Fusion", the stable row softmax):

    s_ij  = scale * sum_c q_ic k_jc          (fp64, whole score row materialised)
    O_i   = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i),   m_i = max_j s_ij
    LSE_i = m_i + ln sum_j exp(s_ij - m_i)

``attn_fwd_online`` computes the same quantities by the online normalisation
identity of that section 2, step 2, tile by tile over the keys.

``softmax_rows`` is the standalone stable row softmax of that chapter's
"Fusion" section (y = exp(x - max) / sum, per row of a float32 matrix);
``softmax_rows_online`` takes the row max and sum in one sweep by the same
running identity, over chunks of any width.

``rmsnorm`` is the RMS normalisation of the TritonForge "Fused RMSNorm" card,
y = x / sqrt(sum_i x_i^2 / d + eps) * w per row, with the optional residual
of that chapter's "Fused residual add + RMSNorm" section added first (in fp32,
as the chapter's kernel adds it); it returns y and the sum.

Attention inputs are numpy arrays of shape [B, H, N, d]: ``float32`` for fp32 data, or
``uint16`` holding bf16 bit patterns.  Outputs are fp64.
"""

from __future__ import annotations

import ctypes
import os
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
# HFA_REF_LIB selects another build (e.g. one with the sanitizers).
LIB_PATH = Path(os.environ["HFA_REF_LIB"]) if os.environ.get("HFA_REF_LIB") else _HERE / "libhfa_ref.so"


def default_threads() -> int:
    """Host threads the oracle uses: OMP_NUM_THREADS if set, else the CPUs this process may use."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _prep(q, k, v):
    arrs = [np.ascontiguousarray(a) for a in (q, k, v)]
    dt = arrs[0].dtype
    if any(a.dtype != dt for a in arrs):
        raise ValueError("q, k, v must share one dtype")
    if dt == np.float32:
        code = 0
    elif dt == np.uint16:
        code = 1
    else:
        raise ValueError("oracle inputs are float32 or uint16 (bf16 bit patterns), got %s" % dt)
    if arrs[0].ndim != 4 or any(a.shape != arrs[0].shape for a in arrs):
        raise ValueError("q, k, v must be equal-shape [B, H, N, d] arrays")
    return arrs, code


class OracleLib:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path):
        lib = ctypes.CDLL(str(path))
        i64 = ctypes.c_int64
        vp = ctypes.c_void_p
        lib.hfa_ref_attn_fwd.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                         ctypes.c_double, vp, i64, vp, vp, ctypes.c_int]
        lib.hfa_ref_attn_fwd.restype = ctypes.c_int
        lib.hfa_ref_attn_fwd_online.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, i64, i64,
                                                ctypes.c_double, i64, vp, i64, vp, vp, ctypes.c_int]
        lib.hfa_ref_attn_fwd_online.restype = ctypes.c_int
        lib.hfa_ref_softmax_rows.argtypes = [vp, i64, i64, vp, i64, vp, ctypes.c_int]
        lib.hfa_ref_softmax_rows.restype = ctypes.c_int
        lib.hfa_ref_softmax_rows_online.argtypes = [vp, i64, i64, i64, vp, i64, vp, ctypes.c_int]
        lib.hfa_ref_softmax_rows_online.restype = ctypes.c_int
        lib.hfa_ref_rmsnorm.argtypes = [vp, vp, vp, ctypes.c_int, i64, i64, ctypes.c_double, vp, i64, vp, vp,
                                        ctypes.c_int]
        lib.hfa_ref_rmsnorm.restype = ctypes.c_int
        self.lib = lib
        self.path = str(path)

    def _call(self, fn_name, q, k, v, scale, rows, threads, tile=None):
        (q, k, v), code = _prep(q, k, v)
        B, H, N, d = q.shape
        rows_arr = None
        if rows is not None:
            rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
            R = rows_arr.shape[0]
        else:
            R = N
        o = np.empty((B, H, R, d), dtype=np.float64)
        lse = np.empty((B, H, R), dtype=np.float64)
        thr = int(threads) if threads else default_threads()
        ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
        args = [ptr(q), ptr(k), ptr(v), code, B, H, N, d, float(scale)]
        if tile is not None:
            args.append(int(tile))
        args += [ptr(rows_arr), R if rows_arr is not None else 0, ptr(o), ptr(lse), thr]
        rc = getattr(self.lib, fn_name)(*args)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (%s)" % fn_name)
        return o, lse

    def _softmax(self, x, rows, threads, chunk=None):
        x = np.ascontiguousarray(x)
        if x.dtype != np.float32 or x.ndim != 2:
            raise ValueError("softmax oracle input is a float32 [R, C] array")
        R, C = x.shape
        rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = R if rows_arr is None else rows_arr.shape[0]
        y = np.empty((n, C), dtype=np.float64)
        thr = int(threads) if threads else default_threads()
        rp = None if rows_arr is None else rows_arr.ctypes.data
        if chunk is None:
            rc = self.lib.hfa_ref_softmax_rows(x.ctypes.data, R, C, rp, n if rows_arr is not None else 0,
                                               y.ctypes.data, thr)
        else:
            rc = self.lib.hfa_ref_softmax_rows_online(x.ctypes.data, R, C, int(chunk), rp,
                                                      n if rows_arr is not None else 0, y.ctypes.data, thr)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (softmax)")
        return y

    def softmax_rows(self, x, rows=None, threads=0):
        """Row softmax of a float32 [R, C] array in fp64 (definition form).  Returns [R or len(rows), C]."""
        return self._softmax(x, rows, threads)

    def softmax_rows_online(self, x, chunk, rows=None, threads=0):
        """Row softmax with (max, sum) taken by the running identity over chunks of ``chunk`` columns."""
        return self._softmax(x, rows, threads, chunk=chunk)

    def rmsnorm(self, x, weight, eps, residual=None, rows=None, threads=0):
        """RMS normalisation of the rows of x [R, C] (float32, or uint16 bf16 patterns) in fp64.

        Returns (y, s): y = s / sqrt(mean_j s_j^2 + eps) * weight and s = x + residual formed in
        fp32 (s = x without a residual), both fp64 [R or len(rows), C]."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(weight)
        if x.ndim != 2 or w.ndim != 1 or w.shape[0] != x.shape[1]:
            raise ValueError("rmsnorm oracle takes x [R, C] and weight [C]")
        if x.dtype == np.float32:
            code = 0
        elif x.dtype == np.uint16:
            code = 1
        else:
            raise ValueError("oracle inputs are float32 or uint16 (bf16 bit patterns), got %s" % x.dtype)
        if w.dtype != x.dtype:
            raise ValueError("weight must have x's dtype")
        r = None
        if residual is not None:
            r = np.ascontiguousarray(residual)
            if r.shape != x.shape or r.dtype != x.dtype:
                raise ValueError("residual must match x")
        R, C = x.shape
        rows_arr = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = R if rows_arr is None else rows_arr.shape[0]
        y = np.empty((n, C), dtype=np.float64)
        s = np.empty((n, C), dtype=np.float64)
        thr = int(threads) if threads else default_threads()
        rc = self.lib.hfa_ref_rmsnorm(x.ctypes.data, None if r is None else r.ctypes.data, w.ctypes.data, code, R, C,
                                      float(eps), None if rows_arr is None else rows_arr.ctypes.data,
                                      n if rows_arr is not None else 0, y.ctypes.data, s.ctypes.data, thr)
        if rc != 0:
            raise ValueError("oracle rejected its arguments (rmsnorm)")
        return y, s

    def attn_fwd(self, q, k, v, scale, rows=None, threads=0):
        """Definition-form attention forward in fp64.  Returns (O [B,H,R,d], LSE [B,H,R])."""
        return self._call("hfa_ref_attn_fwd", q, k, v, scale, rows, threads)

    def attn_fwd_online(self, q, k, v, scale, tile, rows=None, threads=0):
        """Online-normalisation form over key tiles of width ``tile`` (fp64)."""
        return self._call("hfa_ref_attn_fwd_online", q, k, v, scale, rows, threads, tile=tile)


_default = None


def default() -> OracleLib:
    """The oracle built from ``hfa_ref.cpp`` in this directory (built on first use if absent)."""
    global _default
    if _default is None:
        if not LIB_PATH.exists():
            from oracle.build import build

            build()
        _default = OracleLib(LIB_PATH)
    return _default


def attn_fwd(q, k, v, scale, rows=None, threads=0):
    """Definition-form attention forward in fp64.  Returns (O [B,H,R,d], LSE [B,H,R])."""
    return default().attn_fwd(q, k, v, scale, rows, threads)


def attn_fwd_online(q, k, v, scale, tile, rows=None, threads=0):
    """Online-normalisation form over key tiles of width ``tile`` (fp64)."""
    return default().attn_fwd_online(q, k, v, scale, tile, rows, threads)


def softmax_rows(x, rows=None, threads=0):
    """Row softmax of a float32 [R, C] array in fp64 (definition form)."""
    return default().softmax_rows(x, rows, threads)


def softmax_rows_online(x, chunk, rows=None, threads=0):
    """Row softmax in fp64 with (max, sum) by the running identity over chunks of ``chunk`` columns."""
    return default().softmax_rows_online(x, chunk, rows, threads)


def rmsnorm(x, weight, eps, residual=None, rows=None, threads=0):
    """RMS normalisation in fp64 of x [R, C] (+ residual, added in fp32).  Returns (y, s)."""
    return default().rmsnorm(x, weight, eps, residual, rows, threads)
