"""MI355X-native exact attention forward (FlashAttention-2 style online softmax).

A thin ctypes binding over ``libhfa.so`` (C ABI in ``include/hfa.h``).  The
functions named like the C entry points pass raw pointers straight through;
``attn_fwd`` does the argument marshalling for torch tensors on a gfx950
device (torch supplies device memory and the current stream, nothing else).
Every step of the computation runs in the library's HIP kernels: there is no
fallback path, and a missing or unloadable library raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from pathlib import Path

_PKG = Path(__file__).resolve().parent
# HFA_LIB selects another build of the library (e.g. one with host sanitizers).
LIB_PATH = Path(os.environ["HFA_LIB"]) if os.environ.get("HFA_LIB") else _PKG / "libhfa.so"

HFA_F32 = 0
HFA_BF16 = 1

HFA_OK = 0
HFA_ERR_NULL = 1
HFA_ERR_SHAPE = 2
HFA_ERR_UNSUPPORTED = 3
HFA_ERR_SCALE = 4
HFA_ERR_ALIGN = 5
HFA_ERR_ALIAS = 6
HFA_ERR_NO_DEVICE = 7
HFA_ERR_LAUNCH = 8
HFA_ERR_EPS = 9
HFA_ERR_WORKSPACE = 10

EXPORTED = ("hfa_attn_fwd", "hfa_status_str", "hfa_block_rows", "hfa_key_splits", "hfa_attn_fwd_workspace_size",
            "hfa_attn_fwd_split", "hfa_attn_fwd_split_noalloc", "hfa_attn_fwd_graph_create", "hfa_graph_launch", "hfa_graph_destroy",
            "hfa_softmax_rows", "hfa_rmsnorm")

_lib = None


class HfaError(RuntimeError):
    """A status other than HFA_OK returned by the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"hfa status {status}: {hfa_status_str(status)}")


def load_library(path: str | Path | None = None) -> ctypes.CDLL:
    """Load ``libhfa.so`` (building it first if it has never been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        if path is not None:
            raise FileNotFoundError(p)
        from fa2_fwd_amd.build import build

        build()
    lib = ctypes.CDLL(str(p))
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.hfa_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.hfa_attn_fwd.restype = ctypes.c_int
    lib.hfa_status_str.argtypes = [ctypes.c_int]
    lib.hfa_status_str.restype = ctypes.c_char_p
    lib.hfa_block_rows.argtypes = [ctypes.c_int, i64, i64, i64, i64]
    lib.hfa_block_rows.restype = i64
    lib.hfa_key_splits.argtypes = [ctypes.c_int, i64, i64, i64, i64]
    lib.hfa_key_splits.restype = i64
    lib.hfa_attn_fwd_workspace_size.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64]
    lib.hfa_attn_fwd_workspace_size.restype = i64
    lib.hfa_attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int, i64, vp,
                                       i64, vp]
    lib.hfa_attn_fwd_split.restype = ctypes.c_int
    lib.hfa_attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                               i64, vp]
    lib.hfa_attn_fwd_split_noalloc.restype = ctypes.c_int
    lib.hfa_attn_fwd_graph_create.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_int,
                                              i64, ctypes.POINTER(vp)]
    lib.hfa_attn_fwd_graph_create.restype = ctypes.c_int
    lib.hfa_graph_launch.argtypes = [vp, vp]
    lib.hfa_graph_launch.restype = ctypes.c_int
    lib.hfa_graph_destroy.argtypes = [vp]
    lib.hfa_graph_destroy.restype = None
    lib.hfa_softmax_rows.argtypes = [vp, vp, i64, i64, vp]
    lib.hfa_softmax_rows.restype = ctypes.c_int
    lib.hfa_rmsnorm.argtypes = [vp, vp, vp, vp, vp, i64, i64, ctypes.c_float, ctypes.c_int, vp]
    lib.hfa_rmsnorm.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def hfa_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, dtype, stream) -> int:
    """Raw C-ABI call: every pointer an int (device address) or None; returns the status."""
    return load_library().hfa_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, dtype, stream)


def hfa_status_str(status: int) -> str:
    return load_library().hfa_status_str(int(status)).decode()


def hfa_block_rows(dtype: int, B: int, H: int, N: int, d: int) -> int:
    return int(load_library().hfa_block_rows(int(dtype), int(B), int(H), int(N), int(d)))


def hfa_key_splits(dtype: int, B: int, H: int, N: int, d: int) -> int:
    return int(load_library().hfa_key_splits(int(dtype), int(B), int(H), int(N), int(d)))


def hfa_attn_fwd_workspace_size(dtype: int, B: int, H: int, N: int, d: int, splits: int) -> int:
    return int(load_library().hfa_attn_fwd_workspace_size(int(dtype), int(B), int(H), int(N), int(d), int(splits)))


def hfa_attn_fwd_split(q, k, v, o, lse, B, H, N, d, scale, dtype, splits, workspace, workspace_bytes, stream) -> int:
    """Raw C-ABI call: pointers as ints (device addresses) or None; returns the status."""
    return load_library().hfa_attn_fwd_split(q, k, v, o, lse, B, H, N, d, scale, dtype, splits, workspace,
                                             workspace_bytes, stream)


def hfa_attn_fwd_split_noalloc(q, k, v, o, lse, B, H, N, d, scale, dtype, splits, stream) -> int:
    """Raw C-ABI call (the library's own scratch as workspace): pointers as ints; returns the status."""
    return load_library().hfa_attn_fwd_split_noalloc(q, k, v, o, lse, B, H, N, d, scale, dtype, splits, stream)


def hfa_attn_fwd_graph_create(q, k, v, o, lse, B, H, N, d, scale, dtype, count):
    """Raw C-ABI call; returns (status, graph handle or None)."""
    h = ctypes.c_void_p()
    st = load_library().hfa_attn_fwd_graph_create(q, k, v, o, lse, B, H, N, d, scale, dtype, count,
                                                 ctypes.byref(h))
    return st, h.value


def hfa_graph_launch(graph, stream) -> int:
    return load_library().hfa_graph_launch(graph, stream)


def hfa_graph_destroy(graph) -> None:
    load_library().hfa_graph_destroy(graph)


def hfa_softmax_rows(x, y, rows, cols, stream) -> int:
    """Raw C-ABI call: pointers as ints (device addresses) or None; returns the status."""
    return load_library().hfa_softmax_rows(x, y, rows, cols, stream)


def softmax_rows(x, out=None, stream=None):
    """Row softmax of a contiguous float32 [rows, cols] device tensor (``out`` may be ``x``)."""
    import torch

    if not isinstance(x, torch.Tensor) or x.ndim != 2 or x.dtype != torch.float32:
        raise ValueError("softmax_rows needs a float32 [rows, cols] tensor")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("softmax_rows needs a contiguous GPU tensor")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    with torch.cuda.device(x.device):
        st = hfa_softmax_rows(x.data_ptr(), out.data_ptr(), x.shape[0], x.shape[1], _stream_handle(stream, x.device))
    if st != HFA_OK:
        raise HfaError(st)
    return out


def hfa_rmsnorm(x, residual, weight, y, residual_out, rows, cols, eps, dtype, stream) -> int:
    """Raw C-ABI call: pointers as ints (device addresses) or None; returns the status."""
    return load_library().hfa_rmsnorm(x, residual, weight, y, residual_out, rows, cols, eps, dtype, stream)


def rmsnorm(x, weight, eps: float = 1e-6, residual=None, out=None, residual_out=None, stream=None):
    """RMS normalisation over the last dim of a contiguous float32 or bfloat16 device tensor.

    ``y = s / sqrt(mean(s**2) + eps) * weight`` with ``s = x + residual`` (``s = x`` without a
    residual).  Returns ``y``, or ``(y, s)`` when ``residual`` is given.  ``out`` and
    ``residual_out`` may be given to write into caller buffers, and may be ``x`` or ``residual``
    themselves (in place).  Rows are limited to 65536 elements.
    """
    import torch

    tensors = [x, weight] + ([residual] if residual is not None else [])
    if any(not isinstance(t, torch.Tensor) for t in tensors):
        raise ValueError("rmsnorm takes torch tensors")
    if x.ndim < 1 or weight.ndim != 1 or weight.shape[0] != x.shape[-1]:
        raise ValueError("rmsnorm needs x [..., C] and weight [C]")
    code = _dtype_code(x)
    if any(t.dtype != x.dtype for t in tensors):
        raise ValueError("x, weight and residual must share one dtype")
    if residual is not None and residual.shape != x.shape:
        raise ValueError("residual must have x's shape")
    if any(not t.is_cuda or t.device != x.device for t in tensors) or any(not t.is_contiguous() for t in tensors):
        raise ValueError("rmsnorm needs contiguous tensors on one GPU")

    def _buf(t):
        if t is None:
            return torch.empty_like(x)
        if t.shape != x.shape or t.dtype != x.dtype or t.device != x.device or not t.is_contiguous():
            raise ValueError("output buffers must be contiguous tensors like x")
        return t

    out = _buf(out)
    res_out = _buf(residual_out) if residual is not None else None
    cols = x.shape[-1]
    rows = x.numel() // cols if cols else 0
    with torch.cuda.device(x.device):
        st = hfa_rmsnorm(x.data_ptr(), None if residual is None else residual.data_ptr(), weight.data_ptr(),
                         out.data_ptr(), None if res_out is None else res_out.data_ptr(), rows, cols, float(eps),
                         code, _stream_handle(stream, x.device))
    if st != HFA_OK:
        raise HfaError(st)
    return out if residual is None else (out, res_out)


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.float32:
        return HFA_F32
    if t.dtype == torch.bfloat16:
        return HFA_BF16
    raise ValueError(f"float32 and bfloat16 are supported, got {t.dtype}")


def _prepare(q, k, v, scale, out, lse):
    """Checks of attn_fwd's tensor arguments; allocates out / lse when None."""
    import torch

    tensors = (q, k, v)
    if any(not isinstance(t, torch.Tensor) for t in tensors):
        raise ValueError("q, k, v must be torch tensors")
    if q.ndim != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("attn_fwd needs equal-shape [B, H, N, d] tensors")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    code = _dtype_code(q)
    if any(not t.is_cuda for t in tensors) or k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on the same GPU device")
    if any(not t.is_contiguous() for t in tensors):
        raise ValueError("attn_fwd needs contiguous tensors")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    elif lse.shape != (B, H, N) or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    return B, H, N, d, code, float(scale), out, lse


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def attn_fwd(q, k, v, scale: float | None = None, out=None, lse=None, stream=None, splits: int = 0,
             workspace=None):
    """O, LSE = attention forward of device tensors q, k, v of shape [B, H, N, d].

    ``scale`` defaults to 1/sqrt(d).  ``out`` ([B,H,N,d], q's dtype) and ``lse``
    ([B,H,N] float32) may be given to write into caller buffers.  The kernels are
    enqueued on ``stream`` (default: torch's current stream) and not waited for.
    ``splits`` is the key split (hfa_attn_fwd_split): 0 lets the library choose (bf16
    shapes too small to fill the GPU split their keys; fp32 shapes whose key tiles are
    shared by enough workgroups format K and V once per call), 1 never splits (fp32:
    always formats K and V once per call).  Such a call needs a workspace of
    hfa_attn_fwd_workspace_size bytes: ``workspace`` (a device tensor) if given, else
    one from torch's allocator, kept alive for ``stream``.
    Raises ValueError on dtype, shape, device or contiguity mismatch and HfaError on a
    library error.
    """
    import torch

    B, H, N, d, code, scale, out, lse = _prepare(q, k, v, scale, out, lse)
    handle = _stream_handle(stream, q.device)
    need = hfa_attn_fwd_workspace_size(code, B, H, N, d, int(splits))
    if need < 0:
        raise HfaError(HFA_ERR_UNSUPPORTED if int(splits) >= 0 else HFA_ERR_SHAPE)
    with torch.cuda.device(q.device):
        if need == 0:
            st = hfa_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, N, d, scale, code, handle)
        else:
            if workspace is None:
                workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
                if stream is not None:
                    workspace.record_stream(stream if isinstance(stream, torch.cuda.Stream)
                                            else torch.cuda.ExternalStream(handle, device=q.device))
            elif not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or workspace.device != q.device:
                raise ValueError("workspace must be a tensor on q's device")
            st = hfa_attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    B, H, N, d, scale, code, int(splits), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), handle)
    if st != HFA_OK:
        raise HfaError(st)
    return out, lse


class AttnGraph:
    """``count`` attention forwards of fixed tensors, captured once into a HIP graph.

    ``launch()`` replays all of them with one driver call (see
    hfa_attn_fwd_graph_create in include/hfa.h).  ``out`` and ``lse`` are the
    buffers every replay writes.  The tensors must outlive the graph; use
    ``close()`` (or ``with``) to release it once its replays are done.
    """

    def __init__(self, q, k, v, scale: float | None = None, out=None, lse=None, count: int = 1):
        import torch

        B, H, N, d, code, scale, out, lse = _prepare(q, k, v, scale, out, lse)
        self.q, self.k, self.v, self.out, self.lse = q, k, v, out, lse
        self.device = q.device
        with torch.cuda.device(q.device):
            st, h = hfa_attn_fwd_graph_create(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                              lse.data_ptr(), B, H, N, d, scale, code, int(count))
        if st != HFA_OK:
            raise HfaError(st)
        self._graph = h

    def launch(self, stream=None):
        import torch

        if self._graph is None:
            raise ValueError("graph already closed")
        with torch.cuda.device(self.device):
            st = hfa_graph_launch(self._graph, _stream_handle(stream, self.device))
        if st != HFA_OK:
            raise HfaError(st)
        return self.out, self.lse

    def close(self):
        if self._graph is not None:
            hfa_graph_destroy(self._graph)
            self._graph = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
