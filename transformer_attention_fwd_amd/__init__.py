"""MI355X (gfx950) attention forward: a thin ctypes binding of the C-ABI library ``libfa.so``.

Every step of the computation runs in the library's HIP kernels; this module only marshals arguments.
There is no CPU or framework fallback: if ``libfa.so`` is missing the first call raises.

    fa_fwd(q, k, v, o, lse, B, H, N, D, layout, causal, scale, dtype, stream) -> status
        the C entry point with raw device pointers (ints) and sizes, same names and meaning as in
        include/fa.h.
    attention(q, k, v, *, layout="BHSD", causal=False, scale=None, out=None, lse=None) -> (o, lse)
        convenience wrapper for torch device tensors: checks shapes, allocates o and lse with torch,
        passes torch's current stream, raises FaError on a non-zero status.  scale=None means 1/sqrt(D).
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fa_fwd", "attention", "FaError", "library_path", "load", "status_str", "version",
           "LAYOUT_BHSD", "LAYOUT_BSND", "DTYPE_FP32", "DTYPE_FP16", "DTYPE_BF16"]

LAYOUT_BHSD = 0
LAYOUT_BSND = 1
DTYPE_FP32 = 0
DTYPE_FP16 = 1
DTYPE_BF16 = 2
FA_OK = 0
FA_ERR_NULL = 1
FA_ERR_BAD_DIM = 2
FA_ERR_BAD_LAYOUT = 3
FA_ERR_BAD_DTYPE = 4
FA_ERR_UNSUPPORTED = 5
FA_ERR_BAD_SCALE = 6
FA_ERR_MISALIGNED = 7
FA_ERR_ALIAS = 8
FA_ERR_NOT_DEVICE_MEMORY = 9
FA_ERR_HIP = 10

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("fa_fwd failed with status %d: %s" % (status, message))
        self.status = status


def load():
    """Load libfa.so (built in place by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("libfa.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        lib.fa_fwd.restype = ctypes.c_int
        lib.fa_fwd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int,
                               ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
        lib.fa_status_str.restype = ctypes.c_char_p
        lib.fa_status_str.argtypes = [ctypes.c_int]
        lib.fa_last_error.restype = ctypes.c_char_p
        lib.fa_last_error.argtypes = []
        lib.fa_version.restype = ctypes.c_int
        lib.fa_version.argtypes = []
        _lib = lib
    return _lib


def fa_fwd(q, k, v, o, lse, B, H, N, D, layout, causal, scale, dtype, stream) -> int:
    """The C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_fwd(q or None, k or None, v or None, o or None, lse or None, B, H, N, D,
                         layout, int(causal), scale, dtype, stream or None)


def status_str(status: int) -> str:
    return load().fa_status_str(status).decode()


def last_error() -> str:
    return load().fa_last_error().decode()


def version() -> int:
    return load().fa_version()


_LAYOUTS = {"BHSD": LAYOUT_BHSD, "BSND": LAYOUT_BSND}


def _dtype_code(t):
    import torch
    codes = {torch.float32: DTYPE_FP32, torch.float16: DTYPE_FP16, torch.bfloat16: DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError("q, k, v must be float32, float16 or bfloat16 (got %s)" % t.dtype)
    return codes[t.dtype]


def attention(q, k, v, *, layout: str = "BHSD", causal: bool = False, scale: float | None = None,
              out=None, lse=None):
    """O and lse for torch device tensors q, k, v of shape [B,H,N,D] (BHSD) or [B,N,H,D] (BSND)."""
    import torch
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must be 4-D tensors of one shape (got %s, %s, %s)"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous in the given layout")
    if layout == "BHSD":
        B, H, N, D = q.shape
    else:
        B, N, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N]")
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, D,
                _LAYOUTS[layout], causal, float(scale), _dtype_code(q), stream)
    if st != FA_OK:
        msg = status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + last_error()
        raise FaError(st, msg)
    return out, lse
