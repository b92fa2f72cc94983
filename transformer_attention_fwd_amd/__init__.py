"""MI355X (gfx950) attention forward: a thin ctypes binding of the C-ABI library ``libfa.so``.

Every step of the computation runs in the library's HIP kernels; this module only marshals arguments.
There is no CPU or framework fallback: if ``libfa.so`` is missing the first call raises.

    fa_fwd(q, k, v, o, lse, B, H, N, D, layout, causal, scale, dtype, stream) -> status
        the C entry point with raw device pointers (ints) and sizes, same names and meaning as in
        include/fa.h.
    fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, D, layout, causal, window, q_offset, kv_start, kv_len,
              scale, dtype, stream) -> status
    fa_merge(o_parts, lse_parts, n_parts, o, lse, B, H, N, D, layout, dtype, stream) -> status
        the other two C entry points, same conventions.
    attention(q, k, v, *, layout="BHSD", causal=False, scale=None, out=None, lse=None) -> (o, lse)
        convenience wrapper for torch device tensors: checks shapes, allocates o and lse with torch,
        passes torch's current stream, raises FaError on a non-zero status.  scale=None means 1/sqrt(D).
    attention_ex(q, k, v, *, layout, causal, scale=None, window=-1, q_offset=0, kv_start=0, kv_len=None,
                 out=None, lse=None) -> (o, lse)
        the same for fa_fwd_ex (q [B,H,Nq,D] / [B,Nq,H,D], k and v [B,H,Nk,D] / [B,Nk,H,D]).
    merge(o_parts, lse_parts, *, layout, out=None, lse=None) -> (o, lse)
        fa_merge on torch tensors stacked along a leading parts dimension.
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, D, causal,
                  scale, dtype, stream) -> status
    attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, *, causal=False, scale=None, out=None,
                     lse=None) -> (o [total_q, H, D], lse [H, total_q])
        packed sequences of different lengths (int32 offset tensors on the device).
    fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, D, layout, causal, scale, dtype, stream) -> status
        the backward C entry point, same conventions.
    attention_bwd(q, k, v, o, lse, dout, *, layout="BHSD", causal=False, scale=None, delta=None) -> (dq, dk, dv)
        fa_bwd on torch tensors: allocates dq, dk, dv (and the delta workspace unless given).
    fa_bwd_atomic(q, k, v, o, lse, dout, dq, dk, dv, delta, dq_accum, B, H, N, D, layout, causal, scale, dtype,
                  stream) -> status
        the backward that sums dQ with fp32 atomic adds into the dq_accum workspace (B*H*N*D floats).
    attention_bwd(..., deterministic=False) uses it (16-bit inputs).
    fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, layout, causal, scale, dtype, stream) -> status
        fa_bwd for callers that cannot allocate: the D workspace is the library's static per-GPU array
        (B*H*N <= NOALLOC_MAX_ROWS; calls that overlap on one GPU race on it).
    fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, D, layout, causal, window, q_offset,
              kv_start, kv_len, scale, dtype, stream) -> status
    attention_bwd_ex(q, k, v, o, lse, dout, *, layout="BHSD", causal=False, scale=None, window=-1, q_offset=0,
                     kv_start=0, kv_len=None, dk=None, dv=None, delta=None) -> (dq, dk, dv)
        the generalised backward (dk, dv rows outside the key chunk keep the given tensors' values; new
        tensors start at zero).
    fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, D, causal, scale, dtype, stream) -> status
    attention_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, *,
                         causal=False, scale=None, delta=None, out=None) -> (dq, dk, dv)
        the backward of packed variable-length batches.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_fwd_ex", "fa_fwd_varlen", "fa_merge", "fa_bwd", "fa_bwd_ex", "fa_bwd_varlen", "fa_bwd_noalloc", "fa_bwd_atomic", "attention",
           "attention_ex", "attention_varlen", "merge", "attention_bwd", "attention_bwd_ex", "attention_bwd_varlen", "FaError", "library_path",
           "load", "status_str", "version",
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
FA_ERR_BAD_RANGE = 11
FA_ERR_SCRATCH_LIMIT = 12
NOALLOC_MAX_ROWS = 4194304  # FA_NOALLOC_MAX_ROWS

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def library_path() -> str:
    return os.path.join(_HERE, "libfa.so")


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libfa call failed with status %d: %s" % (status, message))
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
        lib.fa_fwd_ex.restype = ctypes.c_int
        lib.fa_fwd_ex.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_int] +
                                  [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
        lib.fa_merge.restype = ctypes.c_int
        lib.fa_merge.argtypes = ([ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p] +
                                 [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
        lib.fa_fwd_varlen.restype = ctypes.c_int
        lib.fa_fwd_varlen.argtypes = ([ctypes.c_void_p] * 7 + [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_void_p])
        lib.fa_bwd.restype = ctypes.c_int
        lib.fa_bwd.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int,
                               ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
        lib.fa_bwd_varlen.restype = ctypes.c_int
        lib.fa_bwd_varlen.argtypes = ([ctypes.c_void_p] * 12 + [ctypes.c_int64] * 7 + [ctypes.c_int, ctypes.c_float,
                                      ctypes.c_int, ctypes.c_void_p])
        lib.fa_bwd_atomic.restype = ctypes.c_int
        lib.fa_bwd_atomic.argtypes = ([ctypes.c_void_p] * 11 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int,
                                      ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
        lib.fa_bwd_noalloc.restype = ctypes.c_int
        lib.fa_bwd_noalloc.argtypes = ([ctypes.c_void_p] * 9 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_int,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
        lib.fa_bwd_ex.restype = ctypes.c_int
        lib.fa_bwd_ex.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int64] * 5 + [ctypes.c_int, ctypes.c_int] +
                                  [ctypes.c_int64] * 4 + [ctypes.c_float, ctypes.c_int, ctypes.c_void_p])
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


def fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, D, layout, causal, window, q_offset, kv_start, kv_len, scale, dtype,
              stream) -> int:
    """The generalised C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_fwd_ex(q or None, k or None, v or None, o or None, lse or None, B, H, Nq, Nk, D, layout,
                            int(causal), window, q_offset, kv_start, kv_len, scale, dtype, stream or None)


def fa_merge(o_parts, lse_parts, n_parts, o, lse, B, H, N, D, layout, dtype, stream) -> int:
    """The C merge entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_merge(o_parts or None, lse_parts or None, n_parts, o or None, lse or None, B, H, N, D,
                           layout, dtype, stream or None)


def fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k,
                  max_seqlen_q, max_seqlen_k, D, causal, scale, dtype, stream) -> int:
    """The packed variable-length backward C entry point: pointers are ints (0 = NULL), returns the status."""
    return load().fa_bwd_varlen(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                                dk or None, dv or None, delta or None, cu_seqlens_q or None, cu_seqlens_k or None, B,
                                H, total_q, total_k, max_seqlen_q, max_seqlen_k, D, int(causal), scale, dtype,
                                stream or None)


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, total_q, total_k, max_seqlen_q, D, causal,
                  scale, dtype, stream) -> int:
    """The packed variable-length C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_fwd_varlen(q or None, k or None, v or None, o or None, lse or None, cu_seqlens_q or None,
                                cu_seqlens_k or None, B, H, total_q, total_k, max_seqlen_q, D, int(causal), scale,
                                dtype, stream or None)


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, D, layout, causal, scale, dtype, stream) -> int:
    """The backward C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_bwd(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                         dk or None, dv or None, delta or None, B, H, N, D, layout, int(causal), scale, dtype,
                         stream or None)


def fa_bwd_atomic(q, k, v, o, lse, dout, dq, dk, dv, delta, dq_accum, B, H, N, D, layout, causal, scale, dtype,
                  stream) -> int:
    """The atomic-mode backward C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_bwd_atomic(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                                dk or None, dv or None, delta or None, dq_accum or None, B, H, N, D, layout,
                                int(causal), scale, dtype, stream or None)


def fa_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, layout, causal, scale, dtype, stream) -> int:
    """fa_bwd without the delta workspace (the library's static per-GPU array; allocates nothing)."""
    return load().fa_bwd_noalloc(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                                 dk or None, dv or None, B, H, N, D, layout, int(causal), scale, dtype, stream or None)


def fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Nq, Nk, D, layout, causal, window, q_offset, kv_start,
              kv_len, scale, dtype, stream) -> int:
    """The generalised backward C entry point: pointers are ints (0 = NULL), returns the status code."""
    return load().fa_bwd_ex(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                            dk or None, dv or None, delta or None, B, H, Nq, Nk, D, layout, int(causal), window,
                            q_offset, kv_start, kv_len, scale, dtype, stream or None)


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


def _raise_on(st):
    if st != FA_OK:
        msg = status_str(st)
        if st == FA_ERR_HIP:
            msg += ": " + last_error()
        raise FaError(st, msg)


def _bhnd(t, layout):
    if layout == "BHSD":
        B, H, N, D = t.shape
    else:
        B, N, H, D = t.shape
    return B, H, N, D


def attention_ex(q, k, v, *, layout: str = "BHSD", causal: bool = False, scale: float | None = None,
                 window: int = -1, q_offset: int = 0, kv_start: int = 0, kv_len: int | None = None,
                 out=None, lse=None):
    """fa_fwd_ex for torch device tensors: q [B,H,Nq,D] / [B,Nq,H,D]; k, v [B,H,Nk,D] / [B,Nk,H,D]."""
    import torch
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be 4-D and k, v 4-D tensors of one shape")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous in the given layout")
    B, H, Nq, D = _bhnd(q, layout)
    Bk, Hk, Nk, Dk = _bhnd(k, layout)
    if (Bk, Hk, Dk) != (B, H, D):
        raise ValueError("k, v must match q in B, H and D")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if kv_len is None:
        kv_len = Nk - kv_start
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, Nq]")
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    _raise_on(fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, D,
                        _LAYOUTS[layout], causal, int(window), int(q_offset), int(kv_start), int(kv_len),
                        float(scale), _dtype_code(q), stream))
    return out, lse


def merge(o_parts, lse_parts, *, layout: str = "BHSD", out=None, lse=None):
    """fa_merge for torch device tensors: o_parts [S, ...one O...], lse_parts [S, B, H, N] (float32)."""
    import torch
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    if o_parts.dim() != 5 or lse_parts.dim() != 4 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts must be [S, 4-D O] and lse_parts a float32 [S, B, H, N] tensor")
    if not o_parts.is_contiguous() or not lse_parts.is_contiguous():
        raise ValueError("o_parts and lse_parts must be contiguous")
    S = o_parts.shape[0]
    B, H, N, D = _bhnd(o_parts[0], layout)
    if tuple(lse_parts.shape) != (S, B, H, N):
        raise ValueError("lse_parts must be [S, B, H, N] matching o_parts")
    if out is None:
        out = torch.empty_like(o_parts[0])
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=o_parts.device)
    # the kernel writes B*H*N*D elements of o_parts' dtype into out and B*H*N floats into lse
    if out.shape != o_parts.shape[1:] or out.dtype != o_parts.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like one part of o_parts")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N]")
    stream = torch.cuda.current_stream(o_parts.device).cuda_stream if o_parts.is_cuda else 0
    _raise_on(fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), S, out.data_ptr(), lse.data_ptr(), B, H, N, D,
                       _LAYOUTS[layout], _dtype_code(o_parts), stream))
    return out, lse


def attention_bwd(q, k, v, o, lse, dout, *, layout: str = "BHSD", causal: bool = False, scale: float | None = None,
                  delta=None, deterministic: bool = True, dq_accum=None):
    """dQ, dK, dV for torch device tensors (q, k, v, o, dout of one shape; lse [B, H, N] fp32 from the forward).

    deterministic=False runs fa_bwd_atomic (16-bit inputs): dQ summed with fp32 atomic adds into dq_accum
    (allocated here unless given: float32, shaped like q)."""
    import torch
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must be 4-D tensors of one shape")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    for t in (q, k, v, o, dout):
        if not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must be contiguous in the given layout")
    B, H, N, D = _bhnd(q, layout)
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if delta.shape != (B, H, N) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 tensor of shape [B, H, N]")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    if deterministic:
        _raise_on(fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                         dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, D, _LAYOUTS[layout],
                         causal, float(scale), _dtype_code(q), stream))
        return dq, dk, dv
    if dq_accum is None:
        dq_accum = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dq_accum.shape != q.shape or dq_accum.dtype != torch.float32 or not dq_accum.is_contiguous():
        raise ValueError("dq_accum must be a contiguous float32 tensor shaped like q")
    _raise_on(fa_bwd_atomic(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), dq_accum.data_ptr(), B, H,
                            N, D, _LAYOUTS[layout], causal, float(scale), _dtype_code(q), stream))
    return dq, dk, dv


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, *, causal: bool = False,
                     scale: float | None = None, out=None, lse=None):
    """fa_fwd_varlen for torch device tensors: q [total_q, H, D], k and v [total_k, H, D], int32 offsets."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    for t in (cu_seqlens_q, cu_seqlens_k):
        if t.dim() != 1 or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 offsets")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    B = cu_seqlens_q.numel() - 1
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [H, total_q]")
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    _raise_on(fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, total_q, total_k, int(max_seqlen_q),
                            D, causal, float(scale), _dtype_code(q), stream))
    return out, lse


def attention_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int, *,
                         causal: bool = False, scale: float | None = None, delta=None, out=None):
    """fa_bwd_varlen for torch device tensors: q, o, dout [total_q, H, D]; k, v [total_k, H, D]; lse [H, total_q]
    of fa_fwd_varlen; int32 offsets.  Returns (dq, dk, dv); out = (dq, dk, dv) tensors to write into (rows of
    skipped sequences keep their values), else new ones."""
    import torch
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must be shaped like q")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    for t in (q, k, v, o, dout):
        if not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must be contiguous")
    for t in (cu_seqlens_q, cu_seqlens_k):
        if t.dim() != 1 or t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 offsets")
    total_q, H, D = q.shape
    total_k = k.shape[0]
    B = cu_seqlens_q.numel() - 1
    if lse.shape != (H, total_q) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [H, total_q]")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if delta is None:
        delta = torch.empty((H, total_q), dtype=torch.float32, device=q.device)
    if delta.shape != (H, total_q) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 tensor of shape [H, total_q]")
    dq, dk, dv = out if out is not None else (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    for t, like in ((dq, q), (dk, k), (dv, v)):
        if t.shape != like.shape or t.dtype != like.dtype or not t.is_contiguous():
            raise ValueError("out must hold contiguous tensors shaped like q, k, v")
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    _raise_on(fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_seqlens_q.data_ptr(),
                            cu_seqlens_k.data_ptr(), B, H, total_q, total_k, int(max_seqlen_q), int(max_seqlen_k), D,
                            causal, float(scale), _dtype_code(q), stream))
    return dq, dk, dv


def attention_bwd_ex(q, k, v, o, lse, dout, *, layout: str = "BHSD", causal: bool = False, scale: float | None = None,
                     window: int = -1, q_offset: int = 0, kv_start: int = 0, kv_len: int | None = None, dk=None,
                     dv=None, delta=None):
    """fa_bwd_ex for torch device tensors: q, o, dout [B,H,Nq,D] / [B,Nq,H,D]; k, v [B,H,Nk,D] / [B,Nk,H,D];
    lse [B,H,Nq] of the forward over every key.  Returns (dq partial of the chunk, dk, dv)."""
    import torch
    if layout not in _LAYOUTS:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, o, dout must share a 4-D shape and k, v another")
    if any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise TypeError("q, k, v, o, dout must share a dtype")
    for t in (q, k, v, o, dout):
        if not t.is_contiguous():
            raise ValueError("q, k, v, o, dout must be contiguous in the given layout")
    B, H, Nq, D = _bhnd(q, layout)
    Bk, Hk, Nk, Dk = _bhnd(k, layout)
    if (Bk, Hk, Dk) != (B, H, D):
        raise ValueError("k and v must match q in B, H and D")
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, H, Nq]")
    if kv_len is None:
        kv_len = Nk - kv_start
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if delta is None:
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if delta.shape != (B, H, Nq) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 tensor of shape [B, H, Nq]")
    dq = torch.empty_like(q)
    dk = torch.zeros_like(k) if dk is None else dk
    dv = torch.zeros_like(v) if dv is None else dv
    for t in (dk, dv):
        if t.shape != k.shape or t.dtype != k.dtype or not t.is_contiguous():
            raise ValueError("dk and dv must be contiguous tensors like k")
    stream = torch.cuda.current_stream(q.device).cuda_stream if q.is_cuda else 0
    _raise_on(fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
                        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, Nq, Nk, D,
                        _LAYOUTS[layout], causal, int(window), int(q_offset), int(kv_start), int(kv_len),
                        float(scale), _dtype_code(q), stream))
    return dq, dk, dv
