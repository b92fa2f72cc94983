"""The attention oracle: a plain fp64 two-pass CPU implementation of the forward pass and its
gradients (``fa_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  It shares no code with the HIP library and imports nothing from
the ``transformer_attention_fwd_amd`` package.

The C file states what is computed and which passage of the pages each step follows.  This module only
builds the C file with gcc, loads it with ctypes and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"fp32": 0, "fp16": 1, "bf16": 2, "fp64": 3}
ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2, "fp64": 8}
LAYOUTS = {"BHSD": 0, "BSND": 1}

_lib = None


def build(force: bool = False) -> str:
    """Compile ``fa_oracle.c`` into ``liboracle.so`` next to it (gcc -O2, pthreads)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.fa_oracle_rows.restype = ctypes.c_int
        lib.fa_oracle_rows.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.fa_oracle_rows_ex.restype = ctypes.c_int
        lib.fa_oracle_rows_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.fa_oracle_bwd_head_ex.restype = ctypes.c_int
        lib.fa_oracle_bwd_head_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.fa_oracle_bwd_head_mag_ex.restype = ctypes.c_int
        lib.fa_oracle_bwd_head_mag_ex.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.fa_oracle_bwd_head.restype = ctypes.c_int
        lib.fa_oracle_bwd_head.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
        ]
        _lib = lib
    return _lib


def _dims(shape, layout):
    if len(shape) != 4:
        raise ValueError("q, k, v must be 4-D")
    if layout == "BHSD":
        B, H, N, D = shape
    elif layout == "BSND":
        B, N, H, D = shape
    else:
        raise ValueError("layout must be 'BHSD' or 'BSND'")
    return B, H, N, D


def attention_rows(q, k, v, *, dtype: str, layout: str, causal: bool, scale: float, rows, nthreads: int = 1):
    """O and lse of the requested query rows, in fp64.

    q, k, v: numpy arrays holding the stored elements, shaped [B,H,N,D] (BHSD) or [B,N,H,D] (BSND),
    with itemsize matching ``dtype`` (bf16 and fp16 as 16-bit patterns, e.g. uint16 or float16).
    rows: int64 array of shape [R, 3] holding (b, h, i) triples.
    scale: used as given (pass the fp32-rounded value to model an fp32 scale argument).
    Returns (o [R, D] float64, lse [R] float64).
    """
    if dtype not in DTYPES:
        raise ValueError("dtype must be one of %s" % sorted(DTYPES))
    B, H, N, D = _dims(q.shape, layout)
    for t in (q, k, v):
        if t.shape != q.shape or t.dtype.itemsize != ITEMSIZE[dtype]:
            raise ValueError("q, k, v must share the shape and have the itemsize of %s" % dtype)
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    R = rows.shape[0]
    o = np.empty((R, D), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    if R == 0:
        return o, lse
    rc = _load().fa_oracle_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPES[dtype], LAYOUTS[layout],
                                B, H, N, D, 1 if causal else 0, float(scale), rows.ctypes.data, R,
                                o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("fa_oracle_rows failed with status %d" % rc)
    return o, lse


def all_rows(B: int, H: int, N: int) -> np.ndarray:
    """Every (b, h, i) triple in [B, H, N] order."""
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    return np.stack([b.ravel(), h.ravel(), i.ravel()], axis=1).astype(np.int64)


def attention(q, k, v, *, dtype: str, layout: str, causal: bool, scale: float, nthreads: int = 1):
    """Full O and lse, in fp64.  O is returned in the input's layout; lse as [B, H, N]."""
    B, H, N, D = _dims(q.shape, layout)
    o_rows, lse = attention_rows(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=scale,
                                 rows=all_rows(B, H, N), nthreads=nthreads)
    o = o_rows.reshape(B, H, N, D)
    if layout == "BSND":
        o = np.ascontiguousarray(o.transpose(0, 2, 1, 3))
    return o, lse.reshape(B, H, N)


def attention_rows_ex(q, k, v, *, dtype: str, layout: str, causal: bool, scale: float, rows, window: int = -1,
                      q_offset: int = 0, kv_start: int = 0, kv_len=None, nthreads: int = 1):
    """O and lse (fp64) of the requested rows under the generalised visibility rule of ``fa_oracle.c``:
    query row i sits at position q_offset + i, key j at position j, only keys in
    [kv_start, kv_start + kv_len) take part, causal hides keys after the query, and window >= 0 (with
    causal) hides keys more than ``window`` positions before it.  q is [B,H,Nq,D] / [B,Nq,H,D]; k and v
    are [B,H,Nk,D] / [B,Nk,H,D].  A row with no visible key gets O = 0 and lse = -inf.
    """
    if dtype not in DTYPES:
        raise ValueError("dtype must be one of %s" % sorted(DTYPES))
    B, H, Nq, D = _dims(q.shape, layout)
    Bk, Hk, Nk, Dk = _dims(k.shape, layout)
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape:
        raise ValueError("k and v must share a shape matching q in B, H and D")
    for t in (q, k, v):
        if t.dtype.itemsize != ITEMSIZE[dtype]:
            raise ValueError("q, k, v must have the itemsize of %s" % dtype)
    if kv_len is None:
        kv_len = Nk - kv_start
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    R = rows.shape[0]
    o = np.empty((R, D), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    if R == 0:
        return o, lse
    rc = _load().fa_oracle_rows_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, DTYPES[dtype], LAYOUTS[layout],
                                   B, H, Nq, Nk, D, 1 if causal else 0, int(window), int(q_offset),
                                   int(kv_start), int(kv_len), float(scale), rows.ctypes.data, R,
                                   o.ctypes.data, lse.ctypes.data, int(nthreads))
    if rc != 0:
        raise ValueError("fa_oracle_rows_ex failed with status %d" % rc)
    return o, lse


def attention_ex(q, k, v, *, dtype: str, layout: str, causal: bool, scale: float, window: int = -1,
                 q_offset: int = 0, kv_start: int = 0, kv_len=None, nthreads: int = 1):
    """Full O (in q's layout) and lse [B, H, Nq] under the generalised rule, in fp64."""
    B, H, Nq, D = _dims(q.shape, layout)
    o_rows, lse = attention_rows_ex(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=scale,
                                    rows=all_rows(B, H, Nq), window=window, q_offset=q_offset,
                                    kv_start=kv_start, kv_len=kv_len, nthreads=nthreads)
    o = o_rows.reshape(B, H, Nq, D)
    if layout == "BSND":
        o = np.ascontiguousarray(o.transpose(0, 2, 1, 3))
    return o, lse.reshape(B, H, Nq)


def merge(o_parts, lse_parts):
    """Combine partial results over disjoint key sets, in fp64.

    o_parts: sequence of arrays [..., D]; lse_parts: matching arrays [...] (natural-log lse of each part;
    -inf for a part with no visible key, whose O must be 0).  With M = max_s lse_s:
        lse = M + log(sum_s exp(lse_s - M)),   O = sum_s exp(lse_s - lse) * O_s,
    the two-term combination of page ai6s.net/6a140d07..., section "第二层：数值稳定性增强", applied to
    any number of parts.  Rows where every part has lse = -inf get O = 0 and lse = -inf.
    """
    lse_s = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])
    o_s = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])
    m = lse_s.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    total = np.exp(lse_s - m_safe).sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    w = np.exp(lse_s - np.where(empty, 0.0, lse))  # 0 for empty parts
    o = (w[..., None] * o_s).sum(axis=0)
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def attention_bwd(q, k, v, dout, *, dtype: str, layout: str, causal: bool, scale: float, heads=None,
                  nthreads: int = 1, mags: bool = False):
    """Gradients (dQ, dK, dV) of O = Softmax(scale Q K^T [+ causal]) V for upstream gradient ``dout``, in fp64.

    q, k, v, dout: stored elements as in ``attention_rows`` (same shape, dtype and layout).
    heads: None for every head -> three arrays in the input's layout; or a sequence of (b, h) pairs ->
    three arrays [len(heads), N, D] in that order.
    mags=True: six arrays, the gradients followed by their term magnitudes (MdQ, MdK, MdV of
    ``fa_oracle.c``, for per-element error bounds), laid out alike.
    """
    if dtype not in DTYPES:
        raise ValueError("dtype must be one of %s" % sorted(DTYPES))
    B, H, N, D = _dims(q.shape, layout)
    for t in (q, k, v, dout):
        if t.shape != q.shape or t.dtype.itemsize != ITEMSIZE[dtype]:
            raise ValueError("q, k, v, dout must share the shape and have the itemsize of %s" % dtype)
    q, k, v, dout = (np.ascontiguousarray(t) for t in (q, k, v, dout))
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else [tuple(x) for x in heads]
    nout = 6 if mags else 3
    out = [np.empty((len(sel), N, D), dtype=np.float64) for _ in range(nout)]
    for n, (b, h) in enumerate(sel):
        res = [np.empty((N, D), dtype=np.float64) for _ in range(nout)]
        if mags:
            rc = _load().fa_oracle_bwd_head_mag_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                                   DTYPES[dtype], LAYOUTS[layout], B, H, N, N, D, 1 if causal else 0,
                                                   -1, 0, 0, N, float(scale), int(b), int(h),
                                                   *[r.ctypes.data for r in res], int(nthreads))
        else:
            rc = _load().fa_oracle_bwd_head(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                            DTYPES[dtype], LAYOUTS[layout], B, H, N, D, 1 if causal else 0,
                                            float(scale), int(b), int(h), *[r.ctypes.data for r in res],
                                            int(nthreads))
        if rc != 0:
            raise ValueError("fa_oracle_bwd_head failed with status %d" % rc)
        for x, r in zip(out, res):
            x[n] = r
    if heads is not None:
        return tuple(out)
    res = []
    for g in out:
        g = g.reshape(B, H, N, D)
        if layout == "BSND":
            g = np.ascontiguousarray(g.transpose(0, 2, 1, 3))
        res.append(g)
    return tuple(res)


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, dtype: str, causal: bool, scale: float,
                     nthreads: int = 1):
    """O and lse (fp64) of a packed batch of sequences of different lengths.

    q: [total_q, H, D] and k, v: [total_k, H, D] stored elements (sequences one after another, each
    [len, H, D] as in the BSND layout); cu_seqlens_q / cu_seqlens_k: B + 1 non-decreasing offsets
    starting at 0.  Sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
    cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 and attends only to its own keys.  With causal, the two ends
    are aligned: query i of a sequence with Nq queries and Nk keys sits at position Nk - Nq + i and sees
    keys 0 .. Nk - Nq + i (the generalised rule of ``attention_rows_ex``).  A query with no visible key
    gets O = 0 and lse = -inf.  Returns (O [total_q, H, D], lse [H, total_q]).
    """
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    if len(cu_q) != len(cu_k) or len(cu_q) < 2 or cu_q[0] != 0 or cu_k[0] != 0:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 offsets starting at 0")
    if any(b < a for a, b in zip(cu_q, cu_q[1:])) or any(b < a for a, b in zip(cu_k, cu_k[1:])):
        raise ValueError("cu_seqlens must be non-decreasing")
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    if cu_q[-1] != q.shape[0] or cu_k[-1] != k.shape[0]:
        raise ValueError("the last offsets must equal total_q and total_k")
    total_q, H, D = q.shape
    o = np.zeros((total_q, H, D), dtype=np.float64)
    lse = np.full((H, total_q), -np.inf, dtype=np.float64)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        nq, nk = qe - qs, ke - ks
        if nq == 0 or nk == 0:
            continue  # no rows, or rows that see no key (O = 0, lse = -inf as initialised)
        ob, lb = attention_ex(q[qs:qe][None], k[ks:ke][None], v[ks:ke][None], dtype=dtype, layout="BSND",
                              causal=causal, scale=scale, q_offset=(nk - nq) if causal else 0,
                              nthreads=nthreads)
        o[qs:qe] = ob[0]
        lse[:, qs:qe] = lb[0]
    return o, lse


def attention_bwd_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, *, dtype: str, causal: bool, scale: float,
                         nthreads: int = 1, mags: bool = False):
    """Gradients (dQ, dK, dV) in fp64 of ``attention_varlen``'s packed batch for upstream gradient ``dout``.

    q, dout: [total_q, H, D]; k, v: [total_k, H, D]; offsets as in ``attention_varlen``.  Each sequence is
    independent: its gradients are ``attention_bwd_ex`` of its own rows (the BSND layout with B = 1) under
    the aligned-ends rule, query offset Nk - Nq when causal.  A sequence without queries contributes
    dK = dV = 0 for its keys; queries without keys get dQ = 0.  Returns (dQ [total_q, H, D], dK, dV
    [total_k, H, D]), followed with mags=True by their term magnitudes, laid out alike.
    """
    cu_q = [int(x) for x in cu_seqlens_q]
    cu_k = [int(x) for x in cu_seqlens_k]
    if len(cu_q) != len(cu_k) or len(cu_q) < 2 or cu_q[0] != 0 or cu_k[0] != 0:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 offsets starting at 0")
    if any(b < a for a, b in zip(cu_q, cu_q[1:])) or any(b < a for a, b in zip(cu_k, cu_k[1:])):
        raise ValueError("cu_seqlens must be non-decreasing")
    if q.ndim != 3 or k.ndim != 3 or v.shape != k.shape or q.shape[1:] != k.shape[1:] or dout.shape != q.shape:
        raise ValueError("q, dout must be [total_q, H, D] and k, v [total_k, H, D]")
    if cu_q[-1] != q.shape[0] or cu_k[-1] != k.shape[0]:
        raise ValueError("the last offsets must equal total_q and total_k")
    shapes = (q.shape, k.shape, k.shape) * (2 if mags else 1)
    out = [np.zeros(sh, dtype=np.float64) for sh in shapes]
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        nq, nk = qe - qs, ke - ks
        if nq == 0 or nk == 0:
            continue  # no queries (dK = dV = 0) or no keys (dQ = 0), as initialised
        res = attention_bwd_ex(q[qs:qe][None], k[ks:ke][None], v[ks:ke][None], dout[qs:qe][None], dtype=dtype,
                               layout="BSND", causal=causal, scale=scale, q_offset=(nk - nq) if causal else 0,
                               nthreads=nthreads, mags=mags)
        for n, r in enumerate(res):
            rows = slice(qs, qe) if n % 3 == 0 else slice(ks, ke)
            out[n][rows] = r[0]
    return tuple(out)


def attention_bwd_ex(q, k, v, dout, *, dtype: str, layout: str, causal: bool, scale: float, window: int = -1,
                     q_offset: int = 0, kv_start: int = 0, kv_len=None, heads=None, nthreads: int = 1,
                     mags: bool = False):
    """Generalised gradients in fp64, the backward of ``attention_ex``'s rule.

    q, dout: [B,H,Nq,D] / [B,Nq,H,D]; k, v: [B,H,Nk,D] / [B,Nk,H,D].  P and D are those of the softmax over
    every visible key of [0, Nk) (query i at q_offset + i, causal and window as in ``attention_rows_ex``);
    the key chunk [kv_start, kv_start + kv_len) restricts what is returned: dQ sums over the chunk's keys
    only, and dK, dV are 0 outside the chunk.  heads=None -> arrays in the input layout; a sequence of
    (b, h) -> arrays [len(heads), Nq or Nk, D].  mags=True: the three term magnitudes follow the gradients.
    """
    if dtype not in DTYPES:
        raise ValueError("dtype must be one of %s" % sorted(DTYPES))
    B, H, Nq, D = _dims(q.shape, layout)
    Bk, Hk, Nk, Dk = _dims(k.shape, layout)
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("k, v must share a shape matching q in B, H, D; dout must be shaped like q")
    for t in (q, k, v, dout):
        if t.dtype.itemsize != ITEMSIZE[dtype]:
            raise ValueError("q, k, v, dout must have the itemsize of %s" % dtype)
    if kv_len is None:
        kv_len = Nk - kv_start
    q, k, v, dout = (np.ascontiguousarray(t) for t in (q, k, v, dout))
    sel = [(b, h) for b in range(B) for h in range(H)] if heads is None else [tuple(x) for x in heads]
    rows = (Nq, Nk, Nk) * (2 if mags else 1)
    acc = [np.empty((len(sel), n, D)) for n in rows]
    for n, (b, h) in enumerate(sel):
        res = [np.empty((r, D)) for r in rows]
        ptrs = [r.ctypes.data for r in res] + ([] if mags else [None, None, None])
        rc = _load().fa_oracle_bwd_head_mag_ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data,
                                               DTYPES[dtype], LAYOUTS[layout], B, H, Nq, Nk, D, 1 if causal else 0,
                                               int(window), int(q_offset), int(kv_start), int(kv_len), float(scale),
                                               int(b), int(h), *ptrs, int(nthreads))
        if rc != 0:
            raise ValueError("fa_oracle_bwd_head_ex failed with status %d" % rc)
        for x, r in zip(acc, res):
            x[n] = r
    if heads is not None:
        return tuple(acc)
    out = []
    for g, n in zip(acc, rows):
        g = g.reshape(B, H, n, D)
        if layout == "BSND":
            g = np.ascontiguousarray(g.transpose(0, 2, 1, 3))
        out.append(g)
    return tuple(out)
