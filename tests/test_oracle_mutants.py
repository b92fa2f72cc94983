"""Plant plausible mistakes in a copy of the oracle's C source and check that the pins catch every one.

Runs on the CPU only: each mutant is compiled with gcc into a temporary directory and called through
ctypes; the committed oracle is never modified.
"""
import ctypes
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

from tests import bruteforce

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fa_oracle.c")

MUTANTS = {
    "dropped_scale": ("srow[j - jbeg] = J->scale * dot;", "srow[j - jbeg] = dot;"),
    "flipped_sign": ("srow[j - jbeg] = J->scale * dot;", "srow[j - jbeg] = -J->scale * dot;"),
    "causal_excludes_diagonal": ("if (J->causal && qpos + 1 < jend) jend = qpos + 1;",
                                 "if (J->causal && qpos < jend) jend = qpos > jbeg ? qpos : jbeg + 1;"),
    "causal_one_extra_key": ("if (J->causal && qpos + 1 < jend) jend = qpos + 1;",
                             "if (J->causal && qpos + 2 < jend) jend = qpos + 2;"),
    "no_max_subtraction": ("exp(srow[j - jbeg] - m)", "exp(srow[j - jbeg])"),
    "bsnd_read_as_bhsd": ("return ((b * N + i) * J->H + h) * J->D + d;", "return ((b * J->H + h) * N + i) * J->D + d;"),
    "key_row_index_is_query": ("qrow[d] * orc_load(J->k, J->dtype, orc_index(J, Nk, b, h, j, d))",
                               "qrow[d] * orc_load(J->k, J->dtype, orc_index(J, Nk, b, h, i, d))"),
    "value_row_index_is_query": ("e * orc_load(J->v, J->dtype, orc_index(J, Nk, b, h, j, d))",
                                 "e * orc_load(J->v, J->dtype, orc_index(J, Nk, b, h, i, d))"),
    "log2_lse": ("J->lse[r] = m + log(l);", "J->lse[r] = m + log2(l);"),
    "no_normalisation": ("o[d] /= l;", "o[d] /= 1.0;"),
    "fp16_exponent_bias": ("e - 25", "e - 24"),
    "bf16_wrong_half": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    # the generalised visibility rule
    "window_excludes_edge": ("if (J->window >= 0 && qpos - J->window > jbeg) jbeg = qpos - J->window;",
                             "if (J->window >= 0 && qpos - J->window + 1 > jbeg) jbeg = qpos - J->window + 1;"),
    "chunk_end_one_short": ("int64_t jbeg = J->kv_start, jend = J->kv_start + J->kv_len;",
                            "int64_t jbeg = J->kv_start, jend = J->kv_start + J->kv_len - 1;"),
    "chunk_start_ignored": ("int64_t jbeg = J->kv_start, jend = J->kv_start + J->kv_len;",
                            "int64_t jbeg = 0, jend = J->kv_start + J->kv_len;"),
    "q_offset_ignored": ("const int64_t qpos = J->q_offset + i;", "const int64_t qpos = i;"),
    "empty_row_lse_zero": ("J->lse[r] = -INFINITY;", "J->lse[r] = 0.0;"),
    "keys_indexed_with_query_length": ("qrow[d] * orc_load(J->k, J->dtype, orc_index(J, Nk, b, h, j, d))",
                                       "qrow[d] * orc_load(J->k, J->dtype, orc_index(J, Nq, b, h, j, d))"),
}


def _build(tmp, name, old, new):
    src = open(SRC).read()
    assert old == "" or src.count(old) == 1, name
    path = os.path.join(tmp, name + ".c")
    open(path, "w").write(src.replace(old, new) if old else src)
    lib = os.path.join(tmp, name + ".so")
    subprocess.check_call(["gcc", "-O1", "-shared", "-fPIC", "-pthread", path, "-o", lib, "-lm"])
    so = ctypes.CDLL(lib)
    f = so.fa_oracle_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_double,
                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    fx = so.fa_oracle_rows_ex
    fx.restype = ctypes.c_int
    fx.argtypes = ([ctypes.c_void_p] * 3 + [ctypes.c_int] * 2 + [ctypes.c_int64] * 5 + [ctypes.c_int] +
                   [ctypes.c_int64] * 4 + [ctypes.c_double, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p, ctypes.c_int])
    f.ex = fx
    return f


def _call(f, q, k, v, dtype, layout, causal, scale):
    B, X, Y, D = q.shape
    B, H, N = (B, X, Y) if layout == 0 else (B, Y, X)
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(N), indexing="ij")
    rows = np.ascontiguousarray(np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64))
    o = np.empty((rows.shape[0], D))
    lse = np.empty(rows.shape[0])
    rc = f(q.ctypes.data, k.ctypes.data, v.ctypes.data, dtype, layout, B, H, N, D, causal, scale,
           rows.ctypes.data, rows.shape[0], o.ctypes.data, lse.ctypes.data, 1)
    assert rc == 0
    return o.reshape(B, H, N, D), lse.reshape(B, H, N)


def _call_ex(f, q, k, v, causal, scale, q_offset, kv_start, kv_len, window):
    """fp64 BHSD call of the generalised entry point on every row."""
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    b, h, i = np.meshgrid(np.arange(B), np.arange(H), np.arange(Nq), indexing="ij")
    rows = np.ascontiguousarray(np.stack([b.ravel(), h.ravel(), i.ravel()], 1).astype(np.int64))
    o = np.empty((rows.shape[0], D))
    lse = np.empty(rows.shape[0])
    rc = f.ex(q.ctypes.data, k.ctypes.data, v.ctypes.data, 3, 0, B, H, Nq, Nk, D, causal, window, q_offset,
              kv_start, kv_len, scale, rows.ctypes.data, rows.shape[0], o.ctypes.data, lse.ctypes.data, 1)
    assert rc == 0
    return o.reshape(B, H, Nq, D), lse.reshape(B, H, Nq)


def _pins_pass(f):
    """A compact subset of the pins; True iff the library passes all of them."""
    rng = np.random.default_rng(6)
    # generalised rule against the explicit-mask brute force: bottom-right causal with Nq != Nk, a key
    # chunk with rows that see nothing, and a sliding window
    for (Nq, Nk, qoff, ks, kl, win) in ((5, 13, 8, 0, 13, -1), (6, 11, 2, 3, 6, 4), (7, 9, 2, 0, 9, 2)):
        q = np.ascontiguousarray(rng.standard_normal((1, 2, Nq, 8)))
        k = np.ascontiguousarray(rng.standard_normal((1, 2, Nk, 8)))
        v = np.ascontiguousarray(rng.standard_normal((1, 2, Nk, 8)))
        o, lse = _call_ex(f, q, k, v, 1, 0.4, qoff, ks, kl, win)
        o_bf, lse_bf = bruteforce.attention_general(q, k, v, causal=True, scale=0.4, q_offset=qoff, kv_start=ks,
                                                    kv_len=kl, window=win)
        if not (np.allclose(o, o_bf, atol=1e-12) and np.array_equal(np.isneginf(lse), np.isneginf(lse_bf))
                and np.allclose(lse[np.isfinite(lse_bf)], lse_bf[np.isfinite(lse_bf)], atol=1e-12)):
            return False
    rng = np.random.default_rng(5)
    for causal in (0, 1):
        q, k, v = (rng.standard_normal((2, 3, 11, 8)) for _ in range(3))
        o, lse = _call(f, q, k, v, 3, 0, causal, 0.4)
        o_bf, lse_bf, _ = bruteforce.attention_bhsd(q, k, v, causal=bool(causal), scale=0.4)
        if not (np.allclose(o, o_bf, atol=1e-12) and np.allclose(lse, lse_bf, atol=1e-12)):
            return False
        t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
        o2, lse2 = _call(f, t(q), t(k), t(v), 3, 1, causal, 0.4)
        if not (np.allclose(o2, o_bf, atol=1e-12) and np.allclose(lse2, lse_bf, atol=1e-12)):
            return False
    # large logits: a missing max subtraction overflows
    q = np.zeros((1, 1, 5, 2)); k = np.zeros((1, 1, 5, 2)); v = rng.standard_normal((1, 1, 5, 2))
    q[..., 0] = 100.0; k[0, 0, :, 0] = np.arange(5) * 10.0
    o, lse = _call(f, q, k, v, 3, 0, 0, 1.0)
    if not (np.allclose(o[0, 0], v[0, 0, 4], atol=1e-12) and np.allclose(lse, 4000.0)):
        return False
    # stored 16-bit types: N = 1 returns the widened v
    vals = np.array([1.0, -2.5, 6.1e-5, 1234.5], dtype=np.float32)
    for dt, bits, expect in ((1, vals.astype(np.float16).view(np.uint16), vals.astype(np.float16).astype(np.float64)),
                             (2, (vals.view(np.uint32) >> 16).astype(np.uint16),
                              ((vals.view(np.uint32) >> 16) << 16).view(np.float32).astype(np.float64))):
        vv = np.ascontiguousarray(bits.reshape(1, 1, 1, 4))
        o, _ = _call(f, np.zeros_like(vv), np.zeros_like(vv), vv, dt, 0, 0, 1.0)
        if not np.array_equal(o.ravel(), expect):
            return False
    return True


def test_unmutated_copy_passes():
    with tempfile.TemporaryDirectory() as tmp:
        assert _pins_pass(_build(tmp, "original", "", ""))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        assert not _pins_pass(_build(tmp, name, old, new)), "pins missed mutant " + name


# ---- backward pass -------------------------------------------------------------------------------
BWD_MUTANTS = {
    "bwd_delta_dropped": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * dp[j];"),
    "bwd_delta_sign": ("const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * (dp[j] + Di);"),
    "bwd_dk_unscaled": ("dkj[d] += J->scale * ds * qrow[d];", "dkj[d] += ds * qrow[d];"),
    "bwd_dq_unscaled": ("dqi[d] += J->scale * ds * orc_load", "dqi[d] += ds * orc_load"),
    "bwd_dv_uses_ds": ("dvj[d] += p[j] * dorow[d];", "dvj[d] += ds * dorow[d];"),
    "bwd_dk_uses_k": ("dkj[d] += J->scale * ds * qrow[d];",
                      "dkj[d] += J->scale * ds * orc_load(J->k, J->dtype, orc_bwd_index(J, Nk, j, d));"),
    "bwd_dp_uses_q": ("dot += dorow[d] * orc_load(J->v", "dot += qrow[d] * orc_load(J->v"),
    "bwd_unnormalised_p": ("for (int64_t j = jbeg; j < jend; ++j) p[j] /= l;",
                           "for (int64_t j = jbeg; j < jend; ++j) p[j] /= 1.0;"),
    "bwd_causal_extra_key": ("if (J->causal && jend > qpos + 1) jend = qpos + 1;",
                             "if (J->causal && jend > qpos + 2) jend = qpos + 2;"),
    "bwd_causal_not_applied": ("if (J->causal && jend > qpos + 1) jend = qpos + 1;", ""),
    "bwd_no_max_subtraction": ("p[j] = exp(p[j] - m);", "p[j] = exp(p[j]);"),
    "bwd_dv_row_is_query": ("double* dvj = J->dv + j * D;", "double* dvj = J->dv + (i % Nk) * D;"),
    "bwd_partials_last_worker_only": ("sk += jobs[t].dk[e];", "sk = jobs[t].dk[e];"),
    "bwd_bsnd_read_as_bhsd": ("if (J->layout == 0) return ((J->b * J->H + J->h) * N + i) * J->D + d;",
                              "return ((J->b * J->H + J->h) * N + i) * J->D + d;"),
    # the generalised rule
    "bwd_q_offset_ignored": ("const int64_t qpos = i + J->q_offset;", "const int64_t qpos = i;"),
    "bwd_window_edge": ("if (J->window >= 0 && jbeg < qpos - J->window) jbeg = qpos - J->window;",
                        "if (J->window >= 0 && jbeg < qpos - J->window + 1) jbeg = qpos - J->window + 1;"),
    "bwd_chunk_restriction_ignored": ("const int64_t kb = jbeg > c0 ? jbeg : c0, ke = jend < c1 ? jend : c1;",
                                      "const int64_t kb = jbeg, ke = jend;"),
    "bwd_softmax_over_chunk_only": ("int64_t jbeg = 0, jend = Nk;", "int64_t jbeg = c0, jend = c1;"),
}


def _build_bwd(tmp, name, old, new):
    src = open(SRC).read()
    assert old == "" or src.count(old) == 1, name
    path = os.path.join(tmp, name + ".c")
    open(path, "w").write(src.replace(old, new) if old else src)
    lib = os.path.join(tmp, name + ".so")
    subprocess.check_call(["gcc", "-O1", "-shared", "-fPIC", "-pthread", path, "-o", lib, "-lm"])
    so = ctypes.CDLL(lib)
    f = so.fa_oracle_bwd_head
    f.restype = ctypes.c_int
    f.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int] * 2 + [ctypes.c_int64] * 4 + [ctypes.c_int, ctypes.c_double]
                  + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 3 + [ctypes.c_int])
    fx = so.fa_oracle_bwd_head_ex
    fx.restype = ctypes.c_int
    fx.argtypes = ([ctypes.c_void_p] * 4 + [ctypes.c_int] * 2 + [ctypes.c_int64] * 5 + [ctypes.c_int]
                   + [ctypes.c_int64] * 4 + [ctypes.c_double] + [ctypes.c_int64] * 2 + [ctypes.c_void_p] * 3
                   + [ctypes.c_int])
    f.ex = fx
    return f


def _bwd_call(f, q, k, v, dout, layout, causal, scale, nthreads):
    if layout == 0:
        B, H, N, D = q.shape
    else:
        B, N, H, D = q.shape
    outs = [np.empty((B, H, N, D)) for _ in range(3)]
    for b in range(B):
        for h in range(H):
            g = [np.empty((N, D)) for _ in range(3)]
            rc = f(q.ctypes.data, k.ctypes.data, v.ctypes.data, dout.ctypes.data, 3, layout, B, H, N, D, causal,
                   scale, b, h, g[0].ctypes.data, g[1].ctypes.data, g[2].ctypes.data, nthreads)
            assert rc == 0
            for o, x in zip(outs, g):
                o[b, h] = x
    return outs


def _torch_ref(q, k, v, dout, causal, scale):
    import torch
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1), float("-inf"))
    (torch.softmax(s, dim=-1) @ tv).backward(torch.tensor(dout))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _bwd_pins_pass(f):
    rng = np.random.default_rng(8)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    for causal in (0, 1):
        q, k, v, dout = (np.ascontiguousarray(rng.standard_normal((1, 2, 9, 4))) for _ in range(4))
        ref = _torch_ref(q, k, v, dout, causal, 0.6)
        for layout, args, back in ((0, (q, k, v, dout), lambda x: x), (1, tuple(map(t, (q, k, v, dout))), lambda x: x)):
            got = _bwd_call(f, *args, layout, causal, 0.6, 3)
            for g, r in zip(got, ref):
                if not np.allclose(g, r, atol=1e-11):
                    return False
    # large logits: exponentials without the maximum overflow
    q = np.zeros((1, 1, 5, 2)); k = np.zeros((1, 1, 5, 2))
    v = np.ascontiguousarray(rng.standard_normal((1, 1, 5, 2))); dout = np.ascontiguousarray(rng.standard_normal((1, 1, 5, 2)))
    q[..., 0] = 100.0; k[0, 0, :, 0] = np.arange(5) * 2.0 + np.array([0, 0, 0, 5.0, 3.001])
    got = _bwd_call(f, q, k, v, dout, 0, 0, 1.0, 1)
    ref = _torch_ref(q, k, v, dout, 0, 1.0)
    if not all(np.all(np.isfinite(g)) and np.allclose(g, r, atol=1e-9) for g, r in zip(got, ref)):
        return False
    # generalised rows: offset + window against the explicit-mask autograd, and chunk partials adding up
    from tests.test_oracle_bwd import _torch_grads_general, _vis
    Nq, Nk, qoff, win = 5, 9, 4, 3
    q, dout = rng.standard_normal((Nq, 4)), rng.standard_normal((Nq, 4))
    k, v = rng.standard_normal((Nk, 4)), rng.standard_normal((Nk, 4))

    def ex(ks, kl):
        dq, dk, dv = np.empty((Nq, 4)), np.empty((Nk, 4)), np.empty((Nk, 4))
        args = [np.ascontiguousarray(x) for x in (q, k, v, dout)]
        rc = f.ex(*[a.ctypes.data for a in args], 3, 0, 1, 1, Nq, Nk, 4, 1, win, qoff, ks, kl, 0.7, 0, 0,
                  dq.ctypes.data, dk.ctypes.data, dv.ctypes.data, 2)
        assert rc == 0
        return dq, dk, dv
    full = ex(0, Nk)
    ref = _torch_grads_general(q, k, v, dout, _vis(Nq, Nk, True, win, qoff), 0.7)
    if not all(np.allclose(g, r, atol=1e-11) for g, r in zip(full, ref)):
        return False
    a, b = ex(0, 5), ex(5, 4)
    if not (np.allclose(a[0] + b[0], full[0], atol=1e-13) and np.allclose(a[1][:5], full[1][:5], atol=1e-14)
            and np.allclose(b[1][5:], full[1][5:], atol=1e-14) and np.all(a[1][5:] == 0) and np.all(b[2][:5] == 0)):
        return False
    return True


def test_unmutated_copy_passes_backward_pins():
    with tempfile.TemporaryDirectory() as tmp:
        assert _bwd_pins_pass(_build_bwd(tmp, "original_bwd", "", ""))


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_mutant_is_caught(name):
    old, new = BWD_MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        assert not _bwd_pins_pass(_build_bwd(tmp, name, old, new)), "backward pins missed mutant " + name
