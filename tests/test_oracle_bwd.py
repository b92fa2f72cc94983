"""Pins of the oracle's backward pass (gradients of the forward) against what mathematics fixes.

* central finite differences of the (separately pinned) forward oracle: the gradient is the limit of
  difference quotients of L = sum(dO * O), whatever formula produced it;
* torch autograd in float64 on the CPU through the plain definition (explicit scores, mask, softmax,
  product), an independent library differentiation;
* identities of softmax attention: sum_j dK_j = 0 (softmax is shift invariant per row), sum_j dV_j =
  sum_i dO_i (rows of P sum to 1), dQ = dK = 0 when every key has the same value row, dQ of causal row 0
  is 0 (it sees one key), and the closed form at scale 0 (uniform P);
* stored 16-bit inputs are read exactly.
"""
import numpy as np
import pytest

import oracle


def _rand(rng, shape, s=1.0):
    return np.ascontiguousarray(rng.standard_normal(shape) * s)


def _loss(q, k, v, dout, causal, scale, layout="BHSD"):
    o, _ = oracle.attention(q, k, v, dtype="fp64", layout=layout, causal=causal, scale=scale)
    return float((o * dout).sum())


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
def test_finite_differences(causal, layout):
    rng = np.random.default_rng(11 + causal)
    shape = (1, 2, 6, 3) if layout == "BHSD" else (1, 6, 2, 3)
    q, k, v, dout = (_rand(rng, shape) for _ in range(4))
    scale = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout=layout, causal=causal, scale=scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dout, causal, scale, layout)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dout, causal, scale, layout)
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, rtol=0, err_msg=name)


def _torch_grads(q, k, v, dout, causal, scale):
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    if causal:
        n = q.shape[2]
        s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), diagonal=1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ tv
    o.backward(torch.tensor(dout, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("logit_scale", [1.0, 8.0])
def test_against_torch_autograd(causal, logit_scale):
    rng = np.random.default_rng(21 + causal)
    shape = (2, 3, 37, 16)
    q, k = _rand(rng, shape, logit_scale), _rand(rng, shape, logit_scale)
    v, dout = _rand(rng, shape), _rand(rng, shape)
    scale = 0.25
    got = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=causal, scale=scale, nthreads=3)
    ref = _torch_grads(q, k, v, dout, causal, scale)
    for name, g, r in zip("qkv", got, ref):
        np.testing.assert_allclose(g, r, atol=1e-11 * max(1.0, np.abs(r).max()), rtol=0, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
def test_identities(causal):
    rng = np.random.default_rng(31)
    shape = (1, 2, 19, 8)
    q, k, v, dout = (_rand(rng, shape) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=causal, scale=0.5)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=2), dout.sum(axis=2), atol=1e-12)
    if causal:
        np.testing.assert_allclose(dq[:, :, 0], 0.0, atol=1e-14)
        # the last key is seen only by the last query: dV_{N-1} = P_{N-1,N-1} dO_{N-1}
        o, lse = oracle.attention(q, k, v, dtype="fp64", layout="BHSD", causal=True, scale=0.5)
        p_last = np.exp(0.5 * (q[:, :, -1] * k[:, :, -1]).sum(-1) - lse[:, :, -1])
        np.testing.assert_allclose(dv[:, :, -1], p_last[..., None] * dout[:, :, -1], atol=1e-13)
    # the same value row for every key: O does not depend on Q or K
    vc = np.ascontiguousarray(np.broadcast_to(v[:, :, :1], shape))
    dq2, dk2, _ = oracle.attention_bwd(q, k, vc, dout, dtype="fp64", layout="BHSD", causal=causal, scale=0.5)
    np.testing.assert_allclose(dq2, 0.0, atol=1e-13)
    np.testing.assert_allclose(dk2, 0.0, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_closed_form(causal):
    rng = np.random.default_rng(41)
    shape = (1, 1, 9, 4)
    q, k, v, dout = (_rand(rng, shape) for _ in range(4))
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=causal, scale=0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    N = shape[2]
    expect = np.zeros(shape)
    for i in range(N):
        vis = range(i + 1) if causal else range(N)
        for j in vis:
            expect[0, 0, j] += dout[0, 0, i] / len(vis)
    np.testing.assert_allclose(dv, expect, atol=1e-14)


@pytest.mark.parametrize("dt", ["fp16", "bf16", "fp32"])
def test_stored_types_read_exactly(dt):
    rng = np.random.default_rng(51)
    shape = (1, 2, 11, 8)
    x = [rng.standard_normal(shape).astype(np.float32) for _ in range(4)]
    if dt == "fp16":
        stored = [a.astype(np.float16) for a in x]
        wide = [a.astype(np.float64) for a in stored]
    elif dt == "bf16":
        stored = [(a.view(np.uint32) >> 16).astype(np.uint16) for a in x]
        wide = [(s.astype(np.uint32) << 16).view(np.float32).astype(np.float64) for s in stored]
    else:
        stored = x
        wide = [a.astype(np.float64) for a in x]
    got = oracle.attention_bwd(*stored, dtype=dt, layout="BHSD", causal=True, scale=0.3)
    ref = oracle.attention_bwd(*wide, dtype="fp64", layout="BHSD", causal=True, scale=0.3)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


def test_head_selection_and_threads():
    rng = np.random.default_rng(61)
    shape = (2, 3, 23, 8)
    q, k, v, dout = (_rand(rng, shape) for _ in range(4))
    full = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=True, scale=0.4)
    sel = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=True, scale=0.4,
                               heads=[(1, 2), (0, 1)], nthreads=5)
    for f, s in zip(full, sel):
        np.testing.assert_allclose(s[0], f[1, 2], atol=1e-14)
        np.testing.assert_allclose(s[1], f[0, 1], atol=1e-14)


def test_bad_arguments():
    q = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, q, q, np.zeros((1, 1, 4, 3)), dtype="fp64", layout="BHSD", causal=False, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_bwd(q, q, q, q, dtype="fp64", layout="BHSD", causal=False, scale=1.0, heads=[(0, 1)])


# ---- generalised rows: query offset, N_q != N_k, window, key chunk ------------------------------------

def _vis(Nq, Nk, causal, window, q_offset):
    qpos = q_offset + np.arange(Nq)[:, None]
    kpos = np.arange(Nk)[None, :]
    vis = np.ones((Nq, Nk), dtype=bool)
    if causal:
        vis &= kpos <= qpos
    if window >= 0:
        vis &= kpos >= qpos - window
    return vis


def _torch_grads_general(q, k, v, dout, vis, scale):
    """Autograd of the explicit-mask attention; rows that see no key have O = 0 (their gradients vanish)."""
    import torch
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * (tq @ tk.transpose(-1, -2))
    m = torch.tensor(vis)
    s = s.masked_fill(~m, float("-inf"))
    any_vis = m.any(dim=-1)
    s = torch.where(any_vis[:, None], s, torch.zeros_like(s))  # keep softmax finite on empty rows
    p = torch.softmax(s, dim=-1) * any_vis[:, None]
    (p @ tv).backward(torch.tensor(dout, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def test_ex_defaults_equal_plain():
    rng = np.random.default_rng(81)
    q, k, v, dout = (_rand(rng, (1, 2, 21, 8)) for _ in range(4))
    a = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout="BHSD", causal=True, scale=0.4)
    b = oracle.attention_bwd_ex(q, k, v, dout, dtype="fp64", layout="BHSD", causal=True, scale=0.4)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("Nq,Nk,causal,window,q_offset", [
    (5, 9, True, -1, 4),    # bottom-right causal, prefill with a key cache
    (7, 7, True, 2, 0),     # sliding window
    (6, 11, True, 3, 5),    # both
    (6, 8, True, -1, -2),   # negative offset: the first rows see nothing
    (5, 7, False, -1, 0),   # N_q != N_k without a mask
])
def test_ex_finite_differences_and_autograd(Nq, Nk, causal, window, q_offset):
    rng = np.random.default_rng([82, Nq, Nk, window + 2, q_offset + 10])
    q, dout = _rand(rng, (1, 1, Nq, 3)), _rand(rng, (1, 1, Nq, 3))
    k, v = _rand(rng, (1, 1, Nk, 3)), _rand(rng, (1, 1, Nk, 3))
    scale = 0.8
    kw = dict(dtype="fp64", layout="BHSD", causal=causal, scale=scale, window=window, q_offset=q_offset)
    dq, dk, dv = oracle.attention_bwd_ex(q, k, v, dout, **kw)
    # torch autograd of the explicit-mask definition
    ref = _torch_grads_general(q[0, 0], k[0, 0], v[0, 0], dout[0, 0], _vis(Nq, Nk, causal, window, q_offset), scale)
    for g, r in zip((dq, dk, dv), ref):
        np.testing.assert_allclose(g[0, 0], r, atol=1e-11)
    # central differences of the forward oracle's generalised rows
    eps = 1e-6

    def loss(qq, kk, vv):
        o, _ = oracle.attention_ex(qq, kk, vv, **{x: kw[x] for x in kw if x != "scale"}, scale=scale)
        return float((o * dout).sum())

    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=2e-8, err_msg=name)


@pytest.mark.parametrize("cuts", [(0, 4, 9, 13), (0, 1, 13), (0, 7, 7, 13)])
def test_ex_chunks_add_up(cuts):
    rng = np.random.default_rng(83)
    Nq, Nk = 6, 13
    q, dout = _rand(rng, (1, 2, Nq, 4)), _rand(rng, (1, 2, Nq, 4))
    k, v = _rand(rng, (1, 2, Nk, 4)), _rand(rng, (1, 2, Nk, 4))
    kw = dict(dtype="fp64", layout="BHSD", causal=True, scale=0.5, window=5, q_offset=Nk - Nq)
    full = oracle.attention_bwd_ex(q, k, v, dout, **kw)
    dq_sum = np.zeros_like(full[0])
    for a, b in zip(cuts, cuts[1:]):
        dq, dk, dv = oracle.attention_bwd_ex(q, k, v, dout, **kw, kv_start=a, kv_len=b - a)
        dq_sum += dq
        np.testing.assert_allclose(dk[:, :, a:b], full[1][:, :, a:b], atol=1e-14)
        np.testing.assert_allclose(dv[:, :, a:b], full[2][:, :, a:b], atol=1e-14)
        assert np.all(dk[:, :, :a] == 0) and np.all(dk[:, :, b:] == 0) and np.all(dv[:, :, :a] == 0)
    np.testing.assert_allclose(dq_sum, full[0], atol=1e-13)


def test_ex_bad_arguments():
    z = np.zeros((1, 1, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_bwd_ex(z, z, z, z, dtype="fp64", layout="BHSD", causal=False, scale=1.0, window=2)
    with pytest.raises(ValueError):
        oracle.attention_bwd_ex(z, z, z, z, dtype="fp64", layout="BHSD", causal=True, scale=1.0, kv_start=3, kv_len=2)


# ---- term magnitudes (the per-element error bounds of the GPU backward tests are multiples of them) ----
def _mags(q, k, v, dout, causal, scale, layout="BHSD", **ex):
    return oracle.attention_bwd_ex(q, k, v, dout, dtype="fp64", layout=layout, causal=causal, scale=scale,
                                   mags=True, **ex)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
def test_mags_bound_their_gradients(causal, layout):
    # |sum of terms| <= sum of |terms|: each magnitude is at least its gradient's absolute value, and the
    # gradients returned beside them are those of the plain call
    rng = np.random.default_rng(31 + causal)
    shape = (2, 3, 70, 16) if layout == "BHSD" else (2, 70, 3, 16)
    q, k, v, dout = (_rand(rng, shape) for _ in range(4))
    res = _mags(q, k, v, dout, causal, 0.4, layout)
    plain = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout=layout, causal=causal, scale=0.4)
    via_plain = oracle.attention_bwd(q, k, v, dout, dtype="fp64", layout=layout, causal=causal, scale=0.4, mags=True)
    for n in range(3):
        np.testing.assert_array_equal(res[n], plain[n])
        np.testing.assert_array_equal(via_plain[n], plain[n])
        np.testing.assert_array_equal(via_plain[n + 3], res[n + 3])
        assert np.all(res[n + 3] >= np.abs(res[n]) * (1 - 1e-12))
        assert np.all(res[n + 3] > 0)


def test_mags_single_key_closed_form():
    # one key: P = 1, dS = 0 and A = sum_d |dO_d| |v_d|, so MdQ = |scale| |k_d| A, MdK = |scale| |q_d| A,
    # MdV = |dO_d|
    rng = np.random.default_rng(33)
    q, k, v, dout = (_rand(rng, (1, 2, 1, 8)) for _ in range(4))
    scale = -0.3
    _, _, _, mq, mk, mv = _mags(q, k, v, dout, True, scale)
    a = (np.abs(dout) * np.abs(v)).sum(-1, keepdims=True)
    np.testing.assert_allclose(mq, abs(scale) * np.abs(k) * a, rtol=1e-14)
    np.testing.assert_allclose(mk, abs(scale) * np.abs(q) * a, rtol=1e-14)
    np.testing.assert_array_equal(mv, np.abs(dout))


@pytest.mark.parametrize("causal", [False, True])
def test_mags_dv_column_sums(causal):
    # rows of P sum to 1, so sum_j MdV_jd = sum_i |dO_id| for every head and d
    rng = np.random.default_rng(35)
    q, k, v, dout = (_rand(rng, (1, 2, 50, 8)) for _ in range(4))
    mv = _mags(q, k, v, dout, causal, 0.5)[5]
    np.testing.assert_allclose(mv.sum(2), np.abs(dout).sum(2), rtol=1e-12)


def test_mags_linear_in_dout():
    # dS, D and A are linear in dO and P does not depend on it: doubling dO (exact in binary) doubles every
    # magnitude exactly, and its sign does not matter
    rng = np.random.default_rng(37)
    q, k, v, dout = (_rand(rng, (1, 2, 40, 8)) for _ in range(4))
    a = _mags(q, k, v, dout, True, 0.6)
    b = _mags(q, k, v, 2.0 * dout, True, 0.6)
    c = _mags(q, k, v, -dout, True, 0.6)
    for n in range(3, 6):
        np.testing.assert_array_equal(b[n], 2.0 * a[n])
        np.testing.assert_array_equal(c[n], a[n])


@pytest.mark.parametrize("cuts", [(0, 13, 40), (0, 1, 2, 40)])
def test_mags_of_key_chunks_partition(cuts):
    # every (i, j) term belongs to one chunk: the chunks' MdQ add up to the whole call's, and each chunk's
    # MdK, MdV rows are the whole call's rows of its keys (0 elsewhere)
    rng = np.random.default_rng(39)
    q, k, v, dout = (_rand(rng, (1, 1, 40, 8)) for _ in range(4))
    whole = _mags(q, k, v, dout, True, 0.5, window=17)
    mq = np.zeros_like(whole[3])
    for a, b in zip(cuts, cuts[1:]):
        part = _mags(q, k, v, dout, True, 0.5, window=17, kv_start=a, kv_len=b - a)
        mq += part[3]
        np.testing.assert_allclose(part[4][:, :, a:b], whole[4][:, :, a:b], rtol=1e-13)
        np.testing.assert_allclose(part[5][:, :, a:b], whole[5][:, :, a:b], rtol=1e-13)
        assert not part[4][:, :, :a].any() and not part[4][:, :, b:].any()
    np.testing.assert_allclose(mq, whole[3], rtol=1e-12)


def test_mags_brute_force_tiny():
    # the definitions evaluated directly with numpy on a tiny causal head
    rng = np.random.default_rng(41)
    n, d, scale = 5, 4, 0.8
    q, k, v, dout = (_rand(rng, (1, 1, n, d)) for _ in range(4))
    _, _, _, mq, mk, mv = _mags(q, k, v, dout, True, scale)
    Q, K, V, dO = q[0, 0], k[0, 0], v[0, 0], dout[0, 0]
    s = scale * Q @ K.T
    s[np.triu_indices(n, 1)] = -np.inf
    P = np.exp(s - s.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    dP = dO @ V.T
    dS = P * (dP - (P * dP).sum(1, keepdims=True))
    A = (np.abs(dO) * (P @ np.abs(V))).sum(1)
    W = abs(scale) * (np.abs(dS) + P * A[:, None])
    np.testing.assert_allclose(mq[0, 0], W @ np.abs(K), rtol=1e-12)
    np.testing.assert_allclose(mk[0, 0], W.T @ np.abs(Q), rtol=1e-12)
    np.testing.assert_allclose(mv[0, 0], P.T @ np.abs(dO), rtol=1e-12)
