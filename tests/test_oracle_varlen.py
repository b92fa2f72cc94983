"""Pins of the oracle's packed variable-length batch (oracle.attention_varlen): equal lengths reproduce
the plain batched oracle, each sequence matches an explicit-mask brute force with its own lengths (ends
aligned under causal), sequences do not see each other, and empty sequences are handled.

The backward (oracle.attention_bwd_varlen) is pinned by torch autograd through one attention over all
packed rows with a block-diagonal visibility mask (a formulation that never splits the batch), and by
equal lengths reproducing the batched gradients."""
import numpy as np
import pytest

import oracle
from tests import bruteforce


def _pack(rng, lens, H, D):
    return np.ascontiguousarray(rng.standard_normal((int(sum(lens)), H, D)))


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_match_batched(causal):
    rng = np.random.default_rng(71)
    B, N, H, D = 3, 17, 2, 8
    q, k, v = (np.ascontiguousarray(rng.standard_normal((B, N, H, D))) for _ in range(3))
    o_ref, lse_ref = oracle.attention(q, k, v, dtype="fp64", layout="BSND", causal=causal, scale=0.4)
    cu = _cu([N] * B)
    o, lse = oracle.attention_varlen(q.reshape(B * N, H, D), k.reshape(B * N, H, D), v.reshape(B * N, H, D), cu, cu,
                                     dtype="fp64", causal=causal, scale=0.4)
    np.testing.assert_allclose(o.reshape(B, N, H, D), o_ref, atol=1e-14)
    np.testing.assert_allclose(lse.reshape(H, B, N).transpose(1, 0, 2), lse_ref, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_each_sequence_against_bruteforce(causal):
    rng = np.random.default_rng(72 + causal)
    lq = [5, 0, 9, 3, 12, 1]
    lk = [5, 4, 6, 11, 0, 7]   # Nq > Nk, Nq < Nk, an empty query set, an empty key set
    H, D = 2, 8
    q, k, v = _pack(rng, lq, H, D), _pack(rng, lk, H, D), _pack(rng, lk, H, D)
    o, lse = oracle.attention_varlen(q, k, v, _cu(lq), _cu(lk), dtype="fp64", causal=causal, scale=0.6)
    cq, ck = _cu(lq), _cu(lk)
    for b in range(len(lq)):
        nq, nk = lq[b], lk[b]
        if nq == 0:
            continue
        qb = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
        if nk == 0:
            assert np.all(o[cq[b]:cq[b + 1]] == 0) and np.all(np.isneginf(lse[:, cq[b]:cq[b + 1]]))
            continue
        kb = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        vb = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        o_bf, lse_bf = bruteforce.attention_general(qb, kb, vb, causal=causal, scale=0.6,
                                                    q_offset=(nk - nq) if causal else 0)
        got_o = o[cq[b]:cq[b + 1]].transpose(1, 0, 2)
        np.testing.assert_allclose(got_o, o_bf[0], atol=1e-12)
        got_l = lse[:, cq[b]:cq[b + 1]]
        assert np.array_equal(np.isneginf(got_l), np.isneginf(lse_bf[0]))
        fin = np.isfinite(lse_bf[0])
        np.testing.assert_allclose(got_l[fin], lse_bf[0][fin], atol=1e-12)


def test_sequences_do_not_see_each_other():
    rng = np.random.default_rng(74)
    lens = [6, 9]
    H, D = 2, 4
    q, k, v = _pack(rng, lens, H, D), _pack(rng, lens, H, D), _pack(rng, lens, H, D)
    o1, l1 = oracle.attention_varlen(q, k, v, _cu(lens), _cu(lens), dtype="fp64", causal=False, scale=0.5)
    k2, v2 = k.copy(), v.copy()
    k2[6:] += 3.0
    v2[6:] -= 1.0
    o2, l2 = oracle.attention_varlen(q, k2, v2, _cu(lens), _cu(lens), dtype="fp64", causal=False, scale=0.5)
    np.testing.assert_array_equal(o1[:6], o2[:6])
    np.testing.assert_array_equal(l1[:, :6], l2[:, :6])
    assert not np.allclose(o1[6:], o2[6:])


def test_bad_offsets_rejected():
    z = np.zeros((4, 1, 4))
    with pytest.raises(ValueError):
        oracle.attention_varlen(z, z, z, [0, 3, 2, 4], [0, 1, 2, 4], dtype="fp64", causal=False, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_varlen(z, z, z, [1, 4], [0, 4], dtype="fp64", causal=False, scale=1.0)
    with pytest.raises(ValueError):
        oracle.attention_varlen(z, z, z, [0, 3], [0, 4], dtype="fp64", causal=False, scale=1.0)


def _packed_visibility(lq, lk, causal):
    """vis[i, j] over packed rows: same sequence and, when causal, key j_local <= Nk - Nq + i_local."""
    tq, tk = int(sum(lq)), int(sum(lk))
    vis = np.zeros((tq, tk), dtype=bool)
    cq, ck = _cu(lq), _cu(lk)
    for b, (nq, nk) in enumerate(zip(lq, lk)):
        for i in range(nq):
            hi = (nk - nq + i) if causal else nk - 1
            if hi >= 0:
                vis[cq[b] + i, ck[b]:ck[b] + min(hi, nk - 1) + 1] = True
    return vis


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_against_block_diagonal_autograd(causal):
    from tests.test_oracle_bwd import _torch_grads_general
    rng = np.random.default_rng(81 + causal)
    lq = [5, 0, 17, 1, 9, 4]
    lk = [7, 3, 17, 0, 4, 9]
    H, D, scale = 2, 16, 0.3
    q, k, v = _pack(rng, lq, H, D), _pack(rng, lk, H, D), _pack(rng, lk, H, D)
    do = _pack(rng, lq, H, D)
    dq, dk, dv = oracle.attention_bwd_varlen(q, k, v, do, _cu(lq), _cu(lk), dtype="fp64", causal=causal, scale=scale)
    vis = _packed_visibility(lq, lk, causal)
    for h in range(H):
        gq, gk, gv = _torch_grads_general(q[:, h], k[:, h], v[:, h], do[:, h], vis, scale)
        for got, ref in ((dq[:, h], gq), (dk[:, h], gk), (dv[:, h], gv)):
            np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # keys of the sequence without queries and queries of the sequence without keys get nothing
    assert not dk[_cu(lk)[1]:_cu(lk)[2]].any() and not dv[_cu(lk)[1]:_cu(lk)[2]].any()
    assert not dq[_cu(lq)[3]:_cu(lq)[4]].any()


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_equal_lengths_match_batched(causal):
    rng = np.random.default_rng(83 + causal)
    B, N, H, D = 3, 21, 2, 8
    q, k, v, do = (np.ascontiguousarray(rng.standard_normal((B, N, H, D))) for _ in range(4))
    ref = oracle.attention_bwd(q, k, v, do, dtype="fp64", layout="BSND", causal=causal, scale=0.25)
    cu = _cu([N] * B)
    got = oracle.attention_bwd_varlen(*(x.reshape(B * N, H, D) for x in (q, k, v, do)), cu, cu, dtype="fp64",
                                      causal=causal, scale=0.25)
    for g, r in zip(got, ref):
        assert np.array_equal(g.reshape(B, N, H, D), r)
