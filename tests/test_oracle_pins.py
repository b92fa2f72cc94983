"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-derived closed form (tests/golden), brute force on
tiny inputs, a library routine for a special case, or an invariant the mathematics of softmax attention
imposes.  Chosen so that a plausible slip in the oracle (a dropped scale, a wrong sign, an index or
layout mix-up, a transposed operand, an off-by-one in the causal range, a missing max subtraction, the
wrong log base) fails at least one of them (tests/test_oracle_mutants.py plants such slips).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests import bruteforce
from tests.ref_tiled import causal_tiles_per_head, tiled_attention
from transformer_attention_fwd_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f64(B, H, N, D, seed, mult=1.0):
    rng = np.random.default_rng([7, seed])
    q, k, v = (rng.standard_normal((B, H, N, D)) for _ in range(3))
    return q * mult, k * mult, v


def _run(q, k, v, *, causal, scale, layout="BHSD", dtype="fp64", nthreads=1):
    return oracle.attention(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=scale, nthreads=nthreads)


# --- closed form (hand-derived fixture) --------------------------------------------------------------

def test_closed_form_worked_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "closed_form_n2.txt")) if l.strip() and l[0] != "#"]
    q = np.array([1.0, 2.0]).reshape(1, 1, 2, 1)
    k = np.array([0.0, math.log(3.0)]).reshape(1, 1, 2, 1)
    v = np.array([4.0, 8.0]).reshape(1, 1, 2, 1)
    for causal in (0, 1):
        o, lse = _run(q, k, v, causal=bool(causal), scale=1.0)
        for c, i, o_ref, lse_ref in rows:
            if int(c) != causal:
                continue
            assert o[0, 0, int(i), 0] == pytest.approx(float(o_ref), rel=1e-14, abs=1e-14)
            assert lse[0, 0, int(i)] == pytest.approx(float(lse_ref), rel=1e-14, abs=1e-14)


# --- brute force on tiny inputs ----------------------------------------------------------------------

@pytest.mark.parametrize("N", [1, 2, 3, 7, 16, 33, 130])
@pytest.mark.parametrize("D", [1, 4, 8, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_bhsd(N, D, causal):
    B, H = 2, 2
    q, k, v = _f64(B, H, N, D, seed=N * 100 + D)
    scale = 1.0 / math.sqrt(D) * 1.7
    o, lse = _run(q, k, v, causal=causal, scale=scale)
    o_bf, lse_bf, _ = bruteforce.attention_bhsd(q, k, v, causal=causal, scale=scale)
    np.testing.assert_allclose(o, o_bf, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_bf, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_bruteforce_bsnd_layout(causal):
    B, H, N, D = 2, 3, 17, 8
    q, k, v = _f64(B, H, N, D, seed=11)
    t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    o, lse = _run(t(q), t(k), t(v), causal=causal, scale=0.3, layout="BSND")
    o_bf, lse_bf, _ = bruteforce.attention_bhsd(q, k, v, causal=causal, scale=0.3)
    np.testing.assert_allclose(o, t(o_bf), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_bf, rtol=0, atol=1e-12)


def test_negative_scale_bruteforce():
    q, k, v = _f64(1, 2, 9, 4, seed=3)
    o, lse = _run(q, k, v, causal=True, scale=-0.8)
    o_bf, lse_bf, _ = bruteforce.attention_bhsd(q, k, v, causal=True, scale=-0.8)
    np.testing.assert_allclose(o, o_bf, atol=1e-12)
    np.testing.assert_allclose(lse, lse_bf, atol=1e-12)


# --- library routine for the special case scale = 1/sqrt(D) ------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    B, H, N, D = 2, 2, 40, 16
    q, k, v = _f64(B, H, N, D, seed=5)
    o, _ = _run(q, k, v, causal=causal, scale=1.0 / math.sqrt(D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal).numpy()
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_lse_matches_torch_logsumexp():
    B, H, N, D = 1, 2, 23, 8
    q, k, v = _f64(B, H, N, D, seed=6)
    _, lse = _run(q, k, v, causal=False, scale=0.5)
    s = 0.5 * torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2)
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


# --- invariants ----------------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_identity_v_exposes_p_rows_sum_to_one(causal):
    # With D = N and V = I, O equals the probability matrix P itself.
    N = 12
    rng = np.random.default_rng(21)
    q = rng.standard_normal((1, 1, N, N))
    k = rng.standard_normal((1, 1, N, N))
    v = np.eye(N).reshape(1, 1, N, N)
    p, lse = _run(q, k, v, causal=causal, scale=0.4)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    s = 0.4 * q[0, 0] @ k[0, 0].T
    expect = np.exp(s - lse[0, 0][:, None])
    if causal:
        expect = np.tril(expect)
        assert np.all(np.triu(p[0, 0], k=1) == 0.0)
    np.testing.assert_allclose(p[0, 0], expect, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_gives_constant_output(causal):
    q, k, _ = _f64(1, 2, 31, 8, seed=8)
    v = np.full_like(q, -2.5)
    o, _ = _run(q, k, v, causal=causal, scale=0.9)
    np.testing.assert_allclose(o, -2.5, rtol=0, atol=1e-13)


def test_causal_row0_is_v0_and_lse0_is_s00():
    q, k, v = _f64(2, 2, 19, 8, seed=9)
    o, lse = _run(q, k, v, causal=True, scale=0.7)
    np.testing.assert_array_equal(o[:, :, 0, :], v[:, :, 0, :])
    np.testing.assert_allclose(lse[:, :, 0], 0.7 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)


def test_single_key():
    q, k, v = _f64(2, 3, 1, 8, seed=10)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal=causal, scale=0.25)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[..., 0], 0.25 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]), atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_scale_zero_gives_mean(causal):
    B, H, N, D = 1, 2, 13, 4
    q, k, v = _f64(B, H, N, D, seed=12)
    o, lse = _run(q, k, v, causal=causal, scale=0.0)
    if causal:
        mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        count = np.arange(1, N + 1)
    else:
        mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        count = np.full(N, N)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(count), lse.shape), rtol=0, atol=1e-14)


def test_noncausal_permutation_equivariance():
    q, k, v = _f64(1, 1, 21, 8, seed=13)
    o, lse = _run(q, k, v, causal=False, scale=0.6)
    rng = np.random.default_rng(1)
    pk, pq = rng.permutation(21), rng.permutation(21)
    o2, lse2 = _run(q[:, :, pq], k[:, :, pk], v[:, :, pk], causal=False, scale=0.6)
    np.testing.assert_allclose(o2, o[:, :, pq], atol=1e-13)
    np.testing.assert_allclose(lse2, lse[:, :, pq], atol=1e-13)


def test_causal_ignores_future_keys():
    N = 25
    q, k, v = _f64(1, 2, N, 8, seed=14)
    o, lse = _run(q, k, v, causal=True, scale=0.5)
    for i in (0, 7, 24):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] += 5.0
        v2[:, :, i + 1:] -= 3.0
        o2, lse2 = _run(q, k2, v2, causal=True, scale=0.5)
        np.testing.assert_array_equal(o2[:, :, i], o[:, :, i])
        np.testing.assert_array_equal(lse2[:, :, i], lse[:, :, i])
    # and a past key does matter
    k3 = k.copy()
    k3[:, :, 3] += 1.0
    o3, _ = _run(q, k3, v, causal=True, scale=0.5)
    assert np.abs(o3[:, :, 10] - o[:, :, 10]).max() > 1e-6


def test_key_shift_moves_lse_only():
    q, k, v = _f64(1, 2, 15, 8, seed=15)
    w = np.random.default_rng(2).standard_normal(8)
    for causal in (False, True):
        o, lse = _run(q, k, v, causal=causal, scale=0.45)
        o2, lse2 = _run(q, k + w, v, causal=causal, scale=0.45)
        np.testing.assert_allclose(o2, o, atol=1e-12)
        np.testing.assert_allclose(lse2 - lse, 0.45 * q @ w, atol=1e-12)


def test_lse_fsum_on_tiny_rows():
    q, k, v = _f64(1, 1, 6, 3, seed=16)
    _, lse = _run(q, k, v, causal=True, scale=1.3)
    for i in range(6):
        s = [1.3 * sum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(3)) for j in range(i + 1)]
        mx = max(s)
        assert lse[0, 0, i] == pytest.approx(mx + math.log(math.fsum(math.exp(x - mx) for x in s)), abs=1e-14)


def test_large_logits_one_hot_limit():
    # Logits of order 1e4: a naive exp overflows; the max-subtracted form must give v_argmax exactly.
    N, D = 9, 4
    q = np.zeros((1, 1, N, D))
    k = np.zeros((1, 1, N, D))
    q[0, 0, :, 0] = 100.0
    k[0, 0, :, 0] = np.arange(N) * 10.0   # s_ij = 1000 * j: key N-1 dominates by > 40
    v = np.random.default_rng(3).standard_normal((1, 1, N, D))
    o, lse = _run(q, k, v, causal=False, scale=1.0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(v[0, 0, N - 1], (N, D)), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], 1000.0 * (N - 1), rtol=1e-15)
    o, _ = _run(q, k, v, causal=True, scale=1.0)
    np.testing.assert_allclose(o[0, 0], v[0, 0], atol=1e-12)  # row i is dominated by key i


# --- stored element types --------------------------------------------------------------------------------

def test_fp16_and_bf16_widening_is_exact():
    # N = 1: O = v exactly, so the oracle returns the widened stored values.
    vals = np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 6.1e-5, 5.96e-8, 3.0e-6, 1e-3, 1234.5], dtype=np.float32)
    for dtype in ("fp16", "bf16"):
        bits = inputs.cast_bits(vals, dtype)
        v = bits.reshape(1, 1, 1, -1)
        q = np.zeros_like(v)
        o, _ = oracle.attention(q, q, v, dtype=dtype, layout="BHSD", causal=False, scale=1.0)
        if dtype == "fp16":
            expect = bits.view(np.float16).astype(np.float64)
        else:
            expect = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
        np.testing.assert_array_equal(o.ravel(), expect)


@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
def test_stored_dtypes_equal_fp64_of_widened(dtype):
    B, H, N, D = 1, 2, 20, 8
    qs, ks, vs = inputs.make(B, H, N, D, layout="BSND", dtype=dtype, seed=99)
    widen = {"fp32": lambda x: x.astype(np.float64),
             "fp16": lambda x: x.view(np.float16).astype(np.float64),
             "bf16": lambda x: inputs.bf16_bits_to_f32(x).astype(np.float64)}[dtype]
    o, lse = oracle.attention(qs, ks, vs, dtype=dtype, layout="BSND", causal=True, scale=0.35)
    o2, lse2 = oracle.attention(widen(qs), widen(ks), widen(vs), dtype="fp64", layout="BSND", causal=True, scale=0.35)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


# --- row subsets and threading -------------------------------------------------------------------------

def test_rows_subset_and_threads_agree_with_full():
    B, H, N, D = 2, 3, 37, 8
    q, k, v = _f64(B, H, N, D, seed=17)
    o, lse = _run(q, k, v, causal=True, scale=0.3)
    rows = inputs.sample_rows(B, H, N, 40, seed=1)
    for nt in (1, 3):
        o_r, lse_r = oracle.attention_rows(q, k, v, dtype="fp64", layout="BHSD", causal=True, scale=0.3,
                                           rows=rows, nthreads=nt)
        np.testing.assert_array_equal(o_r, o[rows[:, 0], rows[:, 1], rows[:, 2]])
        np.testing.assert_array_equal(lse_r, lse[rows[:, 0], rows[:, 1], rows[:, 2]])


def test_bad_arguments_rejected():
    q = np.zeros((1, 1, 4, 4))
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, dtype="fp64", layout="BHSD", causal=False, scale=1.0, rows=[[0, 0, 4]])
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, dtype="fp64", layout="XYZ", causal=False, scale=1.0, rows=[[0, 0, 0]])


# --- the tiled online-softmax recurrence equals the two-pass definition ---------------------------------

@pytest.mark.parametrize("bm,bn", [(4, 4), (8, 3), (3, 8), (16, 5), (128, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tau", [0.0, 8.0 * math.log(2.0)])
def test_tiled_recurrence_equals_two_pass(bm, bn, causal, tau):
    B, H, N, D = 1, 2, 37, 8
    q, k, v = _f64(B, H, N, D, seed=18, mult=2.0)
    o, lse = _run(q, k, v, causal=causal, scale=0.5)
    o_t, lse_t = tiled_attention(q, k, v, causal=causal, scale=0.5, bm=bm, bn=bn, tau=tau)
    np.testing.assert_allclose(o_t, o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse_t, lse, rtol=0, atol=1e-12)


def test_causal_tile_count_closed_form_and_page_table():
    # The visited count of the tiled model equals the closed form, for uneven tiles too.
    for (N, bm, bn) in [(37, 8, 3), (64, 16, 16), (130, 32, 64), (200, 64, 32)]:
        q = np.zeros((1, 1, N, 2))
        seen = []
        tiled_attention(q, q, q + 1.0, causal=True, scale=1.0, bm=bm, bn=bn, count_tiles=seen)
        assert seen[0] == causal_tiles_per_head(N, bm, bn)
    # Against the page's table of 128-row tiles: totals exact, skipped share about half.
    for line in open(os.path.join(GOLDEN, "causal_tile_table.txt")):
        if not line.strip() or line[0] == "#":
            continue
        N, total, skipped, pct = (int(x) for x in line.split())
        T = N // 128
        assert T * T == total
        visited = causal_tiles_per_head(N, 128, 128)
        assert visited == T * (T + 1) // 2
        assert abs((total - visited) - skipped) <= T // 2
        assert abs(100.0 * (total - visited) / total - pct) < 3.5
