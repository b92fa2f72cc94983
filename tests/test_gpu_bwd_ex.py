"""GPU parity of the generalised backward (fa_bwd_ex through the C ABI) against the oracle's fp64 gradients.

The GPU side runs the library's forward over every key (fa_fwd_ex with the same query offset and
window) for O and lse, then fa_bwd_ex, possibly once per key chunk; the oracle computes the chunk's
dQ part and its dK, dV rows from Q, K, V and dO alone (``oracle.attention_bwd_ex``), with each element's
term magnitude.  Every element must lie within the per-element bound of tests/bwd_bound.py (the same
roundings as fa_bwd's; the dQ parts of a chunked call are each rounded once, and their magnitudes add up
to the whole call's, so their sum meets the bound of the whole).
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs
from tests import bwd_bound

pytestmark = pytest.mark.gpu
NTHREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits, dtype):
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to("cuda")
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
        torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.to("cuda")


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def check(name, g, r, m, what, dtype, n, d, abs_term=bwd_bound.ATOL):
    bwd_bound.check(name, g, r, m, dtype, n, d, what, abs_term)


def make_case(B, H, Nq, Nk, D, dtype, layout, seed):
    rng_seed = [seed, Nq, Nk, D]
    q, _, _ = inputs.make(B, H, Nq, D, layout=layout, dtype=dtype, seed=rng_seed + [1])
    _, k, v = inputs.make(B, H, Nk, D, layout=layout, dtype=dtype, seed=rng_seed + [2])
    do = inputs.make_grad(B, H, Nq, D, layout=layout, dtype=dtype, seed=rng_seed)
    return q, k, v, do


def forward(dev, layout, causal, scale, window, q_offset):
    o, lse = fa.attention_ex(dev[0], dev[1], dev[2], layout=layout, causal=causal, scale=scale, window=window,
                             q_offset=q_offset)
    return o, lse


def compare_chunks(B, H, Nq, Nk, D, *, dtype="bf16", layout="BHSD", causal=True, window=-1, q_offset=0,
                   chunks=None, seed=0, what="bwd_ex"):
    """Run fa_bwd_ex once per key chunk into one dk/dv; check each dQ part, the dQ sum and dK, dV."""
    scale = float(np.float32(1 / np.sqrt(D)))
    chunks = chunks or [(0, Nk)]
    n = max(Nq, Nk)
    q, k, v, do = make_case(B, H, Nq, Nk, D, dtype, layout, seed)
    at = bwd_bound.atol(dtype, n, scale, q, k, do)
    _say("%s: B=%d H=%d Nq=%d Nk=%d D=%d %s %s causal=%d window=%d q_offset=%d chunks=%s" %
         (what, B, H, Nq, Nk, D, dtype, layout, causal, window, q_offset, chunks))
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    o, lse = forward(dev, layout, causal, scale, window, q_offset)
    dk = torch.zeros_like(dev[1])
    dv = torch.zeros_like(dev[2])
    dq_sum = torch.zeros(dev[0].shape, dtype=torch.float64, device="cuda")
    for (s, e) in chunks:
        dq, dk, dv = fa.attention_bwd_ex(dev[0], dev[1], dev[2], o, lse, dev[3], layout=layout, causal=causal,
                                         scale=scale, window=window, q_offset=q_offset, kv_start=s, kv_len=e - s,
                                         dk=dk, dv=dv)
        torch.cuda.synchronize()
        ref = oracle.attention_bwd_ex(q, k, v, do, dtype=dtype, layout=layout, causal=causal, scale=scale,
                                      window=window, q_offset=q_offset, kv_start=s, kv_len=e - s, nthreads=NTHREADS,
                                      mags=True)
        check("dQ[%d:%d]" % (s, e), f64(dq), ref[0], ref[3], what, dtype, n, D, at)
        dq_sum += dq.double()
    full = oracle.attention_bwd_ex(q, k, v, do, dtype=dtype, layout=layout, causal=causal, scale=scale,
                                   window=window, q_offset=q_offset, nthreads=NTHREADS, mags=True)
    if len(chunks) > 1:
        check("sum dQ", dq_sum.cpu().numpy(), full[0], full[3], what, dtype, n, D, len(chunks) * at)
    check("dK", f64(dk), full[1], full[4], what, dtype, n, D, at)
    check("dV", f64(dv), full[2], full[5], what, dtype, n, D, at)
    return dev, o, lse


@pytest.mark.parametrize("Nq,Nk", [(1, 300), (64, 200), (100, 357), (129, 129), (256, 1000), (300, 64)])
@pytest.mark.parametrize("D", [64, 128])
def test_bottom_right_causal(Nq, Nk, D):
    # the queries are the last Nq positions of the key sequence (prefill behind a cache); Nq > Nk puts
    # the first queries before every key
    compare_chunks(1, 2, Nq, Nk, D, q_offset=Nk - Nq, seed=1, what="bwd_ex bottom-right")


@pytest.mark.parametrize("Nq,Nk", [(70, 333), (200, 130)])
@pytest.mark.parametrize("D", [64, 128])
def test_non_causal_unequal_lengths(Nq, Nk, D):
    compare_chunks(2, 2, Nq, Nk, D, causal=False, seed=2, what="bwd_ex non-causal")


@pytest.mark.parametrize("window", [0, 1, 63, 64, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_sliding_window(window, D):
    compare_chunks(1, 3, 333, 333, D, window=window, seed=3, what="bwd_ex window")


@pytest.mark.parametrize("window", [1, 100])
def test_sliding_window_fp16(window):
    compare_chunks(1, 2, 333, 333, 128, dtype="fp16", window=window, q_offset=0, chunks=[(0, 129), (129, 333)],
                   seed=14, what="bwd_ex window fp16")


def test_window_with_offset_and_short_keys():
    # positions 100 .. 249 against 250 keys, window 77
    compare_chunks(2, 2, 150, 250, 128, window=77, q_offset=100, seed=4, what="bwd_ex window offset")


@pytest.mark.parametrize("causal,window,q_offset", [(False, -1, 0), (True, -1, 0), (True, -1, 120), (True, 90, 30)])
@pytest.mark.parametrize("D", [64, 128])
def test_key_chunks_add_up(causal, window, q_offset, D):
    # uneven chunks, one of a single key, none aligned to a tile
    compare_chunks(1, 2, 380, 500, D, causal=causal, window=window, q_offset=q_offset,
                   chunks=[(0, 130), (130, 131), (131, 384), (384, 500)], seed=5, what="bwd_ex chunks")


@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_layouts_and_dtypes(layout, dtype):
    compare_chunks(2, 3, 190, 270, 128, dtype=dtype, layout=layout, q_offset=80, chunks=[(0, 141), (141, 270)],
                   seed=6, what="bwd_ex layout")


@pytest.mark.parametrize("causal,window,q_offset", [(False, -1, 0), (True, -1, 120), (True, 90, 30), (True, -1, -50)])
def test_fp32_chunks_offsets_windows(causal, window, q_offset):
    compare_chunks(1, 2, 300, 400, 64, dtype="fp32", causal=causal, window=window, q_offset=q_offset,
                   chunks=[(0, 100), (100, 101), (101, 333), (333, 400)], seed=13, what="bwd_ex fp32")


def test_negative_offset_rows_without_keys():
    # positions -50 .. 149: the first 50 queries see no key, so their dQ is exactly 0
    dev, _, lse = compare_chunks(1, 2, 200, 300, 64, q_offset=-50, seed=7, what="bwd_ex negative offset")
    assert bool(torch.isneginf(lse[:, :, :50]).all())


def test_rows_past_the_window_see_no_key():
    # 100 queries at positions 0 .. 99, 50 keys, window 10: queries from position 60 on see no key
    dev, _, lse = compare_chunks(1, 2, 100, 50, 128, window=10, seed=8, what="bwd_ex past window")
    assert bool(torch.isneginf(lse[:, :, 60:]).all())


@pytest.mark.parametrize("q_offset,window,chunks", [
    (1 << 30, -1, [(0, 300)]),                      # every key visible to every query
    (1 << 30, (1 << 30) - 100, [(0, 140), (140, 300)]),  # a window of 2^30 - 100 starting inside the keys
    (1 << 30, 500, [(0, 300)]),                     # the window reaches no key: all gradients 0
    (-(1 << 30), -1, [(0, 300)]),                   # every query before every key: all gradients 0
])
def test_offsets_at_the_limits(q_offset, window, chunks):
    # |q_offset| = 2^30 is the largest the entry point accepts; positions then need more than 31 bits
    # in the kernels' per-workgroup arithmetic before the clamps
    compare_chunks(1, 2, 70, 300, 128, window=window, q_offset=q_offset, chunks=chunks, seed=12,
                   what="bwd_ex limits")


def test_rows_outside_the_chunk_untouched_and_empty_chunk():
    B, H, Nq, Nk, D = 1, 2, 160, 400, 128
    q, k, v, do = make_case(B, H, Nq, Nk, D, "bf16", "BHSD", 9)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    o, lse = forward(dev, "BHSD", True, 0.088, -1, Nk - Nq)
    sentinel = torch.full_like(dev[1], 1024.0)
    dk, dv = sentinel.clone(), sentinel.clone()
    delta = torch.full((B, H, Nq), float("nan"), device="cuda")
    dq, dk, dv = fa.attention_bwd_ex(dev[0], dev[1], dev[2], o, lse, dev[3], causal=True, scale=0.088,
                                     q_offset=Nk - Nq, kv_start=100, kv_len=128, dk=dk, dv=dv, delta=delta)
    torch.cuda.synchronize()
    for t in (dk, dv):
        assert torch.equal(t[:, :, :100], sentinel[:, :, :100]) and torch.equal(t[:, :, 228:], sentinel[:, :, 228:])
        assert bool((t[:, :, 100:228] != 1024.0).any())
    ref = oracle.attention_bwd_ex(q, k, v, do, dtype="bf16", layout="BHSD", causal=True, scale=0.088,
                                  q_offset=Nk - Nq, kv_start=100, kv_len=128, nthreads=NTHREADS, mags=True)
    check("dQ[100:228]", f64(dq), ref[0], ref[3], "bwd_ex untouched", "bf16", Nk, D)
    check("dK[100:228]", f64(dk[:, :, 100:228]), ref[1][:, :, 100:228], ref[4][:, :, 100:228], "bwd_ex untouched",
          "bf16", Nk, D)
    check("dV[100:228]", f64(dv[:, :, 100:228]), ref[2][:, :, 100:228], ref[5][:, :, 100:228], "bwd_ex untouched",
          "bf16", Nk, D)
    # an empty chunk: dQ's part is 0, dK and dV untouched, D still written for every row
    dk2, dv2 = sentinel.clone(), sentinel.clone()
    delta.fill_(float("nan"))
    dq2, dk2, dv2 = fa.attention_bwd_ex(dev[0], dev[1], dev[2], o, lse, dev[3], causal=True, scale=0.088,
                                        q_offset=Nk - Nq, kv_start=400, kv_len=0, dk=dk2, dv=dv2, delta=delta)
    torch.cuda.synchronize()
    assert not bool(dq2.any())
    assert torch.equal(dk2, sentinel) and torch.equal(dv2, sentinel)
    ref_delta = (o.double() * dev[3].double()).sum(-1)
    assert torch.allclose(delta.double(), ref_delta, atol=1e-4, rtol=1e-5)


def test_plain_entry_point_is_the_whole_range():
    # fa_bwd(...) and fa_bwd_ex over all keys with no offset or window give the same bits
    q, k, v, do = make_case(2, 2, 300, 300, 128, "bf16", "BHSD", 10)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    for causal in (False, True):
        o, lse = fa.attention(dev[0], dev[1], dev[2], causal=causal)
        a = fa.attention_bwd(dev[0], dev[1], dev[2], o, lse, dev[3], causal=causal)
        b = fa.attention_bwd_ex(dev[0], dev[1], dev[2], o, lse, dev[3], causal=causal)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_prefill_behind_cache_sampled_heads():
    # 1024 new queries behind 3072 cached keys (positions 3072 .. 4095), two of eight heads in full
    B, H, Nq, Nk, D = 1, 8, 1024, 4096, 128
    q, k, v, do = make_case(B, H, Nq, Nk, D, "bf16", "BHSD", 11)
    _say("bwd_ex prefill: inputs ready")
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    scale = float(np.float32(1 / np.sqrt(D)))
    o, lse = forward(dev, "BHSD", True, scale, -1, Nk - Nq)
    dq, dk, dv = fa.attention_bwd_ex(dev[0], dev[1], dev[2], o, lse, dev[3], causal=True, scale=scale,
                                     q_offset=Nk - Nq)
    torch.cuda.synchronize()
    heads = [(0, 2), (0, 7)]
    ref = oracle.attention_bwd_ex(q, k, v, do, dtype="bf16", layout="BHSD", causal=True, scale=scale,
                                  q_offset=Nk - Nq, heads=heads, nthreads=NTHREADS, mags=True)
    for i, (name, g) in enumerate(zip(("dQ", "dK", "dV"), (dq, dk, dv))):
        check(name, np.stack([f64(g[b, h]) for (b, h) in heads]), ref[i], ref[i + 3], "bwd_ex prefill", "bf16", Nk, D)
