"""GPU parity of fa_fwd_ex (key chunks, query offsets, sliding windows, Nq != Nk) and fa_merge against the
oracle, on seeded inputs, through the C ABI (the thin torch wrappers attention_ex and merge)."""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs
from tests.test_gpu_parity import check, to_dev

pytestmark = pytest.mark.gpu
NTHREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _make_qk(B, H, Nq, Nk, D, layout, dtype, seed):
    """Q with Nq rows and K, V with Nk rows, drawn by the shared seeded generator."""
    q, _, _ = inputs.make(B, H, Nq, D, layout=layout, dtype=dtype, seed=seed)
    _, k, v = inputs.make(B, H, Nk, D, layout=layout, dtype=dtype, seed=seed + 1000)
    return q, k, v


def _check_ex(o, lse, o_ref, lse_ref, dtype, what):
    """check() plus exact handling of rows without visible keys (O = 0 and lse = -inf on both sides)."""
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), empty), what + ": rows without visible keys differ"
    if empty.any():
        if o.shape[:3] == lse.shape:  # BHSD
            assert np.all(o[empty] == 0.0), what + ": O of rows without visible keys is not 0"
        _say("%s: %d rows without visible keys" % (what, int(empty.sum())))
    lse_c = np.where(empty, 0.0, lse)
    ref_c = np.where(empty, 0.0, lse_ref)
    check(o, lse_c, o_ref, ref_c, dtype, what)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
def test_split_kv_chunks_and_merge(dtype, causal, layout):
    B, H, N, D = 2, 3, 300, 128 if dtype != "fp32" else 64
    cuts = (0, 70, 71, 200, 300)
    q, k, v = inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=200)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o_parts, l_parts = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        o, l = fa.attention_ex(qd, kd, vd, layout=layout, causal=causal, scale=0.1, kv_start=a, kv_len=b - a)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=0.1,
                                           kv_start=a, kv_len=b - a, nthreads=NTHREADS)
        _check_ex(o, l, o_ref, l_ref, dtype, "chunk [%d,%d) %s %s c=%d" % (a, b, dtype, layout, causal))
        o_parts.append(o)
        l_parts.append(l)
    om, lm = fa.merge(torch.stack(o_parts), torch.stack(l_parts), layout=layout)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=0.1, nthreads=NTHREADS)
    _check_ex(om, lm, o_ref, l_ref, dtype, "merged %d chunks %s %s c=%d" % (len(cuts) - 1, dtype, layout, causal))


# Key chunks that the library splits into row ranges (rows before the chunk's first key: no key; the
# square of the chunk: a whole causal problem; later rows: every key of the chunk): the chunk length a
# multiple of 512 and the rows after the square a multiple of 256.  N = 2048 in chunks of 512 is the
# 4-chunk split of a 4096-token sequence at half size; the others start the square at an odd row, leave
# no rows after it, or none before it.
@pytest.mark.parametrize("case", [
    dict(nq=2048, nk=2048, q_offset=0, chunks=((0, 512), (512, 512), (1024, 512), (1536, 512)), D=128,
         dtype="bf16", layout="BHSD", scale=0.09),
    dict(nq=2048, nk=2048, q_offset=0, chunks=((0, 1024), (1024, 1024)), D=64, dtype="fp16", layout="BSND",
         scale=0.125),
    dict(nq=1068, nk=1068, q_offset=0, chunks=((300, 512),), D=128, dtype="bf16", layout="BSND", scale=-0.09),
    dict(nq=1024, nk=2048, q_offset=512, chunks=((1024, 512),), D=64, dtype="bf16", layout="BHSD", scale=0.125),
    dict(nq=768, nk=512, q_offset=0, chunks=((0, 512),), D=128, dtype="fp16", layout="BHSD", scale=0.09),
])
def test_chunk_split_row_ranges(case):
    c = case
    B, H, D, dtype, layout = 1, 2, c["D"], c["dtype"], c["layout"]
    q, k, v = _make_qk(B, H, c["nq"], c["nk"], D, layout, dtype, seed=700 + c["nq"])
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o_parts, l_parts = [], []
    for kv_start, kv_len in c["chunks"]:
        kw = dict(q_offset=c["q_offset"], kv_start=kv_start, kv_len=kv_len)
        what = "split chunk %s nq=%d D=%d %s %s" % (kw, c["nq"], D, dtype, layout)
        _say(what)
        o, l = fa.attention_ex(qd, kd, vd, layout=layout, causal=True, scale=c["scale"], **kw)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout=layout, causal=True, scale=c["scale"],
                                           nthreads=NTHREADS, **kw)
        _check_ex(o, l, o_ref, l_ref, dtype, what)
        # each row range holds what one kernel computes for it alone: the square as a whole causal problem
        # on the chunk's keys, the later rows as a non-causal problem on them
        i0 = kv_start - c["q_offset"]
        rows = (lambda t, a, b: t[:, :, a:b]) if layout == "BHSD" else (lambda t, a, b: t[:, a:b])
        kc, vc = rows(kd, kv_start, kv_start + kv_len).contiguous(), rows(vd, kv_start, kv_start + kv_len).contiguous()
        o_sq, l_sq = fa.attention(rows(qd, i0, i0 + kv_len).contiguous(), kc, vc, layout=layout, causal=True,
                                  scale=c["scale"])
        torch.cuda.synchronize()
        assert torch.equal(rows(o, i0, i0 + kv_len), o_sq) and torch.equal(l[:, :, i0:i0 + kv_len], l_sq), what
        if i0 + kv_len < c["nq"]:
            o_r, l_r = fa.attention_ex(rows(qd, i0 + kv_len, c["nq"]).contiguous(), kc, vc, layout=layout,
                                       causal=False, scale=c["scale"])
            torch.cuda.synchronize()
            assert torch.equal(rows(o, i0 + kv_len, c["nq"]), o_r), what
            assert torch.equal(l[:, :, i0 + kv_len:], l_r), what
        o_parts.append(o)
        l_parts.append(l)
    if len(c["chunks"]) > 1:
        om, lm = fa.merge(torch.stack(o_parts), torch.stack(l_parts), layout=layout)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout=layout, causal=True, scale=c["scale"],
                                           q_offset=c["q_offset"], nthreads=NTHREADS)
        _check_ex(om, lm, o_ref, l_ref, dtype, "merged split nq=%d %s %s" % (c["nq"], dtype, layout))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("nq,nk", [(1, 4097), (100, 1000), (130, 130), (7, 300)])
def test_bottom_right_causal(dtype, nq, nk):
    D = 128
    layout = "BHSD" if nq % 2 else "BSND"
    q, k, v = _make_qk(1, 4, nq, nk, D, layout, dtype, seed=300 + nq)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o, l = fa.attention_ex(qd, kd, vd, layout=layout, causal=True, scale=1 / math.sqrt(D), q_offset=nk - nq)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout=layout, causal=True,
                                       scale=float(np.float32(1 / math.sqrt(D))), q_offset=nk - nq, nthreads=NTHREADS)
    _check_ex(o, l, o_ref, l_ref, dtype, "bottom-right causal Nq=%d Nk=%d %s %s" % (nq, nk, dtype, layout))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("window", [0, 1, 63, 64, 200])
@pytest.mark.parametrize("D", [64, 128])
def test_sliding_window(dtype, window, D):
    N = 500
    layout = "BHSD" if window % 2 == 0 else "BSND"
    q, k, v = inputs.make(1, 3, N, D, layout=layout, dtype=dtype, seed=400 + window)
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o, l = fa.attention_ex(qd, kd, vd, layout=layout, causal=True, scale=0.125, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout=layout, causal=True, scale=0.125, window=window,
                                       nthreads=NTHREADS)
    _check_ex(o, l, o_ref, l_ref, dtype, "window %d D=%d %s %s" % (window, D, dtype, layout))



@pytest.mark.parametrize("dtype,target", [("fp16", 25.0), ("bf16", 110.0)])
@pytest.mark.parametrize("window", [50, 300])
def test_window_negative_logits(dtype, target, window):
    """Windows where a wave's first tile holds none of some rows' keys, with every logit far below 0
    (Q anti-aligned with K: scale * q.k near -target).  The row's reference maximum must follow its visible
    keys: with a placeholder of 0 for the empty start, exp2(logit) underflows (fp16 below 2^-24, fp32
    below 2^-149) and O = 0 (fp16) or lse = -inf (bf16) came out instead of the softmax."""
    B, H, N, D = 1, 2, 600, 128
    scale = float(np.float32(1 / math.sqrt(D)))
    a = math.sqrt(target / (scale * D))
    zq, zk, v32 = inputs.draw_f32(B, H, N, D, seed=(450, window))
    q = inputs.to_layout(inputs.cast_bits((-a + 0.25 * zq).astype(np.float32), dtype), "BHSD")
    k = inputs.to_layout(inputs.cast_bits((a + 0.25 * zk).astype(np.float32), dtype), "BHSD")
    v = inputs.to_layout(inputs.cast_bits(v32, dtype), "BHSD")
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    o, l = fa.attention_ex(qd, kd, vd, layout="BHSD", causal=True, scale=scale, window=window)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout="BHSD", causal=True, scale=scale, window=window,
                                       nthreads=NTHREADS)
    assert float(np.max(l_ref)) < -0.5 * target, "the logits are not as negative as intended"
    _check_ex(o, l, o_ref, l_ref, dtype, "window %d, logits near -%g, %s" % (window, target, dtype))

# Windows at several sizes: ragged last query tiles (1000 rows), windows that are and are not a
# multiple of the 64-key tile, both layouts and D, a query chunk at q_offset 512 against 1024 keys,
# and the benchmark's window of 1024 over 4096 tokens (two heads).
@pytest.mark.parametrize("case", [
    dict(B=1, H=3, nq=1000, nk=1000, q_offset=0, window=256, D=128, dtype="bf16", layout="BHSD"),
    dict(B=2, H=2, nq=1000, nk=1000, q_offset=0, window=256, D=64, dtype="fp16", layout="BSND"),
    dict(B=1, H=3, nq=1000, nk=1000, q_offset=0, window=300, D=128, dtype="bf16", layout="BHSD"),
    dict(B=1, H=2, nq=4096, nk=4096, q_offset=0, window=1024, D=128, dtype="bf16", layout="BHSD"),
    dict(B=1, H=4, nq=512, nk=1024, q_offset=512, window=256, D=128, dtype="bf16", layout="BSND"),
    dict(B=1, H=4, nq=512, nk=1024, q_offset=512, window=300, D=128, dtype="fp16", layout="BHSD"),
])
def test_window_sizes(case):
    c = case
    _say("window sizes: %s" % c)
    q, k, v = _make_qk(c["B"], c["H"], c["nq"], c["nk"], c["D"], c["layout"], c["dtype"], seed=c["window"] + c["nq"])
    qd, kd, vd = (to_dev(x, c["dtype"]) for x in (q, k, v))
    scale = float(np.float32(1 / math.sqrt(c["D"])))
    o, l = fa.attention_ex(qd, kd, vd, layout=c["layout"], causal=True, scale=scale, window=c["window"],
                           q_offset=c["q_offset"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=c["dtype"], layout=c["layout"], causal=True, scale=scale,
                                       window=c["window"], q_offset=c["q_offset"], nthreads=NTHREADS)
    _check_ex(o, l, o_ref, l_ref, c["dtype"], "window sizes %s" % c)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", [
    dict(nq=90, nk=700, q_offset=400, kv_start=128, kv_len=300, window=150),
    dict(nq=257, nk=257, q_offset=0, kv_start=200, kv_len=57, window=-1),
    dict(nq=64, nk=512, q_offset=-40, kv_start=0, kv_len=512, window=-1),
    dict(nq=33, nk=200, q_offset=150, kv_start=0, kv_len=0, window=-1),
    # offsets at the limits the entry point accepts (+-2^30): every key visible, a window of 2^30 - 100
    # that starts inside the chunk, a window that reaches no key, and queries before every key
    dict(nq=70, nk=300, q_offset=1 << 30, kv_start=0, kv_len=300, window=-1),
    dict(nq=70, nk=300, q_offset=1 << 30, kv_start=40, kv_len=200, window=(1 << 30) - 100),
    dict(nq=70, nk=300, q_offset=1 << 30, kv_start=0, kv_len=300, window=500),
    dict(nq=70, nk=300, q_offset=-(1 << 30), kv_start=0, kv_len=300, window=-1),
])
def test_offsets_chunks_windows_combined(dtype, case):
    D = 64
    q, k, v = _make_qk(2, 2, case["nq"], case["nk"], D, "BHSD", dtype, seed=500 + case["nq"])
    qd, kd, vd = (to_dev(x, dtype) for x in (q, k, v))
    kw = dict(q_offset=case["q_offset"], kv_start=case["kv_start"], kv_len=case["kv_len"], window=case["window"])
    o, l = fa.attention_ex(qd, kd, vd, layout="BHSD", causal=True, scale=0.2, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=dtype, layout="BHSD", causal=True, scale=0.2, nthreads=NTHREADS,
                                       **kw)
    _check_ex(o, l, o_ref, l_ref, dtype, "combined %s %s" % (case, dtype))


def test_plain_call_equals_generalised_defaults():
    q, k, v = inputs.make(2, 2, 333, 128, layout="BSND", dtype="bf16", seed=600)
    qd, kd, vd = (to_dev(x, "bf16") for x in (q, k, v))
    o1, l1 = fa.attention(qd, kd, vd, layout="BSND", causal=True, scale=0.1)
    o2, l2 = fa.attention_ex(qd, kd, vd, layout="BSND", causal=True, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
def test_merge_kernel_against_fp64_merge(dtype, layout):
    """fa_merge on given partials (some rows empty in some parts, some in all) against the oracle's fp64 merge
    of the same stored values."""
    S, B, H, N, D = 4, 2, 3, 77, 64
    rng = np.random.default_rng(700)
    parts = [inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=710 + s)[0] for s in range(S)]
    lse = rng.standard_normal((S, B, H, N)).astype(np.float32) * 5.0
    lse[1, :, :, :10] = -np.inf
    lse[:, 0, 0, 20:23] = -np.inf  # rows empty in every part
    o_parts = np.stack(parts)
    for s in range(S):  # a part without visible keys has O = 0
        if layout == "BHSD":
            o_parts[s][np.isneginf(lse[s])] = 0
        else:
            o_parts[s].transpose(0, 2, 1, 3)[np.isneginf(lse[s])] = 0
    od = to_dev(o_parts, dtype)
    ld = torch.from_numpy(lse).cuda()
    om, lm = fa.merge(od, ld, layout=layout)
    torch.cuda.synchronize()
    wid = {"fp32": np.float32, "fp16": np.float16}
    if dtype == "bf16":
        vals = (o_parts.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        vals = o_parts.view(wid[dtype]).astype(np.float64)
    if layout == "BSND":
        vals = vals.transpose(0, 1, 3, 2, 4)
    o_ref, l_ref = oracle.merge(list(vals), list(lse.astype(np.float64)))
    if layout == "BSND":
        o_ref = o_ref.transpose(0, 2, 1, 3)
    _check_ex(om, lm, o_ref, l_ref, dtype, "merge kernel %s %s" % (dtype, layout))
