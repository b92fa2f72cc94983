"""The K/V tiles the forward kernels visit, against the closed form of the visibility rule.

The test-only library libfa_tilecount.so (the same sources built with FA_TILE_COUNT) records, for every
workgroup of a 16-bit forward launch, its head, its query tile(s), how many key tiles it streams and how many
of them each wave computes on.  The expected counts come from the visibility rule alone: query i (at
position q_offset + i) sees key j of the chunk iff j <= i + delta under causal (delta = q_offset - kv_start)
and j >= i + delta - window with a window (why-attention page, `triu(ones, diagonal=1)`; catlass page,
"Causal Mask的实现差异", skip every tile above the diagonal).  A unit of queries [a, b] sees the keys
[a + delta - window, b + delta] clipped to the chunk, so it streams ceil(len / BN) tiles from the first of
them; a wave computes on exactly the tiles that hold a key one of its real rows sees.  Records must also
cover every query row of every head exactly once.  For whole causal problems the per-head totals are also
held against the catlass page's count sum_t (floor(((t+1) bm - 1) / bn) + 1) with real rows only.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "transformer_attention_fwd_amd",
                   "libfa_tilecount.so")
REC = 24
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError("libfa_tilecount.so is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        P, I64, I, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.fa_fwd.argtypes = [P] * 5 + [I64] * 4 + [I, I, F, I, P]
        L.fa_fwd_ex.argtypes = [P] * 5 + [I64] * 5 + [I, I] + [I64] * 4 + [F, I, P]
        L.fa_fwd_varlen.argtypes = [P] * 7 + [I64] * 6 + [I, F, I, P]
        L.fa_test_set_tile_record.argtypes = [P, ctypes.c_longlong]
        for f in (L.fa_fwd, L.fa_fwd_ex, L.fa_fwd_varlen, L.fa_test_set_tile_record):
            f.restype = I
        _lib = L
    return _lib


def run_recorded(launch, max_blocks=1 << 16):
    """Run launch() with tile recording on; return the filled records (rows of REC ints)."""
    rec = torch.full((max_blocks, REC), -1, dtype=torch.int32, device="cuda")
    assert lib().fa_test_set_tile_record(rec.data_ptr(), max_blocks) == 0
    try:
        assert launch() == 0
        torch.cuda.synchronize()
    finally:
        assert lib().fa_test_set_tile_record(None, 0) == 0
    r = rec.cpu().numpy()
    return r[r[:, 0] >= 0]


def expected(nq, nkv, delta, window, causal, a, bm, bn, qw, nw):
    """Tiles streamed by the unit of queries [a, a + bm) and tiles each wave computes on, from the rule."""
    last = min(a + bm, nq) - 1
    lo = min(nkv, max(0, a + delta - window)) if window >= 0 else 0
    hi = max(-1, min(nkv - 1, last + delta)) if causal else nkv - 1
    n = (hi - lo) // bn + 1 if hi >= lo else 0
    waves = []
    for w in range(nw):
        q0 = a + w * qw
        if q0 > last:
            waves.append(0)
            continue
        q1 = min(q0 + qw - 1, last)
        wlo = max(0, q0 + delta - window) if window >= 0 else 0
        whi = min(nkv - 1, q1 + delta) if causal else nkv - 1
        cnt = 0
        for t in range(n):
            k0, k1 = lo + t * bn, min(lo + t * bn + bn, nkv) - 1
            cnt += int(max(k0, wlo) <= min(k1, whi))
        waves.append(cnt)
    return n, waves


def check_records(recs, seqs, causal, window):
    """seqs: {head slot: (nq, nkv, delta)}.  Every record against the rule, every row covered once."""
    assert len(recs) > 0
    covered = {bh: np.zeros(s[0], dtype=np.int64) for bh, s in seqs.items()}
    totals = {bh: [0, 0] for bh in seqs}
    for r in recs:
        bh, bm, bn, qw = int(r[0]), int(r[1]), int(r[2]), int(r[3])
        nw = int(r[16])
        nq, nkv, delta = seqs[bh]
        units = [(int(r[4]), int(r[5]))] + ([(int(r[6]), int(r[7]))] if r[6] >= 0 else [])
        got_waves = [int(x) for x in r[8:8 + nw]]
        exp_waves = [0] * nw
        # a launch over a row range (the library splits some calls) ends its last unit at the range's end
        nq_rec = min(nq, int(r[18]))
        for a, n in units:
            en, ew = expected(nq_rec, nkv, delta, window, causal, a, bm, bn, qw, nw)
            assert n == en, "head slot %d unit %d: streams %d tiles, the rule gives %d" % (bh, a, n, en)
            exp_waves = [x + y for x, y in zip(exp_waves, ew)]
            covered[bh][a:min(a + bm, nq_rec)] += 1
            totals[bh][0] += n
        if int(r[17]) == 1:  # the ping-pong kernel: every wave computes on every streamed tile
            assert got_waves == [sum(n for _, n in units)] * nw
            if causal:  # a wave's tiles wholly above its rows run with P = 0 (only on the diagonal)
                assert all(e <= g for e, g in zip(exp_waves, got_waves)), (bh, exp_waves, got_waves)
            else:
                assert exp_waves == got_waves, "ping-pong workgroup of head slot %d: idle tiles %s" % (bh, exp_waves)
        else:
            assert got_waves == exp_waves, "head slot %d units %s: waves %s, the rule gives %s" % (
                bh, units, got_waves, exp_waves)
        totals[bh][1] += sum(got_waves)
    for bh, c in covered.items():
        assert np.all(c == 1), "head slot %d: rows covered %s times" % (bh, sorted(set(c.tolist())))
    return totals


def tensors(B, H, nq, nkv, D=128, layout="BHSD"):
    g = torch.Generator(device="cuda").manual_seed(5)
    shp = (lambda n: (B, H, n, D)) if layout == "BHSD" else (lambda n: (B, n, H, D))
    q = torch.randn(shp(nq), generator=g, device="cuda").to(torch.bfloat16)
    k = torch.randn(shp(nkv), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn(shp(nkv), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, nq), dtype=torch.float32, device="cuda")
    return q, k, v, o, lse


def catlass_count(n, bm, bn):
    """Tiles visited per head for a whole causal problem of n tokens (real rows only)."""
    return sum((min((t + 1) * bm, n) - 1) // bn + 1 for t in range((n + bm - 1) // bm))


# whole causal problems: ping-pong pairs of 256-query tiles (4096, 512), 8-wave pairs (384, 1000), 4-wave
# pairs (768), single tiles (300, 640)
@pytest.mark.parametrize("n,bm,pingpong", [(4096, 256, True), (512, 256, True), (384, 256, False), (768, 128, False),
                                           (300, 128, False), (1000, 256, False), (640, 128, False)])
def test_whole_causal(n, bm, pingpong):
    B, H, D = 2, 3, 128
    q, k, v, o, lse = tensors(B, H, n, n, D)
    s = torch.cuda.current_stream().cuda_stream
    recs = run_recorded(lambda: lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                            B, H, n, D, 0, 1, 0.088, 2, s))
    assert set(recs[:, 1].tolist()) == {bm}
    assert set(recs[:, 17].tolist()) == {1 if pingpong else 0}
    totals = check_records(recs, {bh: (n, n, 0) for bh in range(B * H)}, True, -1)
    for bh, (streamed, _) in totals.items():
        assert streamed == catlass_count(n, bm, 64), (bh, streamed, catlass_count(n, bm, 64))


@pytest.mark.parametrize("case", [
    dict(nq=1000, nkv=1000, q_offset=0, kv_start=0, kv_len=1000, window=256),
    dict(nq=1000, nkv=1000, q_offset=0, kv_start=0, kv_len=1000, window=300),
    dict(nq=1000, nkv=1000, q_offset=0, kv_start=0, kv_len=1000, window=0),
    dict(nq=1000, nkv=1000, q_offset=0, kv_start=200, kv_len=500, window=-1),    # a key chunk
    dict(nq=1000, nkv=1000, q_offset=0, kv_start=200, kv_len=500, window=150),
    dict(nq=300, nkv=1000, q_offset=700, kv_start=0, kv_len=1000, window=-1),    # prefill behind a cache
    dict(nq=300, nkv=1000, q_offset=-100, kv_start=0, kv_len=1000, window=-1),   # queries end before the keys
    dict(nq=90, nkv=700, q_offset=400, kv_start=128, kv_len=300, window=150),
    # chunks split into row ranges (rows before the chunk's first key, its square as ping-pong pairs, the
    # rows after it as ping-pong non-causal units): one launch per range, recorded as one call
    dict(nq=2048, nkv=2048, q_offset=0, kv_start=1024, kv_len=512, window=-1),
    dict(nq=1068, nkv=1068, q_offset=0, kv_start=300, kv_len=512, window=-1),
    dict(nq=768, nkv=768, q_offset=0, kv_start=0, kv_len=512, window=-1),
])
def test_offsets_chunks_windows(case):
    c = case
    B, H, D = 1, 2, 128
    q, k, v, o, lse = tensors(B, H, c["nq"], c["nkv"], D)
    s = torch.cuda.current_stream().cuda_stream
    recs = run_recorded(lambda: lib().fa_fwd_ex(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, c["nq"], c["nkv"], D, 0, 1,
        c["window"], c["q_offset"], c["kv_start"], c["kv_len"], 0.088, 2, s))
    delta = c["q_offset"] - c["kv_start"]
    check_records(recs, {bh: (c["nq"], c["kv_len"], delta) for bh in range(B * H)}, True, c["window"])
    rest = c["nq"] + delta - c["kv_len"]  # rows after the square
    split = c["window"] < 0 and delta <= 0 and c["kv_len"] % 512 == 0 and rest >= 0 and rest % 256 == 0
    assert (1 in set(recs[:, 17].tolist())) == split


@pytest.mark.parametrize("n,pingpong", [(512, True), (300, False)])
def test_noncausal(n, pingpong):
    B, H, D = 1, 4, 128
    q, k, v, o, lse = tensors(B, H, n, n, D)
    s = torch.cuda.current_stream().cuda_stream
    recs = run_recorded(lambda: lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                            B, H, n, D, 0, 0, 0.088, 2, s))
    assert set(recs[:, 17].tolist()) == {1 if pingpong else 0}
    check_records(recs, {bh: (n, n, 0) for bh in range(B * H)}, False, -1)


def test_varlen():
    lens = [0, 5, 300, 1000, 64, 257]
    H, D = 3, 128
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device="cuda")
    total = int(sum(lens))
    g = torch.Generator(device="cuda").manual_seed(6)
    q, k, v = (torch.randn((total, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    recs = run_recorded(lambda: lib().fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                   lse.data_ptr(), cu.data_ptr(), cu.data_ptr(), len(lens), H, total,
                                                   total, max(lens), D, 1, 0.088, 2, s))
    seqs = {b * H + h: (lens[b], lens[b], 0) for b in range(len(lens)) for h in range(H) if lens[b] > 0}
    recs = recs[np.isin(recs[:, 0], list(seqs))]
    check_records(recs, seqs, True, -1)
