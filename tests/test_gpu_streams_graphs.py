"""The entry points launch only on the caller's stream and allocate nothing, so they run on a side stream
and inside a captured HIP graph.  Each captured graph is replayed several times with the program's own
eager work and synchronisations between the replays, and every replay must reproduce the eager result bit
for bit."""
import numpy as np
import pytest
import torch

import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs
from tests.test_gpu_parity import _say

pytestmark = pytest.mark.gpu


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to("cuda")


def _inputs(B, H, N, D, seed):
    q, k, v = (_dev(x) for x in inputs.make(B, H, N, D, layout="BHSD", dtype="bf16", seed=seed))
    do = _dev(inputs.make_grad(B, H, N, D, layout="BHSD", dtype="bf16", seed=seed))
    return q, k, v, do


def _fwd_bwd(q, k, v, do, bufs):
    o, lse, dq, dk, dv, delta = bufs
    fa.attention(q, k, v, causal=True, out=o, lse=lse)
    B, H, N, D = q.shape
    st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                   dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), B, H, N, D, fa.LAYOUT_BHSD, True,
                   float(np.float32(1 / np.sqrt(D))), fa.DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK


def _buffers(q):
    B, H, N, D = q.shape
    return (torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda"), torch.empty_like(q),
            torch.empty_like(q), torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda"))


def test_side_stream_matches_default_stream():
    q, k, v, do = _inputs(2, 4, 700, 128, 40)
    ref = _buffers(q)
    _fwd_bwd(q, k, v, do, ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = _buffers(q)
        _fwd_bwd(q, k, v, do, got)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


def test_graph_replays_match_eager():
    q, k, v, do = _inputs(2, 4, 700, 128, 41)
    eager = _buffers(q)
    _fwd_bwd(q, k, v, do, eager)
    torch.cuda.synchronize()
    bufs = _buffers(q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one warm call outside the capture
        _fwd_bwd(q, k, v, do, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _fwd_bwd(q, k, v, do, bufs)
    torch.cuda.synchronize()
    for replay in range(4):
        for t in bufs:  # the program's own eager work between replays
            t.fill_(float("nan") if t.dtype == torch.float32 else 3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv", "delta"), bufs, eager):
            assert torch.equal(a, b), "replay %d: %s differs from the eager result" % (replay, name)
        _say("graph replay %d matches the eager forward and backward" % replay)


def test_graph_of_split_kv_and_merge():
    # the chunked forward with its merge, captured: four fa_fwd_ex launches and one fa_merge
    B, H, N, D = 1, 4, 1000, 128
    q, k, v, _ = _inputs(B, H, N, D, 42)
    cuts = [0, 250, 251, 700, 1000]
    o_parts = torch.empty((len(cuts) - 1, B, H, N, D), dtype=torch.bfloat16, device="cuda")
    l_parts = torch.empty((len(cuts) - 1, B, H, N), dtype=torch.float32, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")

    def run():
        for s, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
            fa.attention_ex(q, k, v, causal=True, kv_start=a, kv_len=b - a, out=o_parts[s], lse=l_parts[s])
        fa.merge(o_parts, l_parts, out=o, lse=lse)

    run()
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for replay in range(3):
        o.fill_(5.0)
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "replay %d differs" % replay
