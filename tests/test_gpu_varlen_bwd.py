"""GPU parity of the packed variable-length backward (fa_bwd_varlen through the C ABI) against the oracle's
per-sequence composition (oracle.attention_bwd_varlen), with the backward's per-element bound of
tests/bwd_bound.py (each element within (2 u + c eps) M + 1e-6 of the oracle, M its term magnitude).  The
GPU side runs the library's packed forward first for O and lse."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs
from tests import bwd_bound
from tests.test_gpu_parity import NTHREADS, _say, to_dev

pytestmark = pytest.mark.gpu


def _check(got, ref, what, dtype="bf16", abs_term=bwd_bound.ATOL):
    """got: the GPU's (dQ, dK, dV); ref: the oracle's gradients and term magnitudes, or ``run``'s pair of
    those and the absolute term.  n: the row counts (an upper bound of every sequence's)."""
    if len(ref) == 2:
        ref, abs_term = ref
    d = got[0].shape[-1]
    n = max(got[0].shape[0], got[1].shape[0])
    bwd_bound.check_all([g.float().cpu().numpy().astype(np.float64) for g in got], ref, dtype, n, d, what, abs_term)


def run(lq, lk, H, D, dtype, causal, seed):
    q, k, v = inputs.make_varlen(lq, lk, H, D, dtype=dtype, seed=seed)
    do = inputs.make_grad_varlen(lq, H, D, dtype=dtype, seed=seed)
    cq, ck = inputs.cu_seqlens(lq), inputs.cu_seqlens(lk)
    scale = float(np.float32(1 / np.sqrt(D)))
    _say("varlen bwd: B=%d H=%d D=%d %s causal=%d lq=%s lk=%s" % (len(lq), H, D, dtype, causal, list(lq)[:8],
                                                                  list(lk)[:8]))
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    cqd, ckd = torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda()
    o, lse = fa.attention_varlen(dev[0], dev[1], dev[2], cqd, ckd, max(max(lq), 1), causal=causal, scale=scale)
    got = fa.attention_bwd_varlen(dev[0], dev[1], dev[2], o, lse, dev[3], cqd, ckd, max(max(lq), 1), max(max(lk), 1),
                                  causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_bwd_varlen(q, k, v, do, cq, ck, dtype=dtype, causal=causal, scale=scale, nthreads=NTHREADS,
                                      mags=True)
    # the absolute term of the longest sequence's sums (fp16 only)
    at = bwd_bound.atol(dtype, max(max(lq), max(lk), 1), scale, q, k, do)
    return got, (ref, at)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_self_attention_length_mix(dtype, causal, D):
    lens = [1, 300, 0, 128, 129, 77, 513, 64]
    got, ref = run(lens, lens, 3, D, dtype, causal, [D, causal])
    _check(got, ref, "varlen bwd self D=%d %s causal=%d" % (D, dtype, causal), dtype)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_with_cache_lengths(causal):
    # queries fewer than keys (a cache in front), more than keys (early rows see nothing), no keys, and
    # keys without queries (their dK, dV are 0)
    lq = [100, 257, 5, 40, 16, 0]
    lk = [900, 130, 5, 0, 300, 77]
    got, ref = run(lq, lk, 2, 128, "bf16", causal, 31)
    _check(got, ref, "varlen bwd cache causal=%d" % causal)
    ck = inputs.cu_seqlens(lk)
    assert not got[1][ck[5]:].any() and not got[2][ck[5]:].any()


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_bit_identical_to_batched(causal):
    B, N, H, D = 3, 333, 4, 128
    q, k, v = inputs.make(B, H, N, D, layout="BSND", dtype="bf16", seed=32)
    do = inputs.make_grad(B, H, N, D, layout="BSND", dtype="bf16", seed=32)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    o, lse = fa.attention(dev[0], dev[1], dev[2], layout="BSND", causal=causal)
    g_b = fa.attention_bwd(dev[0], dev[1], dev[2], o, lse, dev[3], layout="BSND", causal=causal)
    cu = torch.from_numpy(inputs.cu_seqlens([N] * B)).cuda()
    pk = [t.reshape(B * N, H, D) for t in (dev[0], dev[1], dev[2], o, dev[3])]
    lse_v = lse.permute(1, 0, 2).reshape(H, B * N).contiguous()
    g_v = fa.attention_bwd_varlen(pk[0], pk[1], pk[2], pk[3], lse_v, pk[4], cu, cu, N, N, causal=causal)
    torch.cuda.synchronize()
    for x, y in zip(g_v, g_b):
        assert torch.equal(x.reshape(B, N, H, D), y)


def test_bad_offsets_skip_only_their_sequence():
    # offsets [0, 50, 40]: sequence 1 decreases and is skipped (rows 50.. of dq, dk, dv and delta keep
    # their values); sequence 0 (rows [0, 50)) is valid and is checked against the oracle
    lens = [50, 70]
    H, D = 2, 64
    q, k, v = inputs.make_varlen(lens, lens, H, D, dtype="bf16", seed=33)
    do = inputs.make_grad_varlen(lens, H, D, dtype="bf16", seed=33)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    good = torch.from_numpy(inputs.cu_seqlens(lens)).cuda()
    o, lse = fa.attention_varlen(dev[0], dev[1], dev[2], good, good, 70, causal=True)
    bad = torch.tensor([0, 50, 40], dtype=torch.int32, device="cuda")
    out = tuple(torch.full_like(t, 5.0) for t in (dev[0], dev[1], dev[2]))
    delta = torch.full((H, 120), 5.0, device="cuda")
    fa.attention_bwd_varlen(dev[0], dev[1], dev[2], o, lse, dev[3], bad, bad, 70, 70, causal=True, delta=delta,
                            out=out)
    torch.cuda.synchronize()
    for t in out:
        assert bool((t[50:] == 5.0).all())
    assert bool((delta[:, 50:] == 5.0).all())
    ref = oracle.attention_bwd_varlen(q[:50], k[:50], v[:50], do[:50], [0, 50], [0, 50], dtype="bf16", causal=True,
                                      scale=float(np.float32(1 / np.sqrt(D))), nthreads=NTHREADS, mags=True)
    _check(tuple(t[:50] for t in out), ref, "varlen bwd bad offsets, sequence 0")


@pytest.mark.parametrize("causal", [False, True])
def test_a_thousand_short_sequences(causal):
    # many tiny sequences: the grid's head spreading and padding with 1000 x 2 (sequence, head) units
    lens = inputs.varlen_lengths(1000, 0, 20, seed=34)
    got, ref = run(lens, lens, 2, 64, "bf16", causal, 34)
    _check(got, ref, "varlen bwd 1000 sequences causal=%d" % causal)
