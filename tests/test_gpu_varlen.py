"""GPU parity of the packed variable-length forward (fa_fwd_varlen through the C ABI) against the
oracle's per-sequence composition, with the forward's tolerances (test_gpu_parity.check)."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs
from tests.test_gpu_parity import NTHREADS, _say, check, to_dev

pytestmark = pytest.mark.gpu


def run(lq, lk, H, D, dtype, causal, seed, max_q=None, scale=None):
    q, k, v = inputs.make_varlen(lq, lk, H, D, dtype=dtype, seed=seed)
    cq, ck = inputs.cu_seqlens(lq), inputs.cu_seqlens(lk)
    scale = float(np.float32(1 / np.sqrt(D))) if scale is None else scale
    _say("varlen: B=%d H=%d D=%d %s causal=%d lq=%s lk=%s" % (len(lq), H, D, dtype, causal, list(lq)[:8], list(lk)[:8]))
    dq, dk, dv = (to_dev(x, dtype) for x in (q, k, v))
    o, lse = fa.attention_varlen(dq, dk, dv, torch.from_numpy(cq).cuda(), torch.from_numpy(ck).cuda(),
                                 max(lq) if max_q is None else max_q, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, cq, ck, scale), o, lse


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_self_attention_length_mix(dtype, causal, D):
    lens = [1, 300, 0, 128, 129, 77, 513, 64]
    (q, k, v, cq, ck, scale), o, lse = run(lens, lens, 3, D, dtype, causal, [D, causal])
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cq, ck, dtype=dtype, causal=causal, scale=scale, nthreads=NTHREADS)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, dtype,
          "varlen self D=%d" % D)


@pytest.mark.parametrize("causal", [False, True])
def test_prefill_with_cache_lengths(causal):
    # queries fewer than keys (a cache in front), more than keys (early rows see nothing), and no keys
    lq = [100, 257, 5, 40, 16]
    lk = [900, 130, 5, 0, 300]
    (q, k, v, cq, ck, scale), o, lse = run(lq, lk, 2, 128, "bf16", causal, 21)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cq, ck, dtype="bf16", causal=causal, scale=scale,
                                             nthreads=NTHREADS)
    o_g, l_g = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l_g), empty)
    assert np.all(o_g.transpose(1, 0, 2)[empty] == 0)
    check(o_g.transpose(1, 0, 2)[~empty], l_g[~empty], o_ref.transpose(1, 0, 2)[~empty], lse_ref[~empty], "bf16",
          "varlen cache causal=%d" % causal)


@pytest.mark.parametrize("causal", [False, True])
def test_equal_lengths_bit_identical_to_batched(causal):
    B, N, H, D = 3, 333, 4, 128
    q, k, v = inputs.make(B, H, N, D, layout="BSND", dtype="bf16", seed=22)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    o_b, lse_b = fa.attention(dq, dk, dv, layout="BSND", causal=causal)
    cu = torch.from_numpy(inputs.cu_seqlens([N] * B)).cuda()
    o_v, lse_v = fa.attention_varlen(dq.reshape(B * N, H, D), dk.reshape(B * N, H, D), dv.reshape(B * N, H, D),
                                     cu, cu, N, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o_v.reshape(B, N, H, D), o_b)
    assert torch.equal(lse_v.reshape(H, B, N).permute(1, 0, 2), lse_b)


@pytest.mark.parametrize("bad", [[0, 50, 40, 40], [0, 50, 110, 999]])
def test_bad_offsets_skip_only_their_sequence(bad):
    # [0, 50, 40, 40]: sequence 1 decreases (skipped), sequence 2 is empty; rows 50.. stay untouched
    # [0, 50, 110, 999]: sequence 2 ends past total_q = 180 (skipped); rows 110.. stay untouched
    lens = [50, 60, 70]
    q, k, v = inputs.make_varlen(lens, lens, 2, 64, dtype="bf16", seed=23)
    cq = inputs.cu_seqlens(lens)
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    o = torch.full_like(dq, 7.0)
    lse = torch.full((2, 180), 7.0, device="cuda")
    cu = torch.tensor(bad, dtype=torch.int32, device="cuda")
    fa.attention_varlen(dq, dk, dv, cu, cu, 70, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cq, cq, dtype="bf16", causal=True, scale=0.125)
    valid_end = 50 if bad[2] < bad[1] else 110
    o_g, l_g = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    check(o_g[:valid_end], l_g[:, :valid_end], o_ref[:valid_end], lse_ref[:, :valid_end], "bf16",
          "varlen bad offsets %s, valid sequences" % bad)
    assert np.all(o_g[valid_end:] == 7.0) and np.all(l_g[:, valid_end:] == 7.0)


def test_rows_beyond_max_seqlen_untouched():
    lens = [300, 100]
    q, k, v = inputs.make_varlen(lens, lens, 2, 128, dtype="bf16", seed=24)
    cu = torch.from_numpy(inputs.cu_seqlens(lens)).cuda()
    dq, dk, dv = (to_dev(x, "bf16") for x in (q, k, v))
    o = torch.full_like(dq, 7.0)
    lse = torch.full((2, 400), 7.0, device="cuda")
    fa.attention_varlen(dq, dk, dv, cu, cu, 128, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o[128:300] == 7.0).all()) and bool((lse[:, 128:300] == 7.0).all())
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, inputs.cu_seqlens(lens), inputs.cu_seqlens(lens), dtype="bf16",
                                             causal=True, scale=float(np.float32(1 / np.sqrt(128))))
    keep = np.r_[0:128, 300:400]
    check(o.float().cpu().numpy().astype(np.float64)[keep], lse.cpu().numpy().astype(np.float64)[:, keep],
          o_ref[keep], lse_ref[:, keep], "bf16", "varlen max_seqlen cut")


@pytest.mark.parametrize("causal", [False, True])
def test_a_thousand_short_sequences(causal):
    # many tiny sequences (lengths 0..20): the grid's head spreading and padding with 1000 x 2 units
    lens = inputs.varlen_lengths(1000, 0, 20, seed=24)
    (q, k, v, cq, ck, scale), o, lse = run(lens, lens, 2, 64, "bf16", causal, 24)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cq, ck, dtype="bf16", causal=causal, scale=scale, nthreads=NTHREADS)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "bf16",
          "varlen 1000 sequences causal=%d" % causal)
