"""GPU parity of the backward pass (fa_bwd through the C ABI) against the oracle's fp64 gradients.

The GPU side runs the library's forward first (its O and lse are the backward's inputs), then fa_bwd;
the oracle computes dQ, dK, dV from Q, K, V and dO alone, by the chain rule, with each element's term
magnitude beside it.  Every element must lie within the per-element bound of tests/bwd_bound.py,
(2 u + c eps) M + 1e-6, derived there from the kernels' roundings (u the 16-bit unit roundoff, 0 for fp32
inputs; M the element's term magnitude).
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


def run(q, k, v, do, dtype, layout, causal, scale):
    dev = [to_dev(x, dtype) for x in (q, k, v, do)]
    o, lse = fa.attention(dev[0], dev[1], dev[2], layout=layout, causal=causal, scale=scale)
    dq, dk, dv = fa.attention_bwd(dev[0], dev[1], dev[2], o, lse, dev[3], layout=layout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (dq, dk, dv), (o, lse)


def check(got, ref, what, dtype, n, d, abs_term=bwd_bound.ATOL):
    bwd_bound.check_all(got, ref, dtype, n, d, what, abs_term)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def full_compare(B, H, N, D, dtype, layout, causal, scale, seed, what, qk_mult=1.0):
    q, k, v = inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=seed, qk_mult=qk_mult)
    do = inputs.make_grad(B, H, N, D, layout=layout, dtype=dtype, seed=seed)
    _say("%s: B=%d H=%d N=%d D=%d %s %s causal=%d" % (what, B, H, N, D, dtype, layout, causal))
    got, _ = run(q, k, v, do, dtype, layout, causal, scale)
    ref = oracle.attention_bwd(q, k, v, do, dtype=dtype, layout=layout, causal=causal, scale=scale, nthreads=NTHREADS,
                               mags=True)
    check([f64(t) for t in got], ref, what, dtype, N, D, bwd_bound.atol(dtype, N, scale, q, k, do))
    return got


@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_c2_shape_full(dtype, causal):
    w = inputs.WORKLOADS["c2"]
    full_compare(w.B, w.H, w.N, w.D, dtype, w.layout, causal, w.scale, w.seed, "bwd c2")


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 200, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sizes(N, D, causal):
    full_compare(2, 3, N, D, "bf16", "BHSD", causal, float(np.float32(1 / np.sqrt(D))), [N, D, causal], "bwd ragged")


@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
@pytest.mark.parametrize("dtype", ["fp16", "bf16", "fp32"])
def test_layouts_and_dtypes(layout, dtype):
    full_compare(2, 2, 333, 128, dtype, layout, True, 0.0883883461356163, [11, len(layout)], "bwd layout")


@pytest.mark.parametrize("N", [1, 31, 32, 33, 127, 128, 129, 300])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_ragged_sizes(N, D, causal):
    # the fp32 kernels tile by 32 keys / query rows: sizes around one and several tiles, and a ragged tail
    full_compare(2, 2, N, D, "fp32", "BHSD", causal, float(np.float32(1 / np.sqrt(D))), [N, D, causal, 32],
                 "bwd fp32 ragged")


def test_large_logits():
    full_compare(1, 4, 520, 128, "bf16", "BHSD", True, 0.0883883461356163, 12, "bwd qk x8", qk_mult=8.0)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.5])
@pytest.mark.parametrize("N", [190, 512])
def test_scale_values(scale, N):
    # N = 512: the paired backward kernels, on O and lse from the ping-pong forward
    full_compare(1, 2, N, 64, "bf16", "BHSD", True, scale, 13 + N, "bwd scale %g N=%d" % (scale, N))


def test_single_key_rows():
    # N = 1: P = 1, so dQ = dK = 0 up to the fp32 evaluation of P (exp2 of an argument with an error of
    # about 2^-24 |scale q.k|, so P = 1 - O(1e-7)) and dS = P (dP - D), the difference of two fp32
    # evaluations of dO . v, O(1e-6); and dV = dO (P = 1 - O(1e-7) times a stored dO rounds back to it)
    q, k, v = inputs.make(2, 3, 1, 64, layout="BHSD", dtype="bf16", seed=14)
    do = inputs.make_grad(2, 3, 1, 64, layout="BHSD", dtype="bf16", seed=14)
    (dq, dk, dv), _ = run(q, k, v, do, "bf16", "BHSD", True, 0.125)
    assert dq.abs().max().item() <= 1e-5 and dk.abs().max().item() <= 1e-5
    assert torch.equal(dv, to_dev(do, "bf16"))


def test_deterministic_bitwise():
    q, k, v = inputs.make(2, 4, 700, 128, layout="BHSD", dtype="bf16", seed=15)
    do = inputs.make_grad(2, 4, 700, 128, layout="BHSD", dtype="bf16", seed=15)
    a, _ = run(q, k, v, do, "bf16", "BHSD", True, 0.088)
    b, _ = run(q, k, v, do, "bf16", "BHSD", True, 0.088)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_delta_workspace_holds_rowsum():
    q, k, v = inputs.make(1, 2, 150, 64, layout="BHSD", dtype="bf16", seed=16)
    do = inputs.make_grad(1, 2, 150, 64, layout="BHSD", dtype="bf16", seed=16)
    dev = [to_dev(x, "bf16") for x in (q, k, v, do)]
    o, lse = fa.attention(dev[0], dev[1], dev[2], causal=True)
    delta = torch.full((1, 2, 150), float("nan"), device="cuda")
    fa.attention_bwd(dev[0], dev[1], dev[2], o, lse, dev[3], causal=True, delta=delta)
    torch.cuda.synchronize()
    ref = (o.double() * dev[3].double()).sum(-1)  # from the same stored O and dO
    assert torch.allclose(delta.double(), ref, atol=1e-4, rtol=1e-5)


def test_c3_full_size_sampled_heads():
    w = inputs.WORKLOADS["c3"]
    q, k, v = inputs.make_workload(w)
    do = inputs.make_grad(w.B, w.H, w.N, w.D, layout=w.layout, dtype="bf16", seed=w.seed)
    _say("bwd c3: inputs ready")
    (dq, dk, dv), _ = run(q, k, v, do, "bf16", w.layout, True, w.scale)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    # properties over every head, from fp32 sums of the outputs: sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    # hold exactly in exact arithmetic; each stored element carries relative rounding errors of a few 2^-9,
    # so the sums must vanish to within 2^-6 of the sums of magnitudes
    dof = to_dev(do, "bf16").float()
    sk = dk.float().sum(2).abs() / dk.float().abs().sum(2)
    sv = (dv.float().sum(2) - dof.sum(2)).abs() / (dv.float().abs().sum(2) + dof.abs().sum(2))
    _say("bwd c3: max relative |sum dK|=%.3e, |sum dV - sum dO|=%.3e" % (sk.max().item(), sv.max().item()))
    assert sk.max().item() <= 2 ** -6 and sv.max().item() <= 2 ** -6
    # two seeded heads in full against the oracle
    rng = np.random.default_rng([4242, 3, 7])
    heads = [divmod(int(x), w.H) for x in rng.choice(w.B * w.H, size=2, replace=False)]
    ref = oracle.attention_bwd(q, k, v, do, dtype="bf16", layout=w.layout, causal=True, scale=w.scale, heads=heads,
                               nthreads=NTHREADS, mags=True)
    got = [np.stack([f64(t[b, h]) for (b, h) in heads]) for t in (dq, dk, dv)]
    check(got, ref, "bwd c3 heads %s" % heads, "bf16", w.N, w.D)


def test_c5_full_size_rows_and_properties():
    # the 65536-token causal shape: every output finite, the two sum identities over every head, and the dQ
    # of sampled rows against the oracle -- a row's dQ depends only on its own query, its dO row and its
    # visible keys, so the generalised backward of that one row (at its position, over keys 0 .. i) is exact
    w = inputs.WORKLOADS["c5"]
    q, k, v = inputs.make_workload(w)
    do = inputs.make_grad(w.B, w.H, w.N, w.D, layout=w.layout, dtype="bf16", seed=w.seed)
    _say("bwd c5: inputs ready")
    (dq, dk, dv), _ = run(q, k, v, do, "bf16", w.layout, True, w.scale)
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    dof = to_dev(do, "bf16").float()
    sk = dk.float().sum(2).abs() / dk.float().abs().sum(2)
    sv = (dv.float().sum(2) - dof.sum(2)).abs() / (dv.float().abs().sum(2) + dof.abs().sum(2))
    _say("bwd c5: max relative |sum dK|=%.3e, |sum dV - sum dO|=%.3e" % (sk.max().item(), sv.max().item()))
    assert sk.max().item() <= 2 ** -6 and sv.max().item() <= 2 ** -6
    rows = inputs.sample_rows(w.B, w.H, w.N, 48, seed=[5, 7], heads_subset=2, rows_per_head=6)
    got, ref, mag = [], [], []
    for b, h, i in rows:
        b, h, i = int(b), int(h), int(i)
        r = oracle.attention_bwd_ex(q[b:b + 1, h:h + 1, i:i + 1], k[b:b + 1, h:h + 1, :i + 1], v[b:b + 1, h:h + 1, :i + 1],
                                    do[b:b + 1, h:h + 1, i:i + 1], dtype="bf16", layout=w.layout, causal=True,
                                    scale=w.scale, q_offset=i, nthreads=NTHREADS, mags=True)
        ref.append(r[0][0, 0, 0])
        mag.append(r[3][0, 0, 0])
        got.append(f64(dq[b, h, i]))
    bwd_bound.check("%d sampled dQ rows" % len(rows), np.stack(got), np.stack(ref), np.stack(mag), "bf16", w.N, w.D,
                    "bwd c5")


def test_host_pointer_rejected():
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 64, device="cuda")
    host = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(fa.FaError) as e:
        fa.attention_bwd(x, x.clone(), x.clone(), x.clone(), lse, host)
    assert e.value.status == fa.FA_ERR_NOT_DEVICE_MEMORY


@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_short_rows(causal):
    # B*H = 2048 (b, h) units of 17 rows: the workgroup -> unit mapping with a large, ragged grid
    full_compare(64, 32, 17, 64, "bf16", "BSND", causal, 0.125, [17, 64, causal], "bwd many heads")
