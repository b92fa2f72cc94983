"""Seeded random configurations of the generalised forward (fa_fwd_ex) and backward (fa_bwd_ex), each
checked against the oracle with the tolerances of the other parity tests.  Sizes, layouts, dtypes,
causal or not, windows, query offsets, key chunks and the sign of the scale are drawn from a fixed
generator, always inside what the entry points accept, and small enough for the oracle to finish in
seconds.  Each case prints its configuration before it runs."""
import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from tests.test_gpu_bwd_ex import compare_chunks
from tests.test_gpu_ex import NTHREADS, _check_ex, _make_qk, _say
from tests.test_gpu_parity import to_dev

pytestmark = pytest.mark.gpu
N_FWD, N_BWD = 100, 30


def _draw(kind, i):
    rng = np.random.default_rng([7, 11, kind, i])
    c = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), Nq=int(rng.integers(1, 400)),
             Nk=int(rng.integers(1, 600)), D=int(rng.choice([64, 128])),
             dtype=str(rng.choice(["bf16", "fp16", "fp32"])), layout=str(rng.choice(["BHSD", "BSND"])),
             causal=bool(rng.integers(0, 2)))
    c["window"] = int(rng.integers(0, 300)) if c["causal"] and rng.random() < 0.5 else -1
    c["q_offset"] = int(rng.integers(-100, c["Nk"] + 100)) if c["causal"] else 0
    return c, rng


@pytest.mark.parametrize("i", range(N_FWD))
def test_random_forward(i):
    c, rng = _draw(0, i)
    kv_start = int(rng.integers(0, c["Nk"])) if rng.random() < 0.5 else 0
    kv_len = int(rng.integers(0, c["Nk"] - kv_start + 1)) if rng.random() < 0.5 else c["Nk"] - kv_start
    scale = float(rng.choice([0.125, float(np.float32(1 / np.sqrt(c["D"]))), -0.1, 0.3]))
    what = "random forward %d: %s kv=[%d,+%d) scale=%g" % (i, c, kv_start, kv_len, scale)
    _say(what)
    q, k, v = _make_qk(c["B"], c["H"], c["Nq"], c["Nk"], c["D"], c["layout"], c["dtype"], seed=900 + i)
    qd, kd, vd = (to_dev(x, c["dtype"]) for x in (q, k, v))
    kw = dict(layout=c["layout"], causal=c["causal"], scale=scale, window=c["window"], q_offset=c["q_offset"],
              kv_start=kv_start, kv_len=kv_len)
    o, l = fa.attention_ex(qd, kd, vd, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_ex(q, k, v, dtype=c["dtype"], nthreads=NTHREADS, **kw)
    _check_ex(o, l, o_ref, l_ref, c["dtype"], what)


@pytest.mark.parametrize("i", range(N_BWD))
def test_random_backward(i):
    c, rng = _draw(1, i)
    n_cuts = int(rng.integers(0, 3))
    cuts = sorted(set(int(x) for x in rng.integers(1, c["Nk"], size=n_cuts))) if c["Nk"] > 1 else []
    bounds = [0] + cuts + [c["Nk"]]
    chunks = list(zip(bounds[:-1], bounds[1:]))
    compare_chunks(c["B"], c["H"], c["Nq"], c["Nk"], c["D"], dtype=c["dtype"], layout=c["layout"],
                   causal=c["causal"], window=c["window"], q_offset=c["q_offset"], chunks=chunks, seed=950 + i,
                   what="random backward %d" % i)


def _draw_varlen(kind, i):
    rng = np.random.default_rng([7, 13, kind, i])
    B = int(rng.integers(1, 7))
    lq = [int(x) for x in rng.integers(0, 301, size=B)]
    lk = list(lq) if rng.random() < 0.5 else [int(x) for x in rng.integers(0, 401, size=B)]
    lq[0], lk[0] = max(lq[0], 1), max(lk[0], 1)  # the entry points need at least one row of each
    return dict(lq=lq, lk=lk, H=int(rng.integers(1, 4)), D=int(rng.choice([64, 128])),
                dtype=str(rng.choice(["bf16", "fp16"])), causal=bool(rng.integers(0, 2)))


@pytest.mark.parametrize("i", range(20))
def test_random_varlen_forward(i):
    from tests.test_gpu_parity import check
    from tests.test_gpu_varlen import run
    c = _draw_varlen(0, i)
    (q, k, v, cq, ck, scale), o, lse = run(c["lq"], c["lk"], c["H"], c["D"], c["dtype"], c["causal"], 970 + i)
    o_ref, lse_ref = oracle.attention_varlen(q, k, v, cq, ck, dtype=c["dtype"], causal=c["causal"], scale=scale,
                                             nthreads=NTHREADS)
    o_g, l_g = o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(lse_ref)  # [H, total_q]: causal rows before every key of a longer query sequence
    assert np.array_equal(np.isneginf(l_g), empty)
    assert np.all(o_g.transpose(1, 0, 2)[empty] == 0)
    check(o_g.transpose(1, 0, 2)[~empty], l_g[~empty], o_ref.transpose(1, 0, 2)[~empty], lse_ref[~empty],
          c["dtype"], "random varlen forward %d: %s" % (i, c))


@pytest.mark.parametrize("i", range(10))
def test_random_varlen_backward(i):
    from tests.test_gpu_varlen_bwd import _check, run
    c = _draw_varlen(1, i)
    got, ref = run(c["lq"], c["lk"], c["H"], c["D"], c["dtype"], c["causal"], 990 + i)
    _check(got, ref, "random varlen backward %d: %s" % (i, c), c["dtype"])
