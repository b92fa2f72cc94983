"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on identical seeded inputs.

Tolerances (fixed before any kernel ran):
  * fp16 / bf16 inputs: max |dO| <= 1e-2, except that a bf16 element may differ by up to one bf16 ulp
    of the oracle value when that ulp exceeds 1e-2 (|O| >= 2: a correctly rounded bf16 output can sit
    half an ulp, up to 0.0156, from the exact value); the number of such elements is reported.
    max |dlse| <= 1e-3.
  * fp32 inputs: max |dO| <= 1e-5 and max |dlse| <= 1e-5.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs

pytestmark = pytest.mark.gpu
NTHREADS = min(16, os.cpu_count() or 1)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits, dtype):
    if dtype == "fp32":
        t = torch.from_numpy(np.ascontiguousarray(bits))
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.float16 if dtype == "fp16" else torch.bfloat16)
    return t.to("cuda")


def ulp_bf16(x):
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, 2.0 ** (e - 7), 2.0 ** -133)


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what):
    """o_gpu/o_ref: float64 [..., D]; lse_gpu/lse_ref float64 [...]."""
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), what + ": non-finite output"
    d_o = np.abs(o_gpu - o_ref)
    d_l = np.abs(lse_gpu - lse_ref)
    if dtype == "fp32":
        tol_o = np.full_like(o_ref, 1e-5)
        tol_l = 1e-5
    elif dtype == "fp16":
        tol_o = np.full_like(o_ref, 1e-2)
        tol_l = 1e-3
    else:
        tol_o = np.maximum(1e-2, ulp_bf16(o_ref))
        tol_l = 1e-3
    n_ulp = int(np.sum((d_o > 1e-2) & (d_o <= tol_o))) if dtype == "bf16" else 0
    _say("%s: max|dO|=%.3e max|dlse|=%.3e elems=%d ulp-allowance=%d" % (what, d_o.max(), d_l.max(), d_o.size, n_ulp))
    bad = d_o > tol_o
    assert not bad.any(), "%s: %d elements over tolerance, worst %.3e" % (what, bad.sum(), d_o.max())
    assert d_l.max() <= tol_l, "%s: lse error %.3e" % (what, d_l.max())


def run_gpu(q, k, v, dtype, layout, causal, scale):
    dev = [to_dev(x, dtype) for x in (q, k, v)]
    o, lse = fa.attention(*dev, layout=layout, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def full_compare(B, H, N, D, dtype, layout, causal, scale, seed, what, qk_mult=1.0):
    q, k, v = inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=seed, qk_mult=qk_mult)
    o, lse = run_gpu(q, k, v, dtype, layout, causal, scale)
    o_ref, lse_ref = oracle.attention(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=scale,
                                      nthreads=NTHREADS)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
          dtype, what)
    return o, lse


# ---- configurations 1 and 2: full comparison ------------------------------------------------------

def test_c1_fp32_bsnd_noncausal_full():
    w = inputs.WORKLOADS["c1"]
    full_compare(w.B, w.H, w.N, w.D, "fp32", w.layout, False, w.scale, w.seed, "c1 fp32")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_c2_16bit_bsnd_full(dtype, causal):
    w = inputs.WORKLOADS["c2"]
    full_compare(w.B, w.H, w.N, w.D, dtype, w.layout, causal, w.scale, w.seed, "c2 %s causal=%d" % (dtype, causal))


# ---- configurations 3 to 5: sampled rows at full size -----------------------------------------------

def sampled_compare(w, rows, what):
    q, k, v = inputs.make_workload(w)
    _say("%s: inputs ready %s" % (what, (w.B, w.H, w.N, w.D)))
    o, lse = run_gpu(q, k, v, "bf16", w.layout, w.causal, w.scale)
    assert w.layout == "BHSD"
    idx = torch.from_numpy(rows).to("cuda")
    o_s = o[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().numpy().astype(np.float64)
    lse_s = lse[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().numpy().astype(np.float64)
    # every output finite, at full size
    assert bool(torch.isfinite(lse).all()), what + ": non-finite lse"
    assert bool(torch.isfinite(o).all()), what + ": non-finite O"
    o_ref, lse_ref = oracle.attention_rows(q, k, v, dtype="bf16", layout=w.layout, causal=w.causal, scale=w.scale,
                                           rows=rows, nthreads=NTHREADS)
    check(o_s, lse_s, o_ref, lse_ref, "bf16", what)


def test_c3_bf16_causal_b8_h32_n4096_sampled():
    w = inputs.WORKLOADS["c3"]
    rows = inputs.sample_rows(w.B, w.H, w.N, 512, seed=3)
    sampled_compare(w, rows, "c3")


def test_c4_bf16_causal_large_logits_sampled():
    w = inputs.WORKLOADS["c4"]
    rows = inputs.sample_rows(w.B, w.H, w.N, 512, seed=4, edge_tiles=1, tile=128, edge_heads=4)
    sampled_compare(w, rows, "c4")


def test_c5_bf16_causal_n65536_sampled():
    w = inputs.WORKLOADS["c5"]
    rows = inputs.sample_rows(w.B, w.H, w.N, 0, seed=5, heads_subset=4, rows_per_head=256)
    sampled_compare(w, rows, "c5")


# ---- ragged sizes, both layouts, all dtypes ----------------------------------------------------------

@pytest.mark.parametrize("N", [200, 256, 384, 385, 456, 512, 640, 768, 1000, 1536])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_causal_tile_pairing_boundary(N, D, dtype):
    # whole causal problems run heavy and light query tiles in pairs when the tile count is even and the
    # sequence spans an even number of 64-key tiles, as 256-query tiles (8 waves) when possible, else as
    # 128-query tiles: N = 512 and 1536 (multiples of 256) pair 256-query tiles on the ping-pong kernel;
    # 384, 456, 1000 pair 256-query tiles on the lockstep kernel; 200, 256, 768 pair 128-query tiles
    # (an odd number of 256-query tiles); 385 (7 key tiles) and 640 (odd tile counts at both sizes) run
    # one 128-query tile per workgroup
    full_compare(2, 3, N, D, dtype, "BHSD", True, 1.0 / math.sqrt(D), 300 + N, "pairing N=%d D=%d %s" % (N, D, dtype))


@pytest.mark.parametrize("N", [1, 7, 64, 100, 130, 257])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_sizes(N, D, dtype, causal):
    layout = "BHSD" if (N + D) % 2 else "BSND"
    full_compare(2, 3, N, D, dtype, layout, causal, 1.0 / math.sqrt(D), 100 + N, "ragged N=%d D=%d %s c=%d %s"
                 % (N, D, dtype, causal, layout))


@pytest.mark.parametrize("layout", ["BHSD", "BSND"])
@pytest.mark.parametrize("dtype", ["fp32", "fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_memory_past_the_end_never_reaches_o(layout, dtype, causal):
    """K and V are views at the start of NaN-filled buffers: the key rows of the last K/V tile that lie past
    the sequence end (of the last head, past the end of the tensor) must not reach O or lse."""
    B, H, N, D = 1, 2, 100, 128
    q, k, v = inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=77)
    qd = to_dev(q, dtype)

    def nan_padded(x):
        t = to_dev(x, dtype)
        buf = torch.full((t.numel() + 64 * H * D + D,), float("nan"), dtype=t.dtype, device="cuda")
        buf[: t.numel()].copy_(t.reshape(-1))
        return buf[: t.numel()].view(t.shape)

    kd, vd = nan_padded(k), nan_padded(v)
    o, lse = fa.attention(qd, kd, vd, layout=layout, causal=causal, scale=0.125)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, dtype=dtype, layout=layout, causal=causal, scale=0.125,
                                      nthreads=NTHREADS)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
          dtype, "NaN past the end %s %s c=%d" % (layout, dtype, causal))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_fp16_large_logits_no_overflow(dtype):
    # Logits of order 300 (Q, K drawn x8, D=128): the fp16 overflow case of the catlass tuning page must
    # stay finite and within tolerance in both 16-bit types.
    full_compare(1, 2, 1000, 128, dtype, "BHSD", True, 1.0 / math.sqrt(128), 41, "large logits " + dtype, qk_mult=8.0)


def test_fp32_large_logits_within_dot_product_bound():
    # fp32 with logits of order 300: |lse| ~ 250, where one fp32 ulp is already 1.5e-5, so the 1e-5
    # bound for unit-scale fp32 inputs cannot apply.  The bound used instead is the a-priori rounding
    # bound of an fp32 dot product of length D: |ds_ij| <= 2*D*u*scale*sum_d |q_id k_jd| (u = 2^-24),
    # hence |dlse_i| <= max_j |ds_ij| and |dO_i| <= 2 max_j |ds_ij| max_j |v_j| (+1e-5 for the rest).
    B, H, N, D = 1, 2, 1000, 128
    scale = 1.0 / math.sqrt(D)
    q, k, v = inputs.make(B, H, N, D, layout="BHSD", dtype="fp32", seed=41, qk_mult=8.0)
    o, lse = run_gpu(q, k, v, "fp32", "BHSD", True, scale)
    o_ref, lse_ref = oracle.attention(q, k, v, dtype="fp32", layout="BHSD", causal=True, scale=scale, nthreads=NTHREADS)
    qa, ka = np.abs(q.astype(np.float64)), np.abs(k.astype(np.float64))
    dot_abs = np.einsum("bhid,bhjd->bhij", qa, ka)
    dot_abs = np.where(np.tril(np.ones((N, N), dtype=bool)), dot_abs, 0.0)
    ds = 2 * D * 2.0 ** -24 * scale * dot_abs.max(axis=-1)          # [B, H, N]
    vmax = np.abs(v.astype(np.float64)).max(axis=(2, 3))[..., None]  # [B, H, 1]
    d_l = np.abs(lse.cpu().numpy().astype(np.float64) - lse_ref)
    d_o = np.abs(o.cpu().numpy().astype(np.float64) - o_ref).max(axis=-1)
    _say("fp32 large logits: max|dlse|=%.3e (bound %.3e)  max|dO|=%.3e (bound %.3e)"
         % (d_l.max(), ds.max(), d_o.max(), (2 * ds * vmax + 1e-5).max()))
    assert np.all(np.isfinite(d_o)) and np.all(np.isfinite(d_l))
    assert np.all(d_l <= ds + 1e-5)
    assert np.all(d_o <= 2 * ds * vmax + 1e-5)


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.7])
@pytest.mark.parametrize("N,D", [(300, 64), (512, 128), (1024, 64)])
def test_scale_values(scale, N, D):
    # a negative scale flips Q's sign bits: N = 300 runs the lockstep kernel, N = 512 and 1024 the ping-pong
    # kernel (causal pairs, non-causal units), which flips each unit's Q right before its first product
    for causal in (False, True):
        full_compare(1, 2, N, D, "bf16", "BSND", causal, scale, 51 + N,
                     "scale=%g N=%d D=%d causal=%d" % (scale, N, D, causal))


# ---- bit-exact properties of the kernel ----------------------------------------------------------------

def test_causal_row0_is_v0_bit_exact():
    for dtype in ("bf16", "fp16", "fp32"):
        q, k, v = inputs.make(2, 4, 300, 128, layout="BHSD", dtype=dtype, seed=61)
        o, lse = run_gpu(q, k, v, dtype, "BHSD", True, 0.0883883)
        vd = to_dev(v, dtype)
        assert torch.equal(o[:, :, 0, :], vd[:, :, 0, :]), dtype


def test_layouts_bit_identical_and_repeat_deterministic():
    for dtype in ("bf16", "fp32"):
        q, k, v = inputs.make(2, 3, 333, 64, layout="BHSD", dtype=dtype, seed=62)
        o1, l1 = run_gpu(q, k, v, dtype, "BHSD", True, 0.125)
        o1b, l1b = run_gpu(q, k, v, dtype, "BHSD", True, 0.125)
        t = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
        o2, l2 = run_gpu(t(q), t(k), t(v), dtype, "BSND", True, 0.125)
        assert torch.equal(o1, o1b) and torch.equal(l1, l1b)
        assert torch.equal(o1, o2.transpose(1, 2)) and torch.equal(l1, l2)


def test_constant_v():
    q, k, _ = inputs.make(1, 2, 200, 64, layout="BHSD", dtype="bf16", seed=63)
    v = inputs.cast_bits(np.full((1, 2, 200, 64), -1.5, dtype=np.float32), "bf16")
    o, _ = run_gpu(q, k, v, "bf16", "BHSD", False, 0.125)
    assert torch.equal(o, torch.full_like(o, -1.5))


def test_host_pointer_rejected():
    q = np.zeros((1, 1, 64, 64), dtype=np.float32)
    dev = torch.zeros(1, 1, 64, 64, device="cuda")
    lse = torch.zeros(1, 1, 64, device="cuda")
    st = fa.fa_fwd(q.ctypes.data, dev.data_ptr(), dev.data_ptr(), torch.empty_like(dev).data_ptr(), lse.data_ptr(),
                   1, 1, 64, 64, 0, 0, 0.125, 0, 0)
    assert st == fa.FA_ERR_NOT_DEVICE_MEMORY


def test_untouched_outputs_on_error():
    q = torch.randn(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 3.0)
    lse = torch.full((1, 2, 64), 7.0, device="cuda")
    st = fa.fa_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 2, 64, 96, 0, 0, 0.1,
                   fa.DTYPE_BF16, 0)
    assert st == fa.FA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 7.0).all())


def test_on_a_side_stream():
    q, k, v = inputs.make(1, 2, 256, 64, layout="BHSD", dtype="bf16", seed=64)
    dev = [to_dev(x, "bf16") for x in (q, k, v)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.attention(*dev, layout="BHSD", causal=True, scale=0.125)
    s.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, dtype="bf16", layout="BHSD", causal=True, scale=0.125)
    check(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
          "bf16", "side stream")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_short_rows(dtype, causal):
    # B*H = 2048 (b, h) units of 17 rows: the workgroup -> unit mapping with a large, ragged grid
    full_compare(64, 32, 17, 64, dtype, "BSND", causal, 0.125, 43, "many heads %s causal=%d" % (dtype, causal))
