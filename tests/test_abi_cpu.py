"""The C-ABI library loads, exports what include/fa.h declares, and rejects bad arguments before any
HIP call (so these run on a host without a GPU)."""
import os
import re
import subprocess

import pytest

import transformer_attention_fwd_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(fa_\w+)\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    declared = _declared()
    assert declared == ["fa_bwd", "fa_bwd_atomic", "fa_bwd_ex", "fa_bwd_noalloc", "fa_bwd_varlen", "fa_fwd", "fa_fwd_ex", "fa_fwd_varlen",
                        "fa_last_error",
                        "fa_merge", "fa_status_str", "fa_version"]
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.split() and l.split()[1] == "T"}
    for name in declared:
        assert name in exported, name
    lib = fa.load()
    for name in declared:
        assert hasattr(lib, name)


def test_header_constants_match_binding():
    src = open(os.path.join(ROOT, "include", "fa.h")).read()
    consts = dict((m[0], int(m[1])) for m in re.findall(r"#define (FA_\w+) (\d+)", src))
    assert consts["FA_LAYOUT_BHSD"] == fa.LAYOUT_BHSD and consts["FA_LAYOUT_BSND"] == fa.LAYOUT_BSND
    assert consts["FA_DTYPE_FP32"] == fa.DTYPE_FP32 and consts["FA_DTYPE_FP16"] == fa.DTYPE_FP16
    assert consts["FA_DTYPE_BF16"] == fa.DTYPE_BF16
    for name in ("FA_OK", "FA_ERR_NULL", "FA_ERR_BAD_DIM", "FA_ERR_BAD_LAYOUT", "FA_ERR_BAD_DTYPE",
                 "FA_ERR_UNSUPPORTED", "FA_ERR_BAD_SCALE", "FA_ERR_MISALIGNED", "FA_ERR_ALIAS",
                 "FA_ERR_NOT_DEVICE_MEMORY", "FA_ERR_HIP", "FA_ERR_BAD_RANGE", "FA_ERR_SCRATCH_LIMIT"):
        assert consts[name] == getattr(fa, name), name
    assert consts["FA_NOALLOC_MAX_ROWS"] == fa.NOALLOC_MAX_ROWS


def test_status_strings_and_version():
    assert fa.version() == 600
    for st in range(12):
        assert fa.status_str(st)
    assert fa.status_str(0) == "ok"
    assert fa.status_str(999) == "unknown status"


# Fake, distinct, 16-byte aligned "device" addresses; pure argument checks must fail before any HIP call.
SZ = 1 << 40
Q, K, V, O, L = (0x10000000000 + i * (SZ * 4) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=64, D=64, layout=0, causal=0, scale=0.125, dtype=2, stream=0)


def _call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"], a["layout"],
                     a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(k=0), fa.FA_ERR_NULL), (dict(v=0), fa.FA_ERR_NULL),
    (dict(o=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL),
    (dict(layout=2), fa.FA_ERR_BAD_LAYOUT), (dict(layout=-1), fa.FA_ERR_BAD_LAYOUT),
    (dict(dtype=3), fa.FA_ERR_BAD_DTYPE), (dict(dtype=-1), fa.FA_ERR_BAD_DTYPE),
    (dict(B=0), fa.FA_ERR_BAD_DIM), (dict(H=0), fa.FA_ERR_BAD_DIM), (dict(N=0), fa.FA_ERR_BAD_DIM),
    (dict(D=0), fa.FA_ERR_BAD_DIM), (dict(N=-5), fa.FA_ERR_BAD_DIM),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED), (dict(D=256), fa.FA_ERR_UNSUPPORTED), (dict(D=32), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 30) + 1), fa.FA_ERR_UNSUPPORTED), (dict(B=1 << 20, H=1 << 12), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 40, H=1 << 40), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE), (dict(scale=float("inf")), fa.FA_ERR_BAD_SCALE),
    (dict(scale=3.0e38), fa.FA_ERR_BAD_SCALE),
    (dict(q=Q + 8), fa.FA_ERR_MISALIGNED), (dict(lse=L + 4), fa.FA_ERR_MISALIGNED),
    (dict(o=Q), fa.FA_ERR_ALIAS), (dict(o=K + 64), fa.FA_ERR_ALIAS), (dict(lse=V + 1024), fa.FA_ERR_ALIAS),
    (dict(lse=O + 16), fa.FA_ERR_ALIAS),
])
def test_pure_argument_checks(kw, status):
    assert _call(**kw) == status


def test_check_order_null_before_layout_before_dims():
    assert _call(q=0, layout=7, B=0) == fa.FA_ERR_NULL
    assert _call(layout=7, dtype=9) == fa.FA_ERR_BAD_LAYOUT
    assert _call(dtype=9, B=0) == fa.FA_ERR_BAD_DTYPE
    assert _call(B=0, D=96) == fa.FA_ERR_BAD_DIM
    assert _call(D=96, scale=float("nan")) == fa.FA_ERR_UNSUPPORTED


def test_inputs_may_alias_each_other():
    # q, k, v are read-only and may share memory (self-attention on one buffer): not an alias error.
    # Without a GPU the call then stops at the device checks, never with FA_ERR_ALIAS.
    st = _call(k=Q, v=Q)
    assert st != fa.FA_ERR_ALIAS and st != fa.FA_OK


def test_wrapper_rejects_shape_mismatch_before_calling():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.attention(q, torch.zeros(1, 2, 9, 64), q)
    with pytest.raises(ValueError):
        fa.attention(q, q, q, layout="BNSD")
    with pytest.raises(TypeError):
        fa.attention(q.double(), q.double(), q.double())



def test_merge_wrapper_rejects_bad_caller_outputs():
    # fa_merge writes one part's worth of O and B*H*N lse floats: an undersized, wrong-dtype or strided
    # out or lse would be written past its end, so the wrapper raises before any library call
    torch = pytest.importorskip("torch")
    parts = torch.zeros(3, 1, 2, 8, 64, dtype=torch.bfloat16)
    lparts = torch.zeros(3, 1, 2, 8)
    with pytest.raises(ValueError):
        fa.merge(parts, lparts, out=torch.zeros(1, 2, 7, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.merge(parts.float(), lparts, out=torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fa.merge(parts, lparts, out=torch.zeros(1, 2, 64, 8, dtype=torch.bfloat16).transpose(2, 3))
    with pytest.raises(ValueError):
        fa.merge(parts, lparts, lse=torch.zeros(1, 2, 4))
    with pytest.raises(ValueError):
        fa.merge(parts, lparts, lse=torch.zeros(1, 2, 8, dtype=torch.float16))
    with pytest.raises(ValueError):
        fa.merge(parts, lparts, lse=torch.zeros(1, 8, 2).transpose(1, 2))

def test_backward_wrappers_reject_bad_caller_buffers():
    # a caller's delta or gradient buffer of the wrong shape, dtype or strides would be written past its
    # end by the kernels: the wrappers raise before any library call
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.float16)
    lse = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        fa.attention_bwd(q, q, q, q, lse, q, delta=torch.zeros(1, 2, 7))
    with pytest.raises(ValueError):
        fa.attention_bwd_ex(q, q, q, q, lse, q, delta=torch.zeros(1, 2, 8, dtype=torch.float64))
    with pytest.raises(ValueError):
        fa.attention_bwd_ex(q, q, q, q, lse, q, dk=torch.zeros(1, 2, 4, 64, dtype=torch.float16))
    p = torch.zeros(12, 2, 64, dtype=torch.float16)
    lse_p = torch.zeros(2, 12)
    cu = torch.tensor([0, 5, 12], dtype=torch.int32)
    with pytest.raises(ValueError):
        fa.attention_bwd_varlen(p, p, p, p, lse_p, p, cu, cu, 7, 7, delta=torch.zeros(12, 2))
    with pytest.raises(ValueError):
        fa.attention_bwd_varlen(p, p, p, p, lse_p, p, cu, cu, 7, 7, out=(p, p, torch.zeros(11, 2, 64,
                                                                                         dtype=torch.float16)))
    with pytest.raises(ValueError):
        fa.attention_bwd_varlen(p, p, p, p, lse_p, p, cu, cu, 7, 7, out=(p, p, p.transpose(0, 1)))


def test_every_kernel_stub_is_defined():
    # A kernel whose host-side stub failed to instantiate leaves an undefined __device_stub__ symbol:
    # the library would then fail to load at run time.
    out = subprocess.run(["nm", "-C", "--undefined-only", fa.library_path()], stdout=subprocess.PIPE, text=True,
                         check=True).stdout
    assert "__device_stub__" not in out, out


# ---- fa_fwd_ex and fa_merge: pure argument checks ----
GOOD_EX = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Nq=64, Nk=100, D=64, layout=0, causal=1, window=-1, q_offset=36,
               kv_start=0, kv_len=100, scale=0.125, dtype=2, stream=0)


def _call_ex(**kw):
    a = dict(GOOD_EX)
    a.update(kw)
    return fa.fa_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"], a["D"],
                        a["layout"], a["causal"], a["window"], a["q_offset"], a["kv_start"], a["kv_len"], a["scale"],
                        a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(v=0), fa.FA_ERR_NULL), (dict(layout=5), fa.FA_ERR_BAD_LAYOUT),
    (dict(dtype=7), fa.FA_ERR_BAD_DTYPE), (dict(Nq=0), fa.FA_ERR_BAD_DIM), (dict(Nk=0), fa.FA_ERR_BAD_DIM),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED), (dict(Nk=(1 << 30) + 1, kv_len=1), fa.FA_ERR_UNSUPPORTED),
    (dict(kv_start=-1), fa.FA_ERR_BAD_RANGE), (dict(kv_len=-1), fa.FA_ERR_BAD_RANGE),
    (dict(kv_start=50, kv_len=51), fa.FA_ERR_BAD_RANGE), (dict(kv_start=101, kv_len=0), fa.FA_ERR_BAD_RANGE),
    (dict(causal=0, window=3), fa.FA_ERR_BAD_RANGE), (dict(q_offset=(1 << 30) + 1), fa.FA_ERR_BAD_RANGE),
    (dict(q_offset=-(1 << 30) - 1), fa.FA_ERR_BAD_RANGE),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE), (dict(k=K + 4), fa.FA_ERR_MISALIGNED),
    (dict(o=K + 64 * 2), fa.FA_ERR_ALIAS), (dict(lse=O + 16), fa.FA_ERR_ALIAS),
])
def test_fa_fwd_ex_argument_checks(kw, status):
    assert _call_ex(**kw) == status


def test_fa_fwd_ex_range_check_comes_after_size_limits():
    # a bad chunk and an unsupported D together: the size error wins (documented order)
    assert _call_ex(D=96, kv_start=-1) == fa.FA_ERR_UNSUPPORTED
    # an empty chunk at the end is a valid range (it fails later, on the fake device pointers)
    assert _call_ex(kv_start=100, kv_len=0) not in (fa.FA_ERR_BAD_RANGE, fa.FA_OK)


GOOD_M = dict(op=Q, lp=K, n=3, o=O, lse=L, B=1, H=2, N=64, D=64, layout=0, dtype=2, stream=0)


def _call_m(**kw):
    a = dict(GOOD_M)
    a.update(kw)
    return fa.fa_merge(a["op"], a["lp"], a["n"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["D"], a["layout"],
                       a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(op=0), fa.FA_ERR_NULL), (dict(lse=0), fa.FA_ERR_NULL), (dict(layout=3), fa.FA_ERR_BAD_LAYOUT),
    (dict(dtype=3), fa.FA_ERR_BAD_DTYPE), (dict(n=0), fa.FA_ERR_BAD_DIM), (dict(N=0), fa.FA_ERR_BAD_DIM),
    (dict(D=100), fa.FA_ERR_UNSUPPORTED), (dict(n=1 << 40), fa.FA_ERR_UNSUPPORTED),
    (dict(o=Q + 8), fa.FA_ERR_MISALIGNED), (dict(o=Q + 2 * 2 * 64 * 64 * 2), fa.FA_ERR_ALIAS),
    (dict(lse=K + 16), fa.FA_ERR_ALIAS), (dict(lse=O), fa.FA_ERR_ALIAS),
])
def test_fa_merge_argument_checks(kw, status):
    assert _call_m(**kw) == status


# ---- fa_bwd: pure argument checks ----
DO, DQ, DK, DV, DL = (0x10000000000 + i * (SZ * 4) for i in range(5, 10))
GOOD_B = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, delta=DL, B=1, H=2, N=64, D=64, layout=0,
              causal=1, scale=0.125, dtype=2, stream=0)


def _call_b(**kw):
    a = dict(GOOD_B)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"], a["B"],
                     a["H"], a["N"], a["D"], a["layout"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(do=0), fa.FA_ERR_NULL), (dict(delta=0), fa.FA_ERR_NULL),
    (dict(dv=0), fa.FA_ERR_NULL), (dict(layout=2), fa.FA_ERR_BAD_LAYOUT), (dict(dtype=5), fa.FA_ERR_BAD_DTYPE),
    (dict(N=0), fa.FA_ERR_BAD_DIM), (dict(B=0), fa.FA_ERR_BAD_DIM), (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=(1 << 30) + 1), fa.FA_ERR_UNSUPPORTED),
    # fp32: 4-byte elements, so dk 16 KiB after dq (clear of 2 x 64 x 64 bf16 elements) overlaps it
    (dict(dtype=0, dk=DQ + 2 * 64 * 64 * 2), fa.FA_ERR_ALIAS),
    (dict(scale=float("inf")), fa.FA_ERR_BAD_SCALE), (dict(dk=DK + 2), fa.FA_ERR_MISALIGNED),
    (dict(delta=L + 4), fa.FA_ERR_MISALIGNED),
    (dict(dq=Q), fa.FA_ERR_ALIAS), (dict(dk=O + 64 * 2), fa.FA_ERR_ALIAS), (dict(dv=DO), fa.FA_ERR_ALIAS),
    (dict(delta=L + 16), fa.FA_ERR_ALIAS), (dict(dv=DQ + 16), fa.FA_ERR_ALIAS), (dict(delta=DK), fa.FA_ERR_ALIAS),
])
def test_fa_bwd_argument_checks(kw, status):
    assert _call_b(**kw) == status


def test_fa_bwd_good_arguments_reach_the_device_check():
    # every pure check passes; the fake pointers then fail the residency check (or HIP is absent)
    assert _call_b() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)



# ---- fa_bwd_noalloc: pure argument checks (fa_bwd's, without delta, plus the scratch limit) ----
def _call_n(**kw):
    a = dict(GOOD_B)
    a.update(kw)
    return fa.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                             a["H"], a["N"], a["D"], a["layout"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(dv=0), fa.FA_ERR_NULL), (dict(layout=2), fa.FA_ERR_BAD_LAYOUT),
    (dict(dtype=5), fa.FA_ERR_BAD_DTYPE), (dict(N=0), fa.FA_ERR_BAD_DIM), (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    # B*H*N one row past the scratch array, and far past it, before any HIP call
    (dict(B=1, H=1, N=4194305), fa.FA_ERR_SCRATCH_LIMIT), (dict(B=8, H=32, N=65536), fa.FA_ERR_SCRATCH_LIMIT),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE), (dict(dk=DK + 2), fa.FA_ERR_MISALIGNED),
    (dict(dq=Q), fa.FA_ERR_ALIAS), (dict(dv=DQ + 16), fa.FA_ERR_ALIAS),
])
def test_fa_bwd_noalloc_argument_checks(kw, status):
    assert _call_n(**kw) == status


def test_fa_bwd_noalloc_good_arguments_reach_the_device_check():
    # the largest accepted size passes the pure checks too
    assert _call_n() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
    assert _call_n(B=1, H=64, N=65536) in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)


# ---- fa_bwd_atomic: fa_bwd's checks plus the fp32 dq_accum workspace ----
ACC = 0x10000000000 + 12 * (SZ * 4)


def _call_a(acc=ACC, **kw):
    a = dict(GOOD_B)
    a.update(kw)
    return fa.fa_bwd_atomic(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                            acc, a["B"], a["H"], a["N"], a["D"], a["layout"], a["causal"], a["scale"], a["dtype"],
                            a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(acc=0), fa.FA_ERR_NULL), (dict(delta=0), fa.FA_ERR_NULL), (dict(q=0), fa.FA_ERR_NULL),
    (dict(layout=2), fa.FA_ERR_BAD_LAYOUT), (dict(dtype=5), fa.FA_ERR_BAD_DTYPE), (dict(N=0), fa.FA_ERR_BAD_DIM),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED), (dict(dtype=0), fa.FA_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE), (dict(acc=ACC + 4), fa.FA_ERR_MISALIGNED),
    # the workspace holds 2 x 64 x 64 floats (32 KiB): it must clear every input, output and delta
    (dict(acc=Q), fa.FA_ERR_ALIAS), (dict(acc=DQ - 2 * 64 * 64 * 4 + 16), fa.FA_ERR_ALIAS),
    (dict(acc=DL + 16), fa.FA_ERR_ALIAS), (dict(acc=DV), fa.FA_ERR_ALIAS), (dict(dq=Q), fa.FA_ERR_ALIAS),
])
def test_fa_bwd_atomic_argument_checks(kw, status):
    assert _call_a(**kw) == status


def test_fa_bwd_atomic_good_arguments_reach_the_device_check():
    assert _call_a() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
    # a workspace right after dq (its 16 KiB of bf16) does not overlap it
    assert _call_a(acc=DQ + 2 * 64 * 64 * 2) in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)


# ---- fa_fwd_varlen: pure argument checks ----
CQ, CK = 0x10000000000 + 10 * (SZ * 4), 0x10000000000 + 11 * (SZ * 4)
GOOD_V = dict(q=Q, k=K, v=V, o=O, lse=L, cq=CQ, ck=CK, B=3, H=2, tq=300, tk=500, mq=128, D=128, causal=1,
              scale=0.088, dtype=2, stream=0)


def _call_v(**kw):
    a = dict(GOOD_V)
    a.update(kw)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["B"], a["H"], a["tq"], a["tk"],
                            a["mq"], a["D"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL), (dict(cq=0), fa.FA_ERR_NULL), (dict(ck=0), fa.FA_ERR_NULL),
    (dict(dtype=9), fa.FA_ERR_BAD_DTYPE), (dict(B=0), fa.FA_ERR_BAD_DIM), (dict(tq=0), fa.FA_ERR_BAD_DIM),
    (dict(tk=0), fa.FA_ERR_BAD_DIM), (dict(mq=0), fa.FA_ERR_BAD_DIM), (dict(D=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED), (dict(tq=(1 << 30) + 1, mq=1), fa.FA_ERR_UNSUPPORTED),
    (dict(mq=301), fa.FA_ERR_BAD_RANGE), (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE),
    (dict(v=V + 8), fa.FA_ERR_MISALIGNED), (dict(cq=CQ + 2), fa.FA_ERR_MISALIGNED),
    (dict(o=Q + 64), fa.FA_ERR_ALIAS), (dict(lse=CK), fa.FA_ERR_ALIAS), (dict(lse=O + 16), fa.FA_ERR_ALIAS),
])
def test_fa_fwd_varlen_argument_checks(kw, status):
    assert _call_v(**kw) == status


def test_fa_fwd_varlen_good_arguments_reach_the_device_check():
    assert _call_v() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)


# ---- fa_bwd_ex: pure argument checks ----
GOOD_BX = dict(GOOD_B, Nq=64, Nk=100, window=-1, q_offset=36, kv_start=0, kv_len=100)
del GOOD_BX["N"]


def _call_bx(**kw):
    a = dict(GOOD_BX)
    a.update(kw)
    return fa.fa_bwd_ex(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"], a["B"],
                        a["H"], a["Nq"], a["Nk"], a["D"], a["layout"], a["causal"], a["window"], a["q_offset"],
                        a["kv_start"], a["kv_len"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dk=0), fa.FA_ERR_NULL), (dict(Nk=0), fa.FA_ERR_BAD_DIM), (dict(Nq=0), fa.FA_ERR_BAD_DIM),
    (dict(kv_start=-1), fa.FA_ERR_BAD_RANGE),
    (dict(kv_start=60, kv_len=41), fa.FA_ERR_BAD_RANGE), (dict(causal=0, window=4), fa.FA_ERR_BAD_RANGE),
    (dict(q_offset=(1 << 30) + 1), fa.FA_ERR_BAD_RANGE), (dict(D=80, kv_start=-1), fa.FA_ERR_UNSUPPORTED),
    (dict(dv=V + 32), fa.FA_ERR_ALIAS), (dict(delta=L + 8), fa.FA_ERR_MISALIGNED),
])
def test_fa_bwd_ex_argument_checks(kw, status):
    assert _call_bx(**kw) == status


def test_fa_bwd_ex_good_arguments_reach_the_device_check():
    assert _call_bx() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
    assert _call_bx(dtype=0) in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
    assert _call_b(dtype=0, dk=DQ + 2 * 64 * 64 * 4) in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
    assert _call_bx(kv_start=100, kv_len=0) in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)


# ---- fa_bwd_varlen: pure argument checks ----
CQ, CK = 0x10000000000 + 11 * (SZ * 4), 0x10000000000 + 12 * (SZ * 4)
GOOD_BV = dict(q=Q, k=K, v=V, o=O, lse=L, do=DO, dq=DQ, dk=DK, dv=DV, delta=DL, cq=CQ, ck=CK, B=3, H=2, tq=300,
               tk=400, mq=150, mk=200, D=128, causal=1, scale=0.1, dtype=2, stream=0)


def _call_bv(**kw):
    a = dict(GOOD_BV)
    a.update(kw)
    return fa.fa_bwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["delta"],
                            a["cq"], a["ck"], a["B"], a["H"], a["tq"], a["tk"], a["mq"], a["mk"], a["D"], a["causal"],
                            a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ck=0), fa.FA_ERR_NULL), (dict(delta=0), fa.FA_ERR_NULL), (dict(dtype=7), fa.FA_ERR_BAD_DTYPE),
    (dict(mk=0), fa.FA_ERR_BAD_DIM), (dict(tq=0), fa.FA_ERR_BAD_DIM), (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=0), fa.FA_ERR_UNSUPPORTED), (dict(mq=301), fa.FA_ERR_BAD_RANGE), (dict(mk=401), fa.FA_ERR_BAD_RANGE),
    (dict(scale=float("nan")), fa.FA_ERR_BAD_SCALE), (dict(cq=CQ + 2), fa.FA_ERR_MISALIGNED),
    (dict(dv=DQ + 16), fa.FA_ERR_ALIAS), (dict(delta=CK), fa.FA_ERR_ALIAS), (dict(dk=V + 16), fa.FA_ERR_ALIAS),
])
def test_fa_bwd_varlen_argument_checks(kw, status):
    assert _call_bv(**kw) == status


def test_fa_bwd_varlen_good_arguments_reach_the_device_check():
    assert _call_bv() in (fa.FA_ERR_NOT_DEVICE_MEMORY, fa.FA_ERR_HIP)
