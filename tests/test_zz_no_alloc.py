"""fa_bwd_noalloc (the backward whose D workspace is the library's static per-GPU array) against fa_bwd.

Two calls in a row on one GPU, the second smaller than the first: the shared array keeps the first call's
values, so the second call shows that nothing in it needs clearing.  The results must equal fa_bwd's bit
for bit (same kernels, same arithmetic; only the workspace differs)."""
import numpy as np
import pytest
import torch

import transformer_attention_fwd_amd as fa
from transformer_attention_fwd_amd import inputs

pytestmark = pytest.mark.gpu
DTYPES = {"fp32": (torch.float32, fa.DTYPE_FP32), "fp16": (torch.float16, fa.DTYPE_FP16),
          "bf16": (torch.bfloat16, fa.DTYPE_BF16)}


def _dev(x, dtype):
    if dtype == "fp32":
        return torch.from_numpy(x).cuda()
    return torch.from_numpy(x.view(np.int16)).view(DTYPES[dtype][0]).cuda()


def _case(B, H, N, D, layout, causal, dtype, seed, on_device=False):
    if on_device:  # large sizes: seeded draws made on the GPU (any values do: the check is fa_bwd's result)
        g = torch.Generator(device="cuda").manual_seed(seed)
        shape = (B, H, N, D) if layout == "BHSD" else (B, N, H, D)
        q, k, v, do = (torch.randn(shape, generator=g, device="cuda").to(DTYPES[dtype][0]) for _ in range(4))
    else:
        q, k, v = (_dev(x, dtype) for x in inputs.make(B, H, N, D, layout=layout, dtype=dtype, seed=seed))
        do = _dev(inputs.make_grad(B, H, N, D, layout=layout, dtype=dtype, seed=seed), dtype)
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o, lse = fa.attention(q, k, v, layout=layout, causal=causal, scale=scale)
    ref = fa.attention_bwd(q, k, v, o, lse, do, layout=layout, causal=causal, scale=scale)
    got = [torch.empty_like(q) for _ in range(3)]
    st = fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                           got[0].data_ptr(), got[1].data_ptr(), got[2].data_ptr(), B, H, N, D,
                           fa.LAYOUT_BHSD if layout == "BHSD" else fa.LAYOUT_BSND, causal, scale, DTYPES[dtype][1],
                           torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, (st, fa.status_str(st), fa.last_error())
    torch.cuda.synchronize()
    for name, r, g in zip(("dQ", "dK", "dV"), ref, got):
        assert torch.equal(r, g), "%s differs from fa_bwd (%s B=%d H=%d N=%d D=%d)" % (name, dtype, B, H, N, D)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_noalloc_two_calls_match_fa_bwd(dtype):
    _case(2, 4, 1000, 128, "BHSD", True, dtype, seed=801)   # 8000 rows of the array
    _case(1, 3, 300, 64, "BSND", False, dtype, seed=802)    # then 900: the first call's values stay behind


def test_noalloc_largest_size_and_limit():
    # B*H*N exactly at the array's size is accepted (and matches fa_bwd); one row more is refused
    B, H, N, D = fa.NOALLOC_MAX_ROWS // (16 * 64), 16, 64, 64
    assert B * H * N == fa.NOALLOC_MAX_ROWS
    _case(B, H, N, D, "BHSD", True, "bf16", seed=803, on_device=True)
    _case(1, 2, 200, 128, "BHSD", True, "bf16", seed=804)  # and a small call after it
    q = torch.zeros((1, 1, fa.NOALLOC_MAX_ROWS + 1, 64), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((1, 1, fa.NOALLOC_MAX_ROWS + 1), dtype=torch.float32, device="cuda")
    st = fa.fa_bwd_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), q.data_ptr(), lse.data_ptr(), q.data_ptr(),
                           q.data_ptr(), q.data_ptr(), q.data_ptr(), 1, 1, fa.NOALLOC_MAX_ROWS + 1, 64, fa.LAYOUT_BHSD,
                           1, 0.125, fa.DTYPE_BF16, 0)
    assert st == fa.FA_ERR_SCRATCH_LIMIT
