"""Seeded input generators: determinism, nearest-even casts against torch's CPU casts, samplers."""
import numpy as np
import torch

from transformer_attention_fwd_amd import inputs


def test_bf16_cast_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.0e38, 1e-40, 1.00390625, 1.01171875, np.inf, -np.inf],
                                 dtype=np.float32)])
    ours = inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy())


def test_f16_cast_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 100
    ours = inputs.f32_to_f16_bits(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_generation_is_deterministic_and_layouts_agree():
    a = inputs.make(1, 3, 20, 8, layout="BHSD", dtype="bf16", seed=3)
    b = inputs.make(1, 3, 20, 8, layout="BHSD", dtype="bf16", seed=3)
    c = inputs.make(1, 3, 20, 8, layout="BSND", dtype="bf16", seed=3)
    for x, y, z in zip(a, b, c):
        np.testing.assert_array_equal(x, y)
        np.testing.assert_array_equal(x, z.transpose(0, 2, 1, 3))
    d = inputs.make(1, 3, 20, 8, layout="BHSD", dtype="bf16", seed=4)
    assert not np.array_equal(a[0], d[0])


def test_qk_multiplier():
    q1, k1, v1 = inputs.draw_f32(1, 1, 8, 4, 9)
    q8, k8, v8 = inputs.draw_f32(1, 1, 8, 4, 9, qk_mult=8.0)
    np.testing.assert_array_equal(q8, q1 * 8)
    np.testing.assert_array_equal(k8, k1 * 8)
    np.testing.assert_array_equal(v8, v1)


def test_workload_table():
    w = inputs.WORKLOADS["c3"]
    assert (w.B, w.H, w.N, w.D, w.layout, w.causal) == (8, 32, 4096, 128, "BHSD", True)
    assert w.flops() == 1099511627776.0
    assert inputs.WORKLOADS["c5"].flops() == 35184372088832.0
    assert inputs.WORKLOADS["c1"].scale == np.float32(0.125)


def test_sampler():
    r = inputs.sample_rows(2, 3, 1000, 50, seed=1)
    assert r.shape == (50, 3) and len(np.unique(r, axis=0)) == 50
    np.testing.assert_array_equal(r, inputs.sample_rows(2, 3, 1000, 50, seed=1))
    r2 = inputs.sample_rows(2, 3, 1000, 0, seed=2, heads_subset=2, rows_per_head=10)
    for bh in np.unique(r2[:, :2], axis=0):
        rows = r2[(r2[:, 0] == bh[0]) & (r2[:, 1] == bh[1]), 2]
        assert 0 in rows and 999 in rows
    r3 = inputs.sample_rows(1, 4, 1000, 5, seed=3, edge_tiles=1, tile=128, edge_heads=2)
    assert len(r3) >= 2 * 256
