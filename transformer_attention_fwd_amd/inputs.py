"""Seeded synthetic inputs for the attention forward: workloads, round-to-nearest-even casts, row samplers.

This module holds no attention arithmetic.  It is the one piece shared by the tests, the benchmark and
the oracle checks: the same host bits are uploaded to the device and handed to the oracle.

Workloads.  The pages measure real models on real prompts; those weights and texts are not available,
so Gaussian activations of the same attention shapes stand in for them:
  * ``c1`` fp32, B=1 H=2 N=512 D=64, BSND, non-causal: the deployment page's smoke-test shape
    (hwcomputing.csdn.net/6a0d4444..., the minimal test with batch 1, 2 heads, seq 512, d 64).
  * ``c2`` fp16 and bf16 from one fp32 draw, B=1 H=8 N=512 D=64, BSND: the same page's precision
    check shape ([1, 512, 8, 64], seed 42).
  * ``c3`` bf16, causal, B=8 H=32 N=4096 D=128, BHSD: page ai6s.net/6a0d3bfb..., the inference
    example with batch 8 and sequence 4096 (32 heads of 128 in its code).
  * ``c4`` bf16, causal, B=2 H=40 N=8192 D=128, BHSD, with Q and K drawn 8 times larger: the long
    sequence that overflowed in fp16 on page hwcomputing.csdn.net/6a0d4681..., section
    "精度选择：FP16还是BF16？" (batch 2 at 8192); the x8 logits stand in for its peaky rows.
  * ``c5`` bf16, causal, B=1 H=32 N=65536 D=128, BHSD: the 64K case of page ai6s.net/6a140d07...

Draw recipe: ``numpy.random.default_rng([42, c])``; Q, K, V = ``standard_normal((B, H, N, D), float32)``
in that order, in logical [B, H, N, D] order, multiplied by the config's factor, rounded to the
config's dtype (nearest-even), then stored in the config's layout.  The upstream gradient dO of the
backward pass comes from its own stream, ``default_rng([42, c, 7])``, as one more standard normal draw
of the same shape, rounded and stored the same way.

Packed variable-length batches (``make_varlen``): Q [total_q, H, D] then K, V [total_k, H, D] from
``default_rng([42, seed, 11])``, rounded the same way; their upstream gradient dO [total_q, H, D]
(``make_grad_varlen``) from ``default_rng([42, seed, 12])``; ``varlen_lengths`` draws the sequence
lengths uniformly from an inclusive range with ``default_rng([4243, seed])``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_DTYPE_ITEMSIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    layout: str          # "BHSD" or "BSND"
    causal: bool
    seed: int            # second word of the generator seed [42, seed]
    qk_mult: float = 1.0  # Q and K are drawn as qk_mult * N(0, 1)
    dtypes: tuple = field(default=("bf16",))

    @property
    def scale(self) -> float:
        """1/sqrt(D) rounded to fp32, the value handed to the library."""
        return float(np.float32(1.0 / math.sqrt(self.D)))

    def flops(self, causal: bool | None = None) -> float:
        """Algorithmic FLOP count 4*B*H*N^2*D, halved when causal."""
        c = self.causal if causal is None else causal
        f = 4.0 * self.B * self.H * float(self.N) ** 2 * self.D
        return f / 2 if c else f


WORKLOADS = {
    "c1": Workload("c1", 1, 2, 512, 64, "BSND", False, 1, dtypes=("fp32",)),
    "c2": Workload("c2", 1, 8, 512, 64, "BSND", False, 2, dtypes=("fp16", "bf16")),
    "c3": Workload("c3", 8, 32, 4096, 128, "BHSD", True, 3),
    "c4": Workload("c4", 2, 40, 8192, 128, "BHSD", True, 4, qk_mult=8.0),
    "c5": Workload("c5", 1, 32, 65536, 128, "BHSD", True, 5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb cannot wrap for finite values or infinities (largest pattern 0xFF800000)
    out = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp32, exact."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 bit patterns (uint16), round to nearest, ties to even (numpy's cast)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def cast_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Stored element bits of ``dtype`` for fp32 values: float32 for fp32, uint16 patterns otherwise."""
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if dtype == "fp16":
        return f32_to_f16_bits(x32)
    raise ValueError("dtype must be fp32, fp16 or bf16")


def to_layout(x_bhsd: np.ndarray, layout: str) -> np.ndarray:
    """Logical [B, H, N, D] array -> packed array in ``layout``."""
    if layout == "BHSD":
        return np.ascontiguousarray(x_bhsd)
    if layout == "BSND":
        return np.ascontiguousarray(x_bhsd.transpose(0, 2, 1, 3))
    raise ValueError("layout must be BHSD or BSND")


def shape_of(B: int, H: int, N: int, D: int, layout: str) -> tuple:
    return (B, H, N, D) if layout == "BHSD" else (B, N, H, D)


def draw_f32(B: int, H: int, N: int, D: int, seed, qk_mult: float = 1.0):
    """The fp32 draws (logical [B, H, N, D]) of Q, K, V for generator seed ``[42, seed]``."""
    rng = np.random.default_rng([42, seed] if np.isscalar(seed) else list(seed))
    shape = (B, H, N, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if qk_mult != 1.0:
        q *= np.float32(qk_mult)
        k *= np.float32(qk_mult)
    return q, k, v


def make(B: int, H: int, N: int, D: int, *, layout: str, dtype: str, seed, qk_mult: float = 1.0):
    """Stored Q, K, V (element bits of ``dtype``, packed in ``layout``) for generator seed ``[42, seed]``."""
    q, k, v = draw_f32(B, H, N, D, seed, qk_mult)
    return tuple(to_layout(cast_bits(t, dtype), layout) for t in (q, k, v))


def make_grad(B: int, H: int, N: int, D: int, *, layout: str, dtype: str, seed):
    """Stored upstream gradient dO (element bits of ``dtype``, packed in ``layout``) for ``[42, seed, 7]``."""
    rng = np.random.default_rng([42] + ([seed] if np.isscalar(seed) else list(seed)) + [7])
    return to_layout(cast_bits(rng.standard_normal((B, H, N, D), dtype=np.float32), dtype), layout)


def varlen_lengths(B: int, lo: int, hi: int, seed) -> np.ndarray:
    """B seeded sequence lengths, uniform in [lo, hi]."""
    rng = np.random.default_rng([4243] + ([seed] if np.isscalar(seed) else list(seed)))
    return rng.integers(lo, hi + 1, size=B).astype(np.int64)


def cu_seqlens(lengths) -> np.ndarray:
    """int32 offsets [0, l0, l0 + l1, ...] of packed sequences."""
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_varlen(lens_q, lens_k, H: int, D: int, *, dtype: str, seed):
    """Stored packed Q [sum(lens_q), H, D] and K, V [sum(lens_k), H, D] for generator ``[42, seed, 11]``."""
    rng = np.random.default_rng([42] + ([seed] if np.isscalar(seed) else list(seed)) + [11])
    tq, tk = int(np.sum(lens_q)), int(np.sum(lens_k))
    q = rng.standard_normal((tq, H, D), dtype=np.float32)
    k = rng.standard_normal((tk, H, D), dtype=np.float32)
    v = rng.standard_normal((tk, H, D), dtype=np.float32)
    return tuple(np.ascontiguousarray(cast_bits(t, dtype)) for t in (q, k, v))


def make_grad_varlen(lens_q, H: int, D: int, *, dtype: str, seed):
    """Stored packed upstream gradient dO [sum(lens_q), H, D] for generator ``[42, seed, 12]``."""
    rng = np.random.default_rng([42] + ([seed] if np.isscalar(seed) else list(seed)) + [12])
    tq = int(np.sum(lens_q))
    return np.ascontiguousarray(cast_bits(rng.standard_normal((tq, H, D), dtype=np.float32), dtype))


def make_workload(w: Workload, dtype: str | None = None):
    """Stored Q, K, V of a named workload (its first dtype unless one is given)."""
    return make(w.B, w.H, w.N, w.D, layout=w.layout, dtype=dtype or w.dtypes[0], seed=w.seed, qk_mult=w.qk_mult)


def sample_rows(B: int, H: int, N: int, count: int, seed, *, edge_tiles: int = 0, tile: int = 128,
                edge_heads: int = 0, heads_subset: int = 0, rows_per_head: int = 0) -> np.ndarray:
    """Seeded (b, h, i) triples, drawn without replacement with ``default_rng([4242, seed])``.

    count:          number of uniformly drawn distinct triples over [B, H, N];
    edge_tiles:     for ``edge_heads`` seeded (b, h) pairs, add every row of the first and the last
                    ``tile``-row tile (``edge_tiles`` = 1 adds both edge tiles);
    heads_subset / rows_per_head: alternatively draw ``heads_subset`` seeded (b, h) pairs and
                    ``rows_per_head`` seeded rows in each, always including rows 0 and N - 1.
    Returns a sorted, duplicate-free int64 array of shape [R, 3].
    """
    rng = np.random.default_rng([4242] + ([seed] if np.isscalar(seed) else list(seed)))
    total = B * H * N
    parts = []
    if count > 0:
        flat = rng.choice(total, size=min(count, total), replace=False)
        parts.append(np.stack(np.unravel_index(flat, (B, H, N)), axis=1))
    if edge_tiles and edge_heads:
        bh = rng.choice(B * H, size=min(edge_heads, B * H), replace=False)
        for x in bh:
            b, h = divmod(int(x), H)
            rows = np.concatenate([np.arange(0, min(tile, N)), np.arange(max(0, N - tile), N)])
            parts.append(np.stack([np.full_like(rows, b), np.full_like(rows, h), rows], axis=1))
    if heads_subset and rows_per_head:
        bh = rng.choice(B * H, size=min(heads_subset, B * H), replace=False)
        for x in bh:
            b, h = divmod(int(x), H)
            rows = rng.choice(N, size=min(rows_per_head, N), replace=False)
            rows = np.unique(np.concatenate([rows, [0, N - 1]]))
            parts.append(np.stack([np.full_like(rows, b), np.full_like(rows, h), rows], axis=1))
    if not parts:
        return np.zeros((0, 3), dtype=np.int64)
    rows = np.unique(np.concatenate(parts).astype(np.int64), axis=0)
    return rows
