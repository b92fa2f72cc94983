"""Brute-force attention in numpy fp64 with the full N x N score matrix, for tiny inputs only.

Independent of the oracle: explicit score matrix, explicit boolean mask, row softmax, matrix product.
Definition: Softmax(Q K^T / sqrt(d)) V with a caller-given scale (page ai6s.net/6a0d42d8..., section
"Attention 的显存黑洞"); causal mask = entries strictly above the diagonal hidden (page ai6s.net/
6a0d3bfb..., causal-mask section, torch.triu(..., diagonal=1)).
"""
import numpy as np


def attention_bhsd(q, k, v, *, causal, scale):
    """q, k, v float64 [B, H, N, D] -> (O [B, H, N, D], lse [B, H, N], P [B, H, N, N])."""
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    N = q.shape[2]
    if causal:
        hidden = np.triu(np.ones((N, N), dtype=bool), k=1)
        s = np.where(hidden, -np.inf, s)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    p = e / e.sum(axis=-1, keepdims=True)
    lse = np.log(e.sum(axis=-1)) + mx[..., 0]
    return p @ v, lse, p
