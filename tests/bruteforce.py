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


def attention_general(q, k, v, *, causal, scale, q_offset=0, kv_start=0, kv_len=None, window=-1):
    """q float64 [B, H, Nq, D], k and v [B, H, Nk, D] -> (O [B, H, Nq, D], lse [B, H, Nq]).

    Explicit visibility matrix from sequence positions: query row i at q_offset + i, key row j at j;
    visible iff kv_start <= j < kv_start + kv_len, j <= q_offset + i when causal, and
    j >= q_offset + i - window when window >= 0.  Rows with no visible key: O = 0, lse = -inf.
    """
    Nq, Nk = q.shape[2], k.shape[2]
    if kv_len is None:
        kv_len = Nk - kv_start
    qpos = q_offset + np.arange(Nq)[:, None]
    kpos = np.arange(Nk)[None, :]
    vis = (kpos >= kv_start) & (kpos < kv_start + kv_len) & np.ones((Nq, 1), dtype=bool)
    if causal:
        vis = vis & (kpos <= qpos)
    if window >= 0:
        vis = vis & (kpos >= qpos - window)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)  # [Nq]
    mx = np.where(any_vis[:, None], s.max(axis=-1, keepdims=True), 0.0)
    e = np.where(vis, np.exp(s - mx), 0.0)
    tot = e.sum(axis=-1)
    p = e / np.where(tot > 0, tot, 1.0)[..., None]
    lse = np.where(any_vis, np.log(np.where(tot > 0, tot, 1.0)) + mx[..., 0], -np.inf)
    return p @ v, lse
