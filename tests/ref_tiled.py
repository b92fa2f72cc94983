"""fp64 model of the tiled online-softmax forward: the executable statement of the loop the kernel runs.

Follows page "FlashAttention：让长文本推理不再"卡显存"" (ai6s.net/6a0d42d8...): section "1. 分块计算（Tiling）"
(Q tiles outer, K/V tiles inner, only inputs and outputs in device memory) and section "2. 在线归一化
（Online Softmax）" (m_new = max(m_old, m_block); l_new = l_old e^(m_old - m_new) + l_block e^(m_block - m_new)).
The page leaves the accumulator update implicit; the reading taken is the only one under which the
tiled result equals the global softmax, as that section claims: the running output is multiplied by
the same factor e^(m_old - m_new) as l, and divided by l at the end.

Causal tile skipping follows page hwcomputing.csdn.net/6a0d4681..., section "Causal Mask的实现差异",
mode 2, with the skip rule made exact: K tile j of Q tile t is visited iff j*bn <= (t+1)*bm - 1, and
keys above the diagonal inside a visited tile are masked.

``tau`` models a deferred rescale: the reference maximum only moves when the new block maximum exceeds
it by more than ``tau`` (in natural-log units).  Any reference value gives the same quotient O = acc/l
in exact arithmetic; tau = 0 is the pages' update.
"""
import numpy as np


def tiled_attention(q, k, v, *, causal, scale, bm, bn, tau=0.0, count_tiles=None):
    """q, k, v: float64 [B, H, N, D].  Returns O [B, H, N, D] and lse [B, H, N] (natural log)."""
    B, H, N, D = q.shape
    o = np.zeros_like(q)
    lse = np.zeros((B, H, N))
    visited = 0
    for b in range(B):
        for h in range(H):
            for t in range(-(-N // bm)):
                r0, r1 = t * bm, min(N, (t + 1) * bm)
                rows = np.arange(r0, r1)
                m = np.full(r1 - r0, -np.inf)
                l = np.zeros(r1 - r0)
                acc = np.zeros((r1 - r0, D))
                for j in range(-(-N // bn)):
                    c0, c1 = j * bn, min(N, (j + 1) * bn)
                    if causal and c0 > (t + 1) * bm - 1:
                        break
                    visited += 1
                    s = scale * (q[b, h, r0:r1] @ k[b, h, c0:c1].T)
                    if causal:
                        cols = np.arange(c0, c1)
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_blk = s.max(axis=1)
                    m_cand = np.maximum(m, m_blk)
                    move = m_cand > m + tau
                    m_new = np.where(move, m_cand, m)
                    finite = np.isfinite(m_new)
                    ref = np.where(finite, m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
                    p = np.exp(s - ref[:, None])
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, c0:c1]
                    m = m_new
                o[b, h, r0:r1] = acc / l[:, None]
                lse[b, h, r0:r1] = m + np.log(l)
    if count_tiles is not None:
        count_tiles.append(visited)
    return o, lse


def causal_tiles_per_head(N, bm, bn):
    """Closed form of the number of (Q tile, K tile) pairs visited per head under causal skipping."""
    T = -(-N // bm)
    KT = -(-N // bn)
    return sum(min(KT, ((t + 1) * bm - 1) // bn + 1) for t in range(T))
