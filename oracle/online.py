"""The blocked online-softmax recurrence, written step by step (test infrastructure).

The pages describe the fused forward as: load one query block, then walk the
key/value blocks in turn, keeping for every query row a running maximum and a
running sum of exponentials, and, whenever a new block raises the maximum,
rescaling what was accumulated so far (52jiny.com explainer, "key ideas"
parts 1 and 2; codechina.net article, sections 4.1 and 4.2, which give the
per-block statistics m = max(row), a = exp(row - m), l = sum(a) but leave the
merge of blocks unstated). The merge used here is the one that makes the
result equal to the plain softmax:

    m_new = max(m_old, max_j s_j)
    l_new = exp(m_old - m_new) * l_old + sum_j exp(s_j - m_new)
    acc_new = exp(m_old - m_new) * acc_old + sum_j exp(s_j - m_new) * v_j

and at the end O = acc / l, LSE = m + ln(l). A fully masked block leaves the
state unchanged (its exponentials are zero; the guard keeps exp(-inf - -inf)
from arising). This module exists so a test can show, for every block size,
that the recurrence reproduces attention.attn_fwd; the oracle itself is the
plain definition.
"""
from __future__ import annotations

import numpy as np


def online_fwd(q, k, v, scale: float, causal: bool, block_q: int, block_k: int):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, N, block_q):
                rows = np.arange(i0, min(N, i0 + block_q))
                m = np.full(len(rows), -np.inf)
                l = np.zeros(len(rows))
                acc = np.zeros((len(rows), d))
                for j0 in range(0, N, block_k):
                    cols = np.arange(j0, min(N, j0 + block_k))
                    s = scale * (q[b, h, rows] @ k[b, h, cols].T)
                    if causal:
                        s = np.where(cols[None, :] > rows[:, None], -np.inf, s)
                    m_new = np.maximum(m, np.max(s, axis=1))
                    safe = np.where(np.isneginf(m_new), 0.0, m_new)   # rows with nothing seen yet
                    alpha = np.exp(m - safe)
                    p = np.exp(s - safe[:, None])
                    l = alpha * l + np.sum(p, axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, cols]
                    m = m_new
                O[b, h, rows] = acc / l[:, None]
                LSE[b, h, rows] = m + np.log(l)
    return O, LSE
