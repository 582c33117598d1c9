"""Attention under a general visibility mask: padded variable-length batches, key/value caches of
different lengths per sequence, and block-sparse tile maps (TEST INFRASTRUCTURE, float64).

Sources (cited by page title and section):
  * 52jiny.com FlashAttention explainer, "why standard attention is IO-bound": the mask is one
    step of the operator chain, applied to the scaled scores before the softmax; its
    deployment advice lists the mask's form among what decides the speed-up.
  * yunthe.com "FlashAttention explained", section 5 (applications and directions), and the
    codechina.net CUDA/FlashAttention article, section 7.2 (other variants): sparse attention,
    i.e. skipping parts of the score matrix by a sparsity pattern.
  * The rest is the same plain definition as attention.py: S = scale * Q K^T, masked entries
    set to -inf, row softmax, O = P V, LSE = ln sum_j exp(S_ij), and the chain-rule backward.

Readings (the pages give no mask format):
  * a mask is a boolean "visible" array [B, H, Nq, Nk]; a masked score is -inf (probability
    exactly zero);
  * padded batch: sequence b occupies rows [0, L_b) of both Q and K/V; query i sees key j iff
    i < L_b and j < L_b (and j <= i under the causal mask);
  * key/value cache of length L_b per sequence with Nq new queries that are its last Nq
    positions: query i sees key j iff j < L_b (and j <= i + L_b - Nq under the causal mask);
  * block-sparse: a byte per (query block, key block) of BLOCK x BLOCK scores; zero removes the
    whole block; it is combined (logical and) with the other conditions;
  * a row that sees no key has an empty softmax: O_i = 0 and LSE_i = -inf, and it receives and
    passes on no gradient. (Under the plain definition it would be 0/0.)

Parity status: pinned (tests/test_oracle_masked.py: torch float64 SDPA with the same boolean
mask, truncation of padded sequences, independence from padding contents, block-diagonal
sparsity as independent attentions, finite differences, brute force).
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_rows

BLOCK = 128  # rows and columns of the score matrix per block-sparse map entry


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def padded_batch_visible(B, H, N, causal, seqlens=None, block_mask=None, block=BLOCK, rows=None):
    """visible[b, h, i, j] for a padded batch of square problems (see the module readings).
    With `rows`, only those query rows i (visible[b, h, r, j] for the r-th entry of rows); every
    row's visibility depends on its own index alone, so this is a slice of the full array."""
    i = (np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64))[:, None]
    j = np.arange(N)[None, :]
    vis = np.ones((B, H, i.shape[0], N), dtype=bool)
    if causal:
        vis &= (j <= i)[None, None]
    if seqlens is not None:
        L = np.asarray(seqlens).reshape(B, 1, 1, 1)
        vis &= (i[None, None] < L) & (j[None, None] < L)
    if block_mask is not None:
        bm = np.asarray(block_mask) != 0  # [B, H, ceil(N/block), ceil(N/block)]
        vis &= bm[:, :, i // block, j // block]
    return vis


def kv_cache_visible(B, H, Nq, Nk, causal, seqlens_k=None):
    """visible[b, h, i, j] for Nq queries that are the last Nq positions of a cache of L_b <= Nk keys
    (L_b = Nk when seqlens_k is None)."""
    L = np.full(B, Nk) if seqlens_k is None else np.asarray(seqlens_k)
    L = L.reshape(B, 1, 1, 1)
    i = np.arange(Nq)[None, None, :, None]
    j = np.arange(Nk)[None, None, None, :]
    vis = j < L
    if causal:
        vis = vis & (j <= i + L - Nq)
    return np.broadcast_to(vis, (B, H, Nq, Nk)).copy()


def _scores(qh, kh, scale, vis):
    return np.where(vis, scale * (qh @ kh.T), -np.inf)


def attn_fwd_masked(q, k, v, scale: float, visible):
    """(O [B,H,Nq,d], LSE [B,H,Nq]) under a boolean visible [B,H,Nq,Nk]; empty rows give 0, -inf."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    O = np.zeros((B, H, Nq, d))
    LSE = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            rows = np.flatnonzero(visible[b, h].any(axis=1))
            if rows.size == 0:
                continue
            S = _scores(q[b, h, rows], k[b, h], scale, visible[b, h, rows])
            P, _, _, lse = softmax_rows(S)
            O[b, h, rows] = P @ v[b, h]
            LSE[b, h, rows] = lse
    return O, LSE


def attn_bwd_masked(q, k, v, do, scale: float, visible):
    """Gradients of sum(O * dO) for attn_fwd_masked: (dQ, dK, dV, D) in float64.

    The same chain rule as attention.attn_bwd on the rows that see a key; an empty row's output
    is the constant 0, so it contributes nothing and its dQ row and D are 0."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, Nq, d = q.shape
    dQ = np.zeros_like(q)
    dK = np.zeros_like(k)
    dV = np.zeros_like(v)
    D = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            rows = np.flatnonzero(visible[b, h].any(axis=1))
            if rows.size == 0:
                continue
            S = _scores(q[b, h, rows], k[b, h], scale, visible[b, h, rows])
            P, _, _, _ = softmax_rows(S)
            dO = do[b, h, rows]
            dV[b, h] = P.T @ dO
            dP = dO @ v[b, h].T
            Dh = np.sum(P * dP, axis=1)
            dS = P * (dP - Dh[:, None])
            dQ[b, h, rows] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h, rows])
            D[b, h, rows] = Dh
    return dQ, dK, dV, D
