"""Attention dropout: the keep mask and attention with it (TEST INFRASTRUCTURE, float64).

Sources (cited by page title and section):
  * 52jiny.com FlashAttention explainer, "why standard attention is IO-bound": dropout is the
    step between the softmax and the product with V.
  * The generator is Philox4x32-10, the counter-based generator of J. K. Salmon, M. A. Moraes,
    R. O. Dror and D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC 2011): a
    128-bit counter and a 64-bit key go through ten rounds, each two 32x32 -> 64-bit products
    with the multipliers 0xD2511F53 and 0xCD9E8D57 plus xors with the key, which is advanced by
    the Weyl increments 0x9E3779B9 and 0xBB67AE85 between rounds. Written here from that
    definition; pinned to the authors' published known-answer vectors.

Readings (the pages give no random-number contract; this is the one the library implements):
  * element (b, h, i, j) of the score matrix belongs to the 32-key block J = j // 32 and to the
    half t = (j // 4) % 2 of that block; Philox4x32-10 with counter (i, J, b*H + h, t) and key
    (seed mod 2^32, seed div 2^32) gives four 32-bit words w_0..w_3; the element's random byte is
    byte (j % 4) of word (j % 32) // 8 (byte 0 = the least significant);
  * the element is kept iff that byte < T, T = round(256 * (1 - p)); the keep probability is
    therefore T / 256 (p is quantised to a multiple of 1/256), and kept probabilities are scaled
    by 256 / T so that the output is unbiased;
  * O = ((P * Z) * 256 / T) V with P the softmax of the masked scores and Z the keep mask; LSE is
    that of P (dropout does not change the normaliser). The backward is the chain rule through
    the same expression with the same Z.
The keep mask is an input of the attention functions below; keep_mask() builds it.

Parity status: pinned (tests/test_oracle_dropout.py: published Philox known-answer vectors, a
pure-Python scalar statement of the element -> (counter, word, byte) map, keep-rate and byte
uniformity statistics, p = 0 reduces to attention without dropout, torch float64 autograd with
the same mask, finite differences).
"""
from __future__ import annotations

import numpy as np

from .attention import softmax_rows

PHILOX_M0, PHILOX_M1 = 0xD2511F53, 0xCD9E8D57
PHILOX_W0, PHILOX_W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32_10(ctr, key):
    """Philox4x32-10 on arrays: ctr uint64 [..., 4] (values < 2^32), key (k0, k1) -> uint64 [..., 4]."""
    c = [np.asarray(ctr[..., i], dtype=np.uint64) & np.uint64(MASK32) for i in range(4)]
    k0, k1 = np.uint64(key[0] & MASK32), np.uint64(key[1] & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        p0 = c[0] * m0  # < 2^64: exact in uint64
        p1 = c[2] * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + np.uint64(PHILOX_W0)) & np.uint64(MASK32)
        k1 = (k1 + np.uint64(PHILOX_W1)) & np.uint64(MASK32)
    return np.stack(c, axis=-1)


def keep_threshold(p: float) -> int:
    """T = round(256 (1 - p)): an element is kept iff its random byte is below T."""
    return int(np.floor(256.0 * (1.0 - p) + 0.5))


def random_bytes(B, H, Nq, Nk, seed: int, heads=None):
    """uint8 [B, H, Nq, Nk]: the random byte of every score element under the contract above.
    With `heads` (flattened indices b * H + h), only those heads: uint8 [len(heads), Nq, Nk]."""
    key = (seed & MASK32, (seed >> 32) & MASK32)
    nJ = -(-Nk // 32)
    hs = np.arange(B * H) if heads is None else np.asarray(heads)
    bh = hs.astype(np.uint64).reshape(-1, 1, 1, 1)
    i = np.arange(Nq, dtype=np.uint64).reshape(1, Nq, 1, 1)
    J = np.arange(nJ, dtype=np.uint64).reshape(1, 1, nJ, 1)
    t = np.arange(2, dtype=np.uint64).reshape(1, 1, 1, 2)
    ctr = np.stack(np.broadcast_arrays(i, J, bh, t), axis=-1)  # [BH, Nq, nJ, 2, 4]
    words = philox4x32_10(ctr, key)                            # [BH, Nq, nJ, 2, 4]
    j = np.arange(Nk)
    jj = j % 32
    w = words[:, :, j // 32, (j // 4) % 2, jj // 8]            # [BH, Nq, Nk]
    byte = (w >> (8 * (jj % 4)).astype(np.uint64)) & np.uint64(0xFF)
    if heads is not None:
        return byte.astype(np.uint8)
    return byte.astype(np.uint8).reshape(B, H, Nq, Nk)


def keep_mask(B, H, Nq, Nk, p: float, seed: int):
    """bool [B, H, Nq, Nk]: True where the element survives dropout with probability p."""
    return random_bytes(B, H, Nq, Nk, seed) < keep_threshold(p)


def attn_fwd_dropout(q, k, v, scale: float, visible, keep, p: float):
    """(O, LSE) with dropout: O = ((P * keep) * 256 / T) V, LSE of the undropped P.
    Rows that see no key: O = 0, LSE = -inf."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, Nq, d = q.shape
    inv_keep = 256.0 / keep_threshold(p)
    O = np.zeros((B, H, Nq, d))
    LSE = np.full((B, H, Nq), -np.inf)
    for b in range(B):
        for h in range(H):
            rows = np.flatnonzero(visible[b, h].any(axis=1))
            if rows.size == 0:
                continue
            S = np.where(visible[b, h, rows], scale * (q[b, h, rows] @ k[b, h].T), -np.inf)
            P, _, _, lse = softmax_rows(S)
            O[b, h, rows] = (P * keep[b, h, rows] * inv_keep) @ v[b, h]
            LSE[b, h, rows] = lse
    return O, LSE


def attn_bwd_dropout(q, k, v, do, scale: float, visible, keep, p: float):
    """Gradients of sum(O * dO) for attn_fwd_dropout with the same keep mask: (dQ, dK, dV, D).

    With Pd = P * keep * 256 / T (the weights applied to V): dV = Pd^T dO; the gradient reaching
    P is dP = (dO V^T) * keep * 256 / T; D_i = sum_j P_ij dP_ij (= dO_i . O_i);
    dS = P * (dP - D); dQ = scale dS K; dK = scale dS^T Q."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H, Nq, d = q.shape
    inv_keep = 256.0 / keep_threshold(p)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    D = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            rows = np.flatnonzero(visible[b, h].any(axis=1))
            if rows.size == 0:
                continue
            S = np.where(visible[b, h, rows], scale * (q[b, h, rows] @ k[b, h].T), -np.inf)
            P, _, _, _ = softmax_rows(S)
            Z = keep[b, h, rows] * inv_keep
            dO = do[b, h, rows]
            dV[b, h] = (P * Z).T @ dO
            dP = (dO @ v[b, h].T) * Z
            Dh = np.sum(P * dP, axis=1)
            dS = P * (dP - Dh[:, None])
            dQ[b, h, rows] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h, rows])
            D[b, h, rows] = Dh
    return dQ, dK, dV, D
