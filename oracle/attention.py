"""Plain float64 attention: the definition the fused method must reproduce exactly.

Sources (cited by page title and section):
  * codechina.net CUDA/FlashAttention article, section 3 ("the attention
    bottleneck from CUDA's point of view"): Q, K, V are N x d; S = Q K^T;
    P = softmax(S); O = P V.
  * 52jiny.com FlashAttention explainer, section "why standard attention is
    IO-bound": the op order is Q K^T, scaling, mask, softmax, (dropout), times V.
  * 52jiny.com, "key ideas" part 2 (online softmax): the tiled method yields
    attention mathematically equal to the plain softmax, differing only by
    floating-point ordering. That is why this plain definition is the oracle.
  * codechina.net section 4.2: per-row statistics m = max(row), l = sum of
    exp(row - m). The saved statistic is their natural-log combination
    LSE = m + ln(l) ("only the output and a few normalisation statistics are
    written back", 52jiny.com "key ideas" part 3).
  * 52jiny.com "key ideas" part 4: the backward recomputes from O and the saved
    softmax statistics. The pages print no gradient formulas; the ones below
    are the chain rule through the row softmax (Jacobian diag(p) - p p^T).

Readings where the pages are silent: the scale is a caller argument; a causal
mask removes key j from query i when j > i (square, top-left aligned) by
setting the score to -inf; there is no dropout; inputs are the exact stored
values (fp32, or bf16 widened), computed on in float64.

Parity status: pinned (tests/test_oracle.py: brute force, closed forms,
invariants, torch float64 SDPA/autograd, finite differences).
"""
from __future__ import annotations

import numpy as np

_ROW_CHUNK = 1024  # rows of S materialised at a time (memory cap only; rows are independent)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def softmax_rows(S: np.ndarray):
    """Row softmax of a score block with -inf entries allowed.

    Returns (P, m, l, lse): m = row max, l = sum_j exp(S_j - m), P = exp(S - m)/l,
    lse = m + ln(l). Max subtraction for stability as the yunthe.com page's
    fusion section does before exponentiating; it changes nothing in exact
    arithmetic."""
    m = np.max(S, axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = np.sum(E, axis=-1, keepdims=True)
    P = E / l
    lse = (m + np.log(l))[..., 0]
    return P, m[..., 0], l[..., 0], lse


def _scores(q_rows, k, scale, causal, row_ids):
    """S = scale * Q K^T for the selected query rows, then the causal mask."""
    S = scale * (q_rows @ k.T)
    if causal:
        cols = np.arange(k.shape[0])
        S = np.where(cols[None, :] > np.asarray(row_ids)[:, None], -np.inf, S)
    return S


def attn_fwd(q, k, v, scale: float, causal: bool):
    """Forward attention for [B, H, N, d] inputs -> (O [B,H,N,d], LSE [B,H,N]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, d = q.shape
    O = np.empty((B, H, N, d))
    LSE = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, _ROW_CHUNK):
                rows = np.arange(r0, min(N, r0 + _ROW_CHUNK))
                S = _scores(q[b, h, rows], k[b, h], scale, causal, rows)
                P, _, _, lse = softmax_rows(S)
                O[b, h, rows] = P @ v[b, h]
                LSE[b, h, rows] = lse
    return O, LSE


def attn_fwd_kv(q, k, v, scale: float, causal: bool):
    """Attention of Nq queries [B, H, Nq, d] against Nk >= Nq keys and values [B, H, Nk, d]
    (decoding new positions against a key/value history) -> (O [B,H,Nq,d], LSE [B,H,Nq]).

    Reading (the pages define only the square case): the queries are the last Nq positions of
    the key sequence, so with the causal mask query i, at position Nk - Nq + i, sees keys
    j <= Nk - Nq + i. Otherwise it is the same definition as attn_fwd: explicit scaled scores,
    mask, row softmax, P V and LSE = m + ln l."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.empty((B, H, Nq, d))
    LSE = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, _ROW_CHUNK):
                rows = np.arange(r0, min(Nq, r0 + _ROW_CHUNK))
                S = _scores(q[b, h, rows], k[b, h], scale, causal, rows + (Nk - Nq))
                P, _, _, lse = softmax_rows(S)
                O[b, h, rows] = P @ v[b, h]
                LSE[b, h, rows] = lse
    return O, LSE


def attn_fwd_rows(q, k, v, scale: float, causal: bool, b: int, h: int, rows):
    """The same definition restricted to some query rows of one (b, h):
    returns (O_rows [len(rows), d], LSE_rows [len(rows)]). Each row of the plain
    definition depends only on its own query, so this is a sample of attn_fwd."""
    rows = np.asarray(rows, dtype=np.int64)
    qh = _f64(q[b, h, rows])
    kh = _f64(k[b, h])
    vh = _f64(v[b, h])
    S = _scores(qh, kh, scale, causal, rows)
    P, _, _, lse = softmax_rows(S)
    return P @ vh, lse


def attn_bwd_rows(q, k, v, do, scale: float, causal: bool, b: int, h: int, rows):
    """dQ of the backward below restricted to some query rows of one (b, h): returns
    (dQ_rows [len(rows), d], D_rows). Row i of dQ = scale * sum_j dS_ij K_j needs only row i's
    probabilities, dP_ij = dO_i . V_j and D_i = sum_j P_ij dP_ij, all formed from its own query
    and gradient row, so this is a sample of attn_bwd's dQ."""
    rows = np.asarray(rows, dtype=np.int64)
    kh, vh = _f64(k[b, h]), _f64(v[b, h])
    S = _scores(_f64(q[b, h, rows]), kh, scale, causal, rows)
    P, _, _, _ = softmax_rows(S)
    dP = _f64(do[b, h, rows]) @ vh.T
    Dr = np.sum(P * dP, axis=1)
    dS = P * (dP - Dr[:, None])
    return scale * (dS @ kh), Dr


def attn_bwd_keys(q, k, v, do, scale: float, causal: bool, b: int, h: int, keys):
    """dK and dV of the backward below restricted to some key rows of one (b, h): returns
    (dK_keys, dV_keys), each [len(keys), d]. Column j of P and dS involves every query row that
    sees key j, and each such row's softmax needs its whole row of scores, so every such row is
    formed in full (in chunks) and only the selected columns are kept:
    dV_j = sum_i P_ij dO_i, dK_j = scale * sum_i dS_ij Q_i. Under the causal mask only rows
    i >= min(keys) see any selected key, so the cost falls with the keys' position."""
    keys = np.asarray(keys, dtype=np.int64)
    qh, kh, vh, doh = _f64(q[b, h]), _f64(k[b, h]), _f64(v[b, h]), _f64(do[b, h])
    N, d = qh.shape
    dK = np.zeros((len(keys), d))
    dV = np.zeros((len(keys), d))
    r_first = int(keys.min()) if causal else 0
    for r0 in range(r_first, N, _ROW_CHUNK):
        rows = np.arange(r0, min(N, r0 + _ROW_CHUNK))
        S = _scores(qh[rows], kh, scale, causal, rows)
        P, _, _, _ = softmax_rows(S)
        dP = doh[rows] @ vh.T
        Dr = np.sum(P * dP, axis=1)
        Pk = P[:, keys]
        dSk = Pk * (dP[:, keys] - Dr[:, None])
        dV += Pk.T @ doh[rows]
        dK += scale * (dSk.T @ qh[rows])
    return dK, dV


def attn_bwd(q, k, v, do, scale: float, causal: bool):
    """Analytic backward of O = softmax(scale*Q K^T + mask) V for the loss sum(O * dO).

    Per (b, h):  dV = P^T dO;  dP = dO V^T;  D_i = sum_j P_ij dP_ij (equal to
    sum_c dO_ic O_ic);  dS = P * (dP - D 1^T);  dQ = scale * dS K;
    dK = scale * dS^T Q. Masked entries have P = 0, hence dS = 0 there.
    Returns (dQ, dK, dV, D) in float64."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, H, N, d = q.shape
    dQ = np.empty_like(q)
    dK = np.empty_like(k)
    dV = np.empty_like(v)
    D = np.empty((B, H, N))
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            S = _scores(q[b, h], k[b, h], scale, causal, rows)
            P, _, _, _ = softmax_rows(S)
            dO = do[b, h]
            dV[b, h] = P.T @ dO
            dP = dO @ v[b, h].T
            Dh = np.sum(P * dP, axis=1)
            dS = P * (dP - Dh[:, None])
            dQ[b, h] = scale * (dS @ k[b, h])
            dK[b, h] = scale * (dS.T @ q[b, h])
            D[b, h] = Dh
    return dQ, dK, dV, D
