"""Pure-Python brute force for tiny shapes (N <= 8, d <= 4 in the tests).

A second, loop-level statement of the same definition (codechina.net article,
section 3: S = Q K^T, P = softmax(S), O = P V; 52jiny.com explainer, "why
standard attention is IO-bound": scale, mask, softmax, then V), written with
math.exp and math.fsum on Python floats and nested lists, so it shares no
NumPy code path with attention.py. The backward writes the softmax Jacobian
element by element: dL/dS_ij = P_ij * sum_c dO_ic (V_jc - O_ic).
"""
from __future__ import annotations

import math


def _tolist4(x):
    return [[[[float(e) for e in row] for row in mat] for mat in head] for head in x]


def brute_fwd(q, k, v, scale, causal):
    """Returns (O, LSE) as nested lists [B][H][N][d] and [B][H][N]."""
    q, k, v = _tolist4(q), _tolist4(k), _tolist4(v)
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    O = [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if not (causal and j > i)]
                s = {j: scale * math.fsum(q[b][h][i][c] * k[b][h][j][c] for c in range(d)) for j in keys}
                top = max(s.values())
                lse = top + math.log(math.fsum(math.exp(s[j] - top) for j in keys))
                p = {j: math.exp(s[j] - lse) for j in keys}
                for c in range(d):
                    O[b][h][i][c] = math.fsum(p[j] * v[b][h][j][c] for j in keys)
                L[b][h][i] = lse
    return O, L


def brute_bwd(q, k, v, do, scale, causal):
    """Returns (dQ, dK, dV) as nested lists, by the elementwise chain rule."""
    q, k, v, do = _tolist4(q), _tolist4(k), _tolist4(v), _tolist4(do)
    O, L = brute_fwd(q, k, v, scale, causal)
    B, H, N, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    z = lambda: [[[[0.0] * d for _ in range(N)] for _ in range(H)] for _ in range(B)]
    dQ, dK, dV = z(), z(), z()
    for b in range(B):
        for h in range(H):
            P = [[0.0] * N for _ in range(N)]
            for i in range(N):
                for j in range(N):
                    if causal and j > i:
                        continue
                    sij = scale * math.fsum(q[b][h][i][c] * k[b][h][j][c] for c in range(d))
                    P[i][j] = math.exp(sij - L[b][h][i])
            G = [[0.0] * N for _ in range(N)]   # dL/dS
            for i in range(N):
                for j in range(N):
                    G[i][j] = P[i][j] * math.fsum(do[b][h][i][c] * (v[b][h][j][c] - O[b][h][i][c]) for c in range(d))
            for i in range(N):
                for c in range(d):
                    dQ[b][h][i][c] = scale * math.fsum(G[i][j] * k[b][h][j][c] for j in range(N))
            for j in range(N):
                for c in range(d):
                    dK[b][h][j][c] = scale * math.fsum(G[i][j] * q[b][h][i][c] for i in range(N))
                    dV[b][h][j][c] = math.fsum(P[i][j] * do[b][h][i][c] for i in range(N))
    return dQ, dK, dV
