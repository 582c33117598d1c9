"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each check takes the implementation under test as callables
    fwd(q, k, v, scale, causal) -> (O, LSE)
    bwd(q, k, v, dO, scale, causal) -> (dQ, dK, dV)
and raises AssertionError on a mismatch. tests/test_oracle.py runs them on the
oracle; tests/test_oracle_mutants.py runs them on copies with planted mistakes
and requires every mutant to fail at least one of them.

Sources of truth used here, none of which is the oracle's own code:
  * closed forms of softmax attention on special inputs (all-equal scores ->
    mean of V; causal row 0 -> V_0; one-hot keys; N = 1; two keys -> logistic);
  * invariants of the definition (rows of P sum to 1; a per-row additive
    constant in the scores leaves O unchanged; linearity in V; permutation
    equivariance; sum_j dK_j = 0; sum_j dV_j = sum_i dO_i; equal keys -> dQ = 0);
  * a library routine: torch's float64 scaled_dot_product_attention, logsumexp
    and autograd on the CPU;
  * central finite differences of the loss sum(O * dO).
"""
from __future__ import annotations

import math

import numpy as np

RNG = np.random.default_rng


def _rand(shape, seed, scale=1.0):
    return RNG(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------------------
def check_all_equal_scores(fwd):
    """Q = 0 makes every score 0: O_i = mean of the visible V rows; LSE_i = ln(#visible keys)."""
    B, H, N, d = 2, 3, 11, 5
    q = np.zeros((B, H, N, d))
    k = _rand((B, H, N, d), 1)
    v = _rand((B, H, N, d), 2)
    O, L = fwd(q, k, v, 0.7, False)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape), atol=1e-13)
    np.testing.assert_allclose(L, np.full((B, H, N), math.log(N)), atol=1e-13)
    O, L = fwd(q, k, v, 0.7, True)
    prefix_mean = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
    np.testing.assert_allclose(O, prefix_mean, atol=1e-13)
    np.testing.assert_allclose(L, np.broadcast_to(np.log(np.arange(1, N + 1)), (B, H, N)), atol=1e-13)


def check_causal_row0(fwd):
    """Under the causal mask query 0 sees only key 0: O_0 = V_0, LSE_0 = scale * q_0 . k_0."""
    B, H, N, d = 2, 2, 9, 6
    q, k, v = _rand((B, H, N, d), 3), _rand((B, H, N, d), 4), _rand((B, H, N, d), 5)
    scale = 0.37
    O, L = fwd(q, k, v, scale, True)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], atol=1e-14)
    np.testing.assert_allclose(L[:, :, 0], scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1), atol=1e-13)


def check_one_hot(fwd):
    """K_j = e_j (N <= d) and q_i = alpha e_pi(i): row i has score s*alpha at key pi(i) and 0
    elsewhere, so O_i = (e^{s alpha} V_pi(i) + sum_{j != pi(i)} V_j) / (e^{s alpha} + N - 1),
    LSE_i = ln(e^{s alpha} + N - 1)."""
    N, d = 6, 8
    k = np.zeros((1, 1, N, d))
    k[0, 0, np.arange(N), np.arange(N)] = 1.0
    pi = np.array([3, 0, 5, 1, 1, 4])
    v = _rand((1, 1, N, d), 6)
    for alpha, s in [(2.0, 0.5), (40.0, 1.0), (1e3, 0.125)]:
        q = np.zeros((1, 1, N, d))
        q[0, 0, np.arange(N), pi] = alpha
        O, L = fwd(q, k, v, s, False)
        big = math.exp(s * alpha) if s * alpha < 700 else None
        for i in range(N):
            rest = v[0, 0].sum(axis=0) - v[0, 0, pi[i]]
            if big is None:
                exp_o, exp_l = v[0, 0, pi[i]], s * alpha
            else:
                exp_o = (big * v[0, 0, pi[i]] + rest) / (big + N - 1)
                exp_l = math.log(big + N - 1)
            np.testing.assert_allclose(O[0, 0, i], exp_o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(L[0, 0, i], exp_l, rtol=1e-13)


def check_single_key_and_two_keys(fwd):
    """N = 1 gives O = V_0 and LSE = scale q.k. With two keys and no mask,
    P_i0 = logistic(scale q_i . (k_0 - k_1))."""
    q, k, v = _rand((1, 2, 1, 4), 7), _rand((1, 2, 1, 4), 8), _rand((1, 2, 1, 4), 9)
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.9, causal)
        np.testing.assert_allclose(O, v, atol=1e-15)
        np.testing.assert_allclose(L, 0.9 * np.sum(q * k, axis=-1), atol=1e-14)
    q, k = _rand((1, 1, 2, 3), 10), _rand((1, 1, 2, 3), 11)
    v = np.zeros((1, 1, 2, 3))
    v[0, 0, 0, 0] = 1.0  # O[:, 0] exposes P_i0
    O, _ = fwd(q, k, v, 1.3, False)
    for i in range(2):
        z = 1.3 * np.dot(q[0, 0, i], k[0, 0, 0] - k[0, 0, 1])
        np.testing.assert_allclose(O[0, 0, i, 0], 1.0 / (1.0 + math.exp(-z)), rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------------------------
def check_rows_sum_to_one(fwd):
    """With V = I (N = d) the output IS P: rows sum to 1, entries are >= 0, and the causal P is
    lower-triangular."""
    N = 7
    q, k = _rand((1, 1, N, N), 12), _rand((1, 1, N, N), 13)
    v = np.eye(N)[None, None]
    for causal in (False, True):
        P, _ = fwd(q, k, v, 0.8, causal)
        np.testing.assert_allclose(P.sum(axis=-1), 1.0, atol=1e-13)
        assert np.all(P >= 0)
        if causal:
            assert np.all(np.triu(P[0, 0], 1) == 0.0)


def check_row_shift(fwd):
    """K -> K + 1 u^T adds scale q_i . u to every score of row i: O unchanged, LSE_i shifted."""
    B, H, N, d = 1, 2, 10, 4
    q, k, v = _rand((B, H, N, d), 14), _rand((B, H, N, d), 15), _rand((B, H, N, d), 16)
    u = _rand((d,), 17)
    for causal in (False, True):
        O1, L1 = fwd(q, k, v, 0.6, causal)
        O2, L2 = fwd(q, k + u, v, 0.6, causal)
        np.testing.assert_allclose(O2, O1, atol=1e-12)
        np.testing.assert_allclose(L2, L1 + 0.6 * np.einsum("bhnd,d->bhn", q, u), atol=1e-12)


def check_v_linearity(fwd):
    """V -> a V + 1 c^T gives O -> a O + 1 c^T, and LSE does not depend on V."""
    q, k, v = _rand((1, 1, 9, 3), 18), _rand((1, 1, 9, 3), 19), _rand((1, 1, 9, 3), 20)
    c = np.array([0.5, -2.0, 3.0])
    for causal in (False, True):
        O1, L1 = fwd(q, k, v, 1.1, causal)
        O2, L2 = fwd(q, k, -1.7 * v + c, 1.1, causal)
        np.testing.assert_allclose(O2, -1.7 * O1 + c, atol=1e-12)
        np.testing.assert_allclose(L2, L1, atol=1e-14)


def check_permutations(fwd):
    """Non-causal: permuting K and V rows together changes nothing; permuting Q rows permutes O and LSE."""
    N = 8
    q, k, v = _rand((1, 1, N, 5), 21), _rand((1, 1, N, 5), 22), _rand((1, 1, N, 5), 23)
    perm = RNG(24).permutation(N)
    O1, L1 = fwd(q, k, v, 0.5, False)
    O2, L2 = fwd(q, k[:, :, perm], v[:, :, perm], 0.5, False)
    np.testing.assert_allclose(O2, O1, atol=1e-13)
    np.testing.assert_allclose(L2, L1, atol=1e-13)
    O3, L3 = fwd(q[:, :, perm], k, v, 0.5, False)
    np.testing.assert_allclose(O3, O1[:, :, perm], atol=1e-13)
    np.testing.assert_allclose(L3, L1[:, :, perm], atol=1e-13)


# ---------------------------------------------------------------------------------------------
# library routine (special case) and brute force
# ---------------------------------------------------------------------------------------------
def check_torch_sdpa(fwd, bwd):
    """torch's float64 CPU scaled_dot_product_attention (is_causal masks j > i for square inputs),
    logsumexp over the masked scaled scores, and autograd gradients of sum(O * dO)."""
    import torch

    B, H, N, d = 2, 3, 13, 6
    for causal in (False, True):
        for scale in (0.25, 1.0 / math.sqrt(d), 1.9):
            q, k, v, do = (_rand((B, H, N, d), 30 + i) for i in range(4))
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            tO = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
            s = scale * (tq.detach() @ tk.detach().transpose(-1, -2))
            if causal:
                s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
            tL = torch.logsumexp(s, dim=-1)
            (tO * torch.tensor(do)).sum().backward()
            O, L = fwd(q, k, v, scale, causal)
            np.testing.assert_allclose(O, tO.detach().numpy(), atol=1e-12)
            np.testing.assert_allclose(L, tL.numpy(), atol=1e-12)
            dQ, dK, dV = bwd(q, k, v, do, scale, causal)[:3]
            np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-11)
            np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-11)
            np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-11)


def check_brute_force(fwd, bwd):
    """Pure-Python loops (math.exp, math.fsum) on N <= 8, d <= 4."""
    from oracle.brute import brute_bwd, brute_fwd

    for (B, H, N, d), seed in [((1, 1, 1, 1), 40), ((1, 2, 5, 3), 41), ((2, 1, 8, 4), 42), ((1, 1, 7, 2), 43)]:
        q, k, v, do = (_rand((B, H, N, d), seed + 10 * i) for i in range(4))
        for causal in (False, True):
            for scale in (0.3, 1.0, 2.5):
                O, L = fwd(q, k, v, scale, causal)
                Ob, Lb = brute_fwd(q, k, v, scale, causal)
                np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
                np.testing.assert_allclose(L, np.array(Lb), atol=1e-12)
                got = bwd(q, k, v, do, scale, causal)[:3]
                exp = brute_bwd(q, k, v, do, scale, causal)
                for g, e in zip(got, exp):
                    np.testing.assert_allclose(g, np.array(e), atol=1e-11)


def check_finite_differences(fwd, bwd):
    """Central differences of L(q, k, v) = sum(O * dO) (h = 1e-6), every input element."""
    B, H, N, d = 1, 1, 5, 3
    h = 1e-6
    for causal in (False, True):
        q, k, v, do = (_rand((B, H, N, d), 50 + i + 7 * causal) for i in range(4))
        scale = 0.8
        grads = bwd(q, k, v, do, scale, causal)[:3]
        base = [q, k, v]
        for which in range(3):
            num = np.zeros_like(base[which])
            for idx in np.ndindex(base[which].shape):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += h
                minus[which][idx] -= h
                lp = np.sum(fwd(*plus, scale, causal)[0] * do)
                lm = np.sum(fwd(*minus, scale, causal)[0] * do)
                num[idx] = (lp - lm) / (2 * h)
            np.testing.assert_allclose(grads[which], num, rtol=1e-6, atol=1e-8)


def check_backward_invariants(fwd, bwd):
    """sum_j dK_j = 0 (rows of dS sum to 0), sum_j dV_j = sum_i dO_i (rows of P sum to 1),
    D = rowsum(dO * O), and equal key rows give dQ = 0."""
    B, H, N, d = 2, 2, 12, 5
    q, k, v, do = (_rand((B, H, N, d), 60 + i) for i in range(4))
    for causal in (False, True):
        res = bwd(q, k, v, do, 0.45, causal)
        dQ, dK, dV = res[:3]
        np.testing.assert_allclose(dK.sum(axis=2), 0.0, atol=1e-12)
        np.testing.assert_allclose(dV.sum(axis=2), do.sum(axis=2), atol=1e-12)
        if len(res) > 3:
            O, _ = fwd(q, k, v, 0.45, causal)
            np.testing.assert_allclose(res[3], np.sum(do * O, axis=-1), atol=1e-12)
        k_eq = np.broadcast_to(k[:, :, :1], k.shape).copy()
        dQ0 = bwd(q, k_eq, v, do, 0.45, causal)[0]
        np.testing.assert_allclose(dQ0, 0.0, atol=1e-12)


FWD_PINS = [check_all_equal_scores, check_causal_row0, check_one_hot, check_single_key_and_two_keys,
            check_rows_sum_to_one, check_row_shift, check_v_linearity, check_permutations]
FWD_BWD_PINS = [check_torch_sdpa, check_brute_force, check_finite_differences, check_backward_invariants]
