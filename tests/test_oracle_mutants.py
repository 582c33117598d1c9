"""Pin strength: copies of the oracle with one planted mistake each must fail at least one pin.

The mutants mirror the oracle's steps (scores, mask, row softmax, P.V, LSE; the analytic
backward) with a single plausible error: a dropped term, a wrong sign or index, a transposed
operand, the wrong reduction axis, the yunthe.com page's epsilon in the softmax denominator, or
an online recurrence without the rescale. Mistakes are planted only here, on the CPU.
"""
import numpy as np
import pytest

from oracle import attn_fwd
from tests import oracle_pins as pins


def _fwd_factory(mut):
    def fwd(q, k, v, scale, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        N = q.shape[2]
        sc = {"no_scale": 1.0, "scale_squared": scale * scale}.get(mut, scale)
        S = sc * (k @ np.swapaxes(q, -1, -2) if mut == "transposed_scores" else q @ np.swapaxes(k, -1, -2))
        if causal:
            i = np.arange(N)[:, None]
            j = np.arange(N)[None, :]
            masked = {"mask_includes_diagonal": j >= i, "mask_lower": j < i}.get(mut, j > i)
            S = np.where(masked, -np.inf, S)
        axis = -2 if mut == "softmax_over_queries" else -1
        m = np.max(S, axis=axis, keepdims=True)
        E = np.exp(S - m)
        l = np.sum(E, axis=axis, keepdims=True)
        if mut == "epsilon_denominator":
            P = E / (l + 1e-6)
        elif mut == "unnormalised":
            P = E
        else:
            P = E / l
        O = (np.swapaxes(P, -1, -2) if mut == "pv_transposed" else P) @ v
        if axis == -2:
            m, l = np.swapaxes(m, -1, -2), np.swapaxes(l, -1, -2)
        if mut == "lse_without_max":
            L = np.log(l)[..., 0]
        elif mut == "lse_log2":
            L = (m + np.log2(l))[..., 0]
        else:
            L = (m + np.log(l))[..., 0]
        return O, L
    return fwd


def _bwd_factory(mut):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        N = q.shape[2]
        S = scale * (q @ np.swapaxes(k, -1, -2))
        if causal:
            S = np.where(np.arange(N)[None, :] > np.arange(N)[:, None], -np.inf, S)
        m = np.max(S, axis=-1, keepdims=True)
        P = np.exp(S - m)
        P = P / np.sum(P, axis=-1, keepdims=True)
        T = lambda x: np.swapaxes(x, -1, -2)  # noqa: E731
        dV = (P @ do) if mut == "dV_untransposed" else (T(P) @ do)
        dP = do @ (T(k) if mut == "dP_uses_K" else T(v))
        D = np.sum(P * dP, axis=-1, keepdims=True)
        if mut == "dS_without_D":
            dS = P * dP
        elif mut == "dS_D_sign":
            dS = P * (dP + D)
        else:
            dS = P * (dP - D)
        dQ = (1.0 if mut == "dQ_unscaled" else scale) * (dS @ (q if mut == "dQ_uses_Q" else k))
        dK = (1.0 if mut == "dK_unscaled" else scale) * ((dS if mut == "dK_untransposed" else T(dS)) @ q)
        return dQ, dK, dV, D[..., 0]
    return bwd


def _online_no_rescale(q, k, v, scale, causal, block_k=3):
    """The yunthe.com page's fused pseudocode shape: each key block is normalised by its own
    statistics and added to the output, with no cross-block rescale."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    N = q.shape[2]
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for j0 in range(0, N, block_k):
        cols = np.arange(j0, min(N, j0 + block_k))
        s = scale * (q @ np.swapaxes(k[:, :, cols], -1, -2))
        if causal:
            s = np.where(cols[None, :] > np.arange(N)[:, None], -np.inf, s)
        m = np.max(s, axis=-1, keepdims=True)
        e = np.nan_to_num(np.exp(s - m))
        l = np.sum(e, axis=-1, keepdims=True)
        O += (e / (l + 1e-6)) @ v[:, :, cols]
        L = np.logaddexp(L, (m + np.log(l))[..., 0])
    return O, L


FWD_MUTANTS = ["no_scale", "scale_squared", "transposed_scores", "mask_includes_diagonal", "mask_lower",
               "softmax_over_queries", "epsilon_denominator", "unnormalised", "pv_transposed",
               "lse_without_max", "lse_log2"]
BWD_MUTANTS = ["dV_untransposed", "dP_uses_K", "dS_without_D", "dS_D_sign", "dQ_unscaled", "dQ_uses_Q",
               "dK_unscaled", "dK_untransposed"]


def _fails_some_pin(fwd, bwd, pin_list):
    for pin in pin_list:
        try:
            with np.errstate(all="ignore"):
                if pin in pins.FWD_PINS:
                    pin(fwd)
                else:
                    pin(fwd, bwd)
        except (AssertionError, ValueError, FloatingPointError):
            return pin.__name__
    return None


# Independent families of pins: a mutant must be caught by at least two of them, so no single
# source of truth (for instance the torch library) carries the whole burden.
FWD_FAMILIES = {
    "closed_forms": [pins.check_all_equal_scores, pins.check_causal_row0, pins.check_one_hot,
                     pins.check_single_key_and_two_keys],
    "invariants": [pins.check_rows_sum_to_one, pins.check_row_shift, pins.check_v_linearity,
                   pins.check_permutations],
    "library": [pins.check_torch_sdpa],
    "brute_force": [pins.check_brute_force],
}
BWD_FAMILIES = {
    "library": [pins.check_torch_sdpa],
    "brute_force": [pins.check_brute_force],
    "finite_differences_and_invariants": [pins.check_finite_differences, pins.check_backward_invariants],
}


def test_unmutated_copies_pass_every_pin():
    """The mutant harness itself is right: with no mutation it passes all pins."""
    assert _fails_some_pin(_fwd_factory(None), _bwd_factory(None), pins.FWD_PINS + pins.FWD_BWD_PINS) is None


@pytest.mark.parametrize("mut", FWD_MUTANTS)
def test_forward_mutant_is_caught(mut):
    caught = {fam: _fails_some_pin(_fwd_factory(mut), _bwd_factory(None), lst) for fam, lst in FWD_FAMILIES.items()}
    assert sum(c is not None for c in caught.values()) >= 2, f"forward mutant {mut}: {caught}"


@pytest.mark.parametrize("mut", BWD_MUTANTS)
def test_backward_mutant_is_caught(mut):
    caught = {fam: _fails_some_pin(attn_fwd, _bwd_factory(mut), lst) for fam, lst in BWD_FAMILIES.items()}
    assert sum(c is not None for c in caught.values()) >= 2, f"backward mutant {mut}: {caught}"


def test_unrescaled_blockwise_softmax_is_caught():
    caught = {fam: _fails_some_pin(_online_no_rescale, _bwd_factory(None), lst)
              for fam, lst in FWD_FAMILIES.items() if fam != "library" and fam != "brute_force"}
    assert all(c is not None for c in caught.values()), caught
