"""CPU tests of the float64 oracle against its pins (no GPU)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attn_bwd, attn_bwd_keys, attn_bwd_rows, attn_fwd, attn_fwd_rows, online_fwd
from io_aware_flashattention_flash_amd import inputs
from tests import oracle_pins as pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("pin", pins.FWD_PINS, ids=lambda f: f.__name__)
def test_forward_pin(pin):
    pin(attn_fwd)


@pytest.mark.parametrize("pin", pins.FWD_BWD_PINS, ids=lambda f: f.__name__)
def test_forward_backward_pin(pin):
    pin(attn_fwd, attn_bwd)


@pytest.mark.parametrize("causal", [False, True])
def test_online_recurrence_matches_definition_for_every_block_size(causal):
    """The running-max / running-sum recurrence is an identity: any (block_q, block_k) gives the
    plain softmax attention (ragged last blocks included)."""
    rng = np.random.default_rng(70)
    N, d = 11, 4
    q, k, v = (rng.standard_normal((1, 2, N, d)) * 1.5 for _ in range(3))
    O, L = attn_fwd(q, k, v, 0.9, causal)
    for bq in range(1, N + 1):
        for bk in range(1, N + 1):
            Oo, Lo = online_fwd(q, k, v, 0.9, causal, bq, bk)
            np.testing.assert_allclose(Oo, O, atol=1e-12)
            np.testing.assert_allclose(Lo, L, atol=1e-12)


def test_row_sampler_is_a_slice_of_the_full_forward():
    rng = np.random.default_rng(71)
    q, k, v = (rng.standard_normal((2, 2, 37, 8)) for _ in range(3))
    for causal in (False, True):
        O, L = attn_fwd(q, k, v, 0.3, causal)
        rows = [0, 5, 17, 36]
        Or, Lr = attn_fwd_rows(q, k, v, 0.3, causal, 1, 1, rows)
        np.testing.assert_array_equal(Or, O[1, 1, rows])
        np.testing.assert_array_equal(Lr, L[1, 1, rows])


def test_backward_samplers_are_slices_of_the_full_backward(monkeypatch):
    """dQ of some query rows and dK, dV of some keys equal the same rows of the full backward
    (which its own pins tie to autograd, brute force and finite differences), with the key
    sampler's row chunks smaller than the sequence so chunk boundaries are crossed."""
    rng = np.random.default_rng(74)
    q, k, v, do = (rng.standard_normal((2, 2, 37, 8)) for _ in range(4))
    monkeypatch.setattr(oracle.attention, "_ROW_CHUNK", 5)
    for causal in (False, True):
        dQ, dK, dV, D = attn_bwd(q, k, v, do, 0.3, causal)
        rows = [0, 5, 17, 36]
        dQr, Dr = attn_bwd_rows(q, k, v, do, 0.3, causal, 1, 0, rows)
        np.testing.assert_allclose(dQr, dQ[1, 0, rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Dr, D[1, 0, rows], rtol=0, atol=1e-13)
        for keys in ([0, 1, 36], [20, 33, 35, 36], [36]):
            dKk, dVk = attn_bwd_keys(q, k, v, do, 0.3, causal, 0, 1, keys)
            np.testing.assert_allclose(dKk, dK[0, 1, keys], rtol=0, atol=1e-13)
            np.testing.assert_allclose(dVk, dV[0, 1, keys], rtol=0, atol=1e-13)


def test_row_chunking_does_not_change_results(monkeypatch):
    rng = np.random.default_rng(72)
    q, k, v = (rng.standard_normal((1, 1, 50, 4)) for _ in range(3))
    O1, L1 = attn_fwd(q, k, v, 0.5, True)
    monkeypatch.setattr(oracle.attention, "_ROW_CHUNK", 7)
    O2, L2 = attn_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(O2, O1, atol=1e-14)
    np.testing.assert_allclose(L2, L1, atol=1e-14)


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(73).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]  # exact ties both ways
    ours = inputs.round_to_bf16(x)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_fp16_rounding_matches_torch():
    """The fp16 input rounding (NumPy's cast) agrees with torch's float32 -> float16 conversion,
    including ties and values near the binary16 subnormal boundary."""
    import torch

    x = np.random.default_rng(74).standard_normal(100000).astype(np.float32) * 3
    x[:5] = [1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -(1.0 + 2 ** -11), 0.0, 2 ** -15]  # exact ties both ways
    ours = inputs.round_to_fp16(x)
    ref = torch.tensor(x).to(torch.float16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_recipe_regression_golden():
    """Oracle output on the fp32 N=128 d=64 workload under the seeded recipe, stored by
    tests/golden/make_golden.py (which calls only the oracle and the input module)."""
    with open(os.path.join(GOLDEN, "recipe_fwd_fp32_b1h1n128d64.json")) as f:
        g = json.load(f)
    w = inputs.WORKLOADS["fwd_fp32_b1h1n128d64"]
    x = inputs.make_inputs(w)
    O, L = attn_fwd(x["q"], x["k"], x["v"], w.scale, w.causal)
    np.testing.assert_allclose(O[0, 0, 0, :4], g["O_0_0_0_first4"], atol=1e-12)
    np.testing.assert_allclose(L[0, 0, :4], g["LSE_0_0_first4"], atol=1e-12)
    assert abs(O.sum() - g["sum_O"]) < 1e-9
    assert abs(L.sum() - g["sum_LSE"]) < 1e-9
    assert abs(np.abs(O).max() - g["max_abs_O"]) < 1e-12


def test_pages_quadratic_intermediate_sizes():
    """The codechina.net article (section 3.3) prints the fp32 N x N score-matrix size per head:
    about 4 MB at N=1024, 256 MB at 8192 and 4 GB at 32768. N^2 * 4 bytes reproduces them in MiB;
    the fused path's caller-visible buffers are O(N d) instead (checked on the GPU)."""
    with open(os.path.join(GOLDEN, "pages_n2_fp32_sizes.json")) as f:
        g = json.load(f)
    for row in g["rows"]:
        mib = row["N"] ** 2 * 4 / 2 ** 20
        assert mib == row["printed_MiB"], row


def test_lse_definition_on_causal_prefix():
    """LSE_i is the natural log of the normaliser of row i: exp(LSE_i) = sum over visible keys of
    exp(s_ij). Check on a case small enough to sum by hand with math.fsum."""
    q = np.array([[[[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]]]])
    k = np.array([[[[0.5, -1.0], [2.0, 0.0], [0.0, 0.0]]]])
    v = np.zeros_like(k)
    _, L = attn_fwd(q, k, v, 1.0, True)
    s = [[0.5], [-1.0, 0.0], [-0.5, 2.0, 0.0]]
    for i in range(3):
        assert abs(L[0, 0, i] - math.log(math.fsum(math.exp(t) for t in s[i]))) < 1e-14


# ---------------------------------------------------------------------------------------------
# Nq queries against Nk >= Nq keys (decode / chunked prefill)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq", [1, 5, 37])
def test_kv_oracle_matches_torch_sdpa_with_bottom_right_mask(causal, nq):
    """torch's float64 scaled_dot_product_attention with an explicit mask that lets query i see
    keys j <= Nk - Nq + i (and the matching logsumexp) on non-square inputs."""
    import torch

    from oracle import attn_fwd_kv

    rng = np.random.default_rng(80 + nq)
    B, H, Nk, d = 2, 3, 37, 6
    q = rng.standard_normal((B, H, nq, d))
    k, v = rng.standard_normal((B, H, Nk, d)), rng.standard_normal((B, H, Nk, d))
    scale = 0.7
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    visible = torch.ones(nq, Nk, dtype=torch.bool)
    if causal:
        visible = torch.arange(Nk)[None, :] <= (torch.arange(nq)[:, None] + Nk - nq)
    tO = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=visible, scale=scale)
    s = (scale * (tq @ tk.transpose(-1, -2))).masked_fill(~visible, float("-inf"))
    O, L = attn_fwd_kv(q, k, v, scale, causal)
    np.testing.assert_allclose(O, tO.numpy(), atol=1e-12)
    np.testing.assert_allclose(L, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_oracle_is_the_tail_of_the_full_sequence(causal):
    """Decoding property: the last Nq rows of the square problem over the whole sequence are the
    non-square problem of those Nq queries against all keys (for every Nq, including Nq = Nk)."""
    from oracle import attn_fwd_kv

    rng = np.random.default_rng(81)
    N, d = 29, 5
    q, k, v = (rng.standard_normal((1, 2, N, d)) for _ in range(3))
    O_full, L_full = attn_fwd(q, k, v, 0.8, causal)
    for nq in (1, 2, 13, N):
        O, L = attn_fwd_kv(q[:, :, N - nq:], k, v, 0.8, causal)
        np.testing.assert_allclose(O, O_full[:, :, N - nq:], atol=1e-13)
        np.testing.assert_allclose(L, L_full[:, :, N - nq:], atol=1e-13)


def test_kv_oracle_equal_keys_give_the_mean_of_values():
    """Closed form: with every key equal, every visible score is equal, so a single decoded query
    (which sees all Nk keys, causal or not) returns the mean of V and LSE = scale*q.k + ln Nk."""
    from oracle import attn_fwd_kv

    rng = np.random.default_rng(82)
    Nk, d = 23, 4
    q = rng.standard_normal((1, 1, 1, d))
    k = np.repeat(rng.standard_normal((1, 1, 1, d)), Nk, axis=2)
    v = rng.standard_normal((1, 1, Nk, d))
    for causal in (False, True):
        O, L = attn_fwd_kv(q, k, v, 1.3, causal)
        np.testing.assert_allclose(O[0, 0, 0], v[0, 0].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(L[0, 0, 0], 1.3 * float(q[0, 0, 0] @ k[0, 0, 0]) + math.log(Nk), atol=1e-13)


def test_grid_codes_widen_exactly_to_16_bit():
    """The size-limit tests' inputs: codes / 64 are exact in bf16 and fp16, and cover the grid."""
    import torch
    c = inputs.grid_codes((4096,), 5)
    assert c.dtype == np.int8 and c.min() == -128 and c.max() == 127
    v = c.astype(np.float64) * inputs.GRID_STEP
    for dt in (torch.bfloat16, torch.float16):
        t = torch.from_numpy(c).to(dt).mul_(inputs.GRID_STEP)
        np.testing.assert_array_equal(t.double().numpy(), v)
