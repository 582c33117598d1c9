"""CPU tests of the float64 oracle against its pins (no GPU)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attn_bwd, attn_fwd, attn_fwd_rows, online_fwd
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
