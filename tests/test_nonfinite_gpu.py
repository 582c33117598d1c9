"""Non-finite inputs (reading: propagate, never crash, never silently hide). Under the plain definition
a NaN in query row i makes row i's scores, O_i and LSE_i NaN and leaves every other row alone; a NaN
in key j reaches exactly the rows that see key j. The GPU path must agree on which rows are NaN and
stay within the usual gates on the others; the backward must complete."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import flash_attn_bwd, flash_attn_fwd, inputs
from oracle import attn_fwd
from tests.test_parity_gpu import BF16_LSE, BF16_O, dev, host

pytestmark = pytest.mark.gpu


def _x(N, d, seed):
    return {n: inputs.random_tensor((1, 2, N, d), seed + i, "bf16") for i, n in enumerate(("q", "k", "v", "do"))}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_nan_query_row_stays_in_its_row(causal, d):
    N = 300
    x = _x(N, d, 5)
    x["q"][0, 1, 77, 3] = np.nan
    o, lse = flash_attn_fwd(*(dev(x[n], torch.bfloat16) for n in ("q", "k", "v")), d ** -0.5, causal)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], d ** -0.5, causal)
    ho, hl = host(o), host(lse)
    bad = ~np.isfinite(L)
    assert bad[0, 1, 77] and bad.sum() == 1
    assert np.isnan(ho[bad]).all() and np.isnan(hl[bad]).all()
    assert np.abs(ho[~bad] - O[~bad]).max() <= BF16_O and np.abs(hl[~bad] - L[~bad]).max() <= BF16_LSE


@pytest.mark.parametrize("d", [64, 128])
def test_nan_key_reaches_exactly_the_rows_that_see_it(d):
    N, j = 400, 250
    x = _x(N, d, 6)
    x["k"][0, 0, j, 0] = np.nan
    o, lse = flash_attn_fwd(*(dev(x[n], torch.bfloat16) for n in ("q", "k", "v")), d ** -0.5, True)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], d ** -0.5, True)
    ho, hl = host(o), host(lse)
    bad = np.isnan(L)
    assert bad[0, 0, j:].all() and not bad[0, 0, :j].any() and not bad[0, 1].any()
    assert np.isnan(hl[bad]).all() and np.isnan(ho[bad]).all()
    assert np.abs(ho[~bad] - O[~bad]).max() <= BF16_O and np.abs(hl[~bad] - L[~bad]).max() <= BF16_LSE


def test_infinite_query_gives_nan_row_and_backward_completes():
    """+inf in a query makes its scores +-inf and the row's softmax inf/inf = NaN (as in the plain
    definition); the backward over NaN inputs finishes and leaves the untouched head finite."""
    N, d = 260, 64
    x = _x(N, d, 7)
    x["q"][0, 0, 10, :] = np.inf
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = flash_attn_fwd(q, k, v, 0.125, False)
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, 0.125, False)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], 0.125, False)
    assert np.isnan(L[0, 0, 10]) and np.isnan(host(lse)[0, 0, 10])
    assert np.isnan(host(o)[0, 0, 10]).all()
    for g in (dq, dk, dv):
        assert torch.isfinite(g[0, 1]).all()  # the other head never sees the infinity
