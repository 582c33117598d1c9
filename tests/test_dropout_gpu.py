"""GPU parity of attention dropout against the float64 oracle, through the C ABI.

The keep mask is integer work and must match the oracle's Philox4x32-10 mask bit for bit. The
forward and backward with dropout are then held to the dense gates (O <= 1e-2 and LSE <= 1e-3
max-abs on rows that see a key, gradients <= 5e-2 relative to their norm), the oracle using its
own mask. Kept weights grow by 256 / T, so |O| can pass 4, where half a bf16 ulp alone is 0.0156:
as for the other outputs that large, O's gate applies to the error beyond O's own rounding."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd_masked, flash_attn_dropout_mask, flash_attn_fwd_masked,
                                               inputs)
from oracle import attn_bwd_dropout, attn_fwd_dropout, keep_mask, padded_batch_visible
from tests.test_parity_gpu import BF16_LSE, BF16_O, DEV, GRAD, beyond_rounding, dev, grad_errors, host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 1, 1, 1), (2, 3, 37, 100), (1, 2, 300, 1000), (2, 1, 129, 33)])
@pytest.mark.parametrize("p,seed", [(0.1, 0), (0.5, 2 ** 64 - 1), (0.9, 0x0123456789ABCDEF)])
def test_keep_mask_is_bit_exact(B, H, Nq, Nk, p, seed):
    got = flash_attn_dropout_mask(B, H, Nq, Nk, p, seed, device=DEV).cpu().numpy()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.astype(bool), keep_mask(B, H, Nq, Nk, p, seed))


def _case(B, H, N, d, causal, p, seed, seqlens=None, bmap=None, dtype="bf16", backward=True, in_seed=0):
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    names = ("q", "k", "v", "do")
    x = {n: inputs.random_tensor((B, H, N, d), in_seed + i, dtype) for i, n in enumerate(names)}
    q, k, v, do = (dev(x[n], tdt) for n in names)
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    bm = None if bmap is None else torch.from_numpy(bmap).to(DEV)
    scale = d ** -0.5
    o, lse = flash_attn_fwd_masked(q, k, v, scale, causal, seqlens=sl, block_mask=bm, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    vis = padded_batch_visible(B, H, N, causal, seqlens, bmap, 128)
    keep = keep_mask(B, H, N, N, p, seed)
    O, L = attn_fwd_dropout(x["q"], x["k"], x["v"], scale, vis, keep, p)
    full = np.isfinite(L)
    ho, hl = host(o), host(lse)
    assert np.isfinite(ho).all() and (ho[~full] == 0).all() and np.isneginf(hl[~full]).all()
    assert beyond_rounding(ho[full], O[full]) <= BF16_O
    assert np.abs(hl[full] - L[full]).max(initial=0) <= BF16_LSE
    if not backward:
        return o, lse
    dq, dk, dv = flash_attn_bwd_masked(do, q, k, v, o, lse, scale, causal, seqlens=sl, block_mask=bm, dropout_p=p,
                                       seed=seed)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = attn_bwd_dropout(x["q"], x["k"], x["v"], x["do"], scale, vis, keep, p)
    for name, g, r in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
        g = host(g)
        assert np.isfinite(g).all(), name
        e_inf, e_fro = grad_errors(g, r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,p", [(200, 0.1), (700, 0.3), (1100, 0.5)])
def test_dropout_fwd_bwd(N, p, causal, d):
    _case(2, 2, N, d, causal, p, seed=1234 + N, in_seed=N + d)


def test_dropout_with_padding_and_block_map():
    N = 900
    bmap = (np.random.default_rng(5).random((2, 2, 8, 8)) < 0.6).astype(np.uint8)
    bmap[:, :, np.arange(8), np.arange(8)] = 1
    _case(2, 2, N, 128, True, 0.2, seed=77, seqlens=[900, 555], bmap=bmap, in_seed=3)


def test_dropout_with_padding_eight_heads():
    """Lengths with eight heads per sequence (the forward's tiles with work run first and write the
    padding rows)."""
    _case(3, 8, 500, 64, True, 0.2, seed=11, seqlens=[500, 0, 333], in_seed=13)


def test_dropout_fp16():
    _case(1, 4, 600, 128, True, 0.25, seed=5, dtype="fp16", in_seed=9)


def test_dropout_deterministic_and_seed_dependent():
    B, H, N, d = 2, 4, 1000, 64
    q, k, v = (dev(inputs.random_tensor((B, H, N, d), s, "bf16"), torch.bfloat16) for s in (1, 2, 3))
    a = flash_attn_fwd_masked(q, k, v, 0.125, True, dropout_p=0.3, seed=42)
    b = flash_attn_fwd_masked(q, k, v, 0.125, True, dropout_p=0.3, seed=42)
    c = flash_attn_fwd_masked(q, k, v, 0.125, True, dropout_p=0.3, seed=43)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0])
    assert torch.equal(a[1], c[1])  # LSE does not depend on the dropout draw
