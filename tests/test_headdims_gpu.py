"""GPU parity at head dims 32, 96 and 256 (the 16-bit paths; 64 and 128 are covered with the five
workloads) against the float64 oracle, through the C ABI: forward, backward, key-split decode, and
the masked / dropout paths. Same gates as the other 16-bit tests."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd, flash_attn_bwd_masked, flash_attn_fwd,
                                               flash_attn_fwd_kvsplit, flash_attn_fwd_masked, inputs)
from oracle import (attn_bwd, attn_bwd_dropout, attn_fwd, attn_fwd_dropout, attn_fwd_kv, attn_fwd_rows, keep_mask,
                    padded_batch_visible)
from tests.test_parity_gpu import BF16_LSE, BF16_O, DEV, GRAD, beyond_rounding, dev, grad_errors, host

pytestmark = pytest.mark.gpu

DIMS = [32, 96, 256]
TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _x(B, H, N, d, seed, dtype, names=("q", "k", "v", "do")):
    return {n: inputs.random_tensor((B, H, N, d), seed + i, dtype) for i, n in enumerate(names)}


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 200, 1000])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fwd_bwd(N, causal, d, dtype):
    x = _x(1, 2, N, d, seed=N + d, dtype=dtype)
    q, k, v, do = (dev(x[n], TDT[dtype]) for n in ("q", "k", "v", "do"))
    scale = d ** -0.5
    o, lse = flash_attn_fwd(q, k, v, scale, causal)
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], scale, causal)
    assert np.abs(host(o) - O).max() <= BF16_O
    assert np.abs(host(lse) - L).max() <= BF16_LSE
    dQ, dK, dV, _ = attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
    for name, g, r in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
        e_inf, e_fro = grad_errors(host(g), r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)


@pytest.mark.parametrize("d", DIMS)
def test_fwd_long_sequence_sampled_rows(d):
    """A long causal sequence, checked on sampled rows (first, tile edges, ragged tail)."""
    B, H, N = 1, 4, 4100
    x = _x(B, H, N, d, seed=d, dtype="bf16", names=("q", "k", "v"))
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd(q, k, v, d ** -0.5, True)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 2047, 4095, 4096, 4099]
    for h in (0, 3):
        Or, Lr = attn_fwd_rows(x["q"], x["k"], x["v"], d ** -0.5, True, 0, h, rows)
        assert np.abs(host(o[0, h, rows]) - Or).max() <= BF16_O
        assert np.abs(host(lse[0, h, rows]) - Lr).max() <= BF16_LSE


@pytest.mark.parametrize("d", DIMS)
@pytest.mark.parametrize("Nq,Nk", [(1, 3000), (100, 777)])
def test_kvsplit(Nq, Nk, d):
    x = {"q": inputs.random_tensor((2, 2, Nq, d), 1, "bf16"), "k": inputs.random_tensor((2, 2, Nk, d), 2, "bf16"),
         "v": inputs.random_tensor((2, 2, Nk, d), 3, "bf16")}
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd_kvsplit(q, k, v, d ** -0.5, True, 0)
    torch.cuda.synchronize()
    O, L = attn_fwd_kv(x["q"], x["k"], x["v"], d ** -0.5, True)
    assert np.abs(host(o) - O).max() <= BF16_O
    assert np.abs(host(lse) - L).max() <= BF16_LSE


@pytest.mark.parametrize("d", DIMS)
def test_masked_with_dropout(d):
    B, H, N, p, seed = 2, 2, 700, 0.2, 31
    x = _x(B, H, N, d, seed=5 * d, dtype="bf16")
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    bmap = (np.random.default_rng(d).random((B, H, 6, 6)) < 0.6).astype(np.uint8)
    bmap[:, :, np.arange(6), np.arange(6)] = 1
    seqlens = [700, 450]
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    bm = torch.from_numpy(bmap).to(DEV)
    scale = d ** -0.5
    o, lse = flash_attn_fwd_masked(q, k, v, scale, True, seqlens=sl, block_mask=bm, dropout_p=p, seed=seed)
    g = flash_attn_bwd_masked(do, q, k, v, o, lse, scale, True, seqlens=sl, block_mask=bm, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    vis = padded_batch_visible(B, H, N, True, seqlens, bmap, 128)
    keep = keep_mask(B, H, N, N, p, seed)
    O, L = attn_fwd_dropout(x["q"], x["k"], x["v"], scale, vis, keep, p)
    full = np.isfinite(L)
    ho = host(o)
    assert (ho[~full] == 0).all()
    assert beyond_rounding(ho[full], O[full]) <= BF16_O
    assert np.abs(host(lse)[full] - L[full]).max() <= BF16_LSE
    ref = attn_bwd_dropout(x["q"], x["k"], x["v"], x["do"], scale, vis, keep, p)
    for name, gg, r in zip(("dQ", "dK", "dV"), g, ref[:3]):
        e_inf, e_fro = grad_errors(host(gg), r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)
