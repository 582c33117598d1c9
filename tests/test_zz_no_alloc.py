"""The no-allocation key-split forward (flash_attn_fwd_kvsplit_noalloc) against the entry point
that takes a workspace (flash_attn_fwd_kvsplit), through the C ABI, on two calls in a row, the
second with a smaller input than the first (the shared scratch keeps the first call's contents).
Both are also held to the bf16 oracle gates (O <= 1e-2, LSE <= 1e-3)."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import flash_attn_fwd_kvsplit, flash_attn_fwd_kvsplit_noalloc, inputs
from oracle import attn_fwd_kv
from tests.test_parity_gpu import BF16_LSE, BF16_O, DEV, dev, host

pytestmark = pytest.mark.gpu

CASES = [  # (B, H, Nq, Nk, d, causal, num_splits): the second is smaller in every dimension
    (4, 8, 3, 2000, 128, True, 0),
    (2, 4, 1, 700, 64, False, 5),
]


def _qkv(B, H, Nq, Nk, d, seed):
    q = inputs.random_tensor((B, H, Nq, d), seed, "bf16")
    k = inputs.random_tensor((B, H, Nk, d), seed + 1, "bf16")
    v = inputs.random_tensor((B, H, Nk, d), seed + 2, "bf16")
    return q, k, v


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    for i, (B, H, Nq, Nk, d, causal, S) in enumerate(CASES):
        print(f"case {i}: B{B} H{H} Nq{Nq} Nk{Nk} d{d} causal={causal} splits={S}", flush=True)
        q, k, v = _qkv(B, H, Nq, Nk, d, 90 + 10 * i)
        tq, tk, tv = (dev(x, torch.bfloat16) for x in (q, k, v))
        o_na = torch.full_like(tq, float("nan"))
        l_na = torch.full((B, H, Nq), float("nan"), device=DEV)
        flash_attn_fwd_kvsplit_noalloc(tq, tk, tv, o_na, l_na, None, causal, S)
        o_ws, l_ws = flash_attn_fwd_kvsplit(tq, tk, tv, None, causal, S)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws), "O differs from the workspace entry point"
        assert torch.equal(l_na, l_ws), "LSE differs from the workspace entry point"
        O, L = attn_fwd_kv(q, k, v, d ** -0.5, causal)
        err_o, err_l = np.abs(host(o_na) - O).max(), np.abs(host(l_na) - L).max()
        print(f"  O err {err_o:.3e} LSE err {err_l:.3e}", flush=True)
        assert err_o <= BF16_O and err_l <= BF16_LSE
