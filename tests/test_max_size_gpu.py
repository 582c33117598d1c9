"""GPU parity at the largest sizes the library accepts. A head is addressed with 32-bit byte
offsets, so N * d must stay below 2^29 elements, and a tensor must hold fewer than 2^31 elements.
Causal bf16 launches sit just under those limits, with ragged lengths (forward and backward
unless stated):
  * one head of N = 2^21 - 32 at d = 256 (N * d = 2^29 - 8192: byte offsets within a head reach
    ~2^30);
  * B2 H64 N = 2^17 - 32 at d = 128 (2^31 - 524288 elements per tensor: the last heads start
    beyond 2^32 bytes);
  * the key-split forward (decoding) of a few queries against a cache of 2^21 - 32 keys at d = 256
    (forward only; every query row is checked).
The oracle cannot form these launches in full on the host, so it checks what it can compute one
sample at a time: query rows at the start, across tile edges, in the middle and at the end (O,
LSE, dQ), and the last keys of a head (dK, dV; under the causal mask only the last rows see them,
and the last tiles carry the largest offsets). Every output element is poisoned with NaN
beforehand and must come back finite. Inputs are uniform codes times 1/64, exact in bf16. Gates
as for the full-size workloads: O <= 1e-2 beyond its bf16 rounding, LSE <= 1e-3, gradients
<= 5e-2 relative (max and Frobenius over the sample)."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import flash_attn_bwd, flash_attn_fwd, flash_attn_fwd_kvsplit, inputs
from oracle import attn_bwd_keys, attn_bwd_rows, attn_fwd_kv, attn_fwd_rows
from tests.test_parity_gpu import BF16_LSE, BF16_O, GRAD, DEV, beyond_rounding, grad_errors, host

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "do")


def _rows(N):
    return sorted({0, 1, 63, 64, 127, 128, 129, 4097, N // 2 + 5, N - 130, N - 65, N - 33, N - 1})


def _check_launch(B, H, N, d, heads, seed):
    shape = (B, H, N, d)
    print(f"size-limit launch {shape}, causal bf16, seed {seed}", flush=True)
    codes = {n: inputs.grid_codes(shape, seed + i) for i, n in enumerate(NAMES)}
    t = {n: torch.from_numpy(c).to(DEV).to(torch.bfloat16).mul_(inputs.GRID_STEP) for n, c in codes.items()}
    q, k, v, do = (t[n] for n in NAMES)
    scale = d ** -0.5
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=DEV)
    flash_attn_fwd(q, k, v, scale, True, out=o, lse=lse)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    flash_attn_bwd(do, q, k, v, o, lse, scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, x in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(x).all()), name
    rows = _rows(N)
    keys = [N - 64, N - 63, N - 40, N - 33, N - 32, N - 2, N - 1]
    for b, h in heads:
        x = {n: codes[n][b:b + 1, h:h + 1].astype(np.float64) * inputs.GRID_STEP for n in NAMES}
        Or, Lr = attn_fwd_rows(x["q"], x["k"], x["v"], scale, True, 0, 0, rows)
        go, gl = host(o[b, h, rows]), host(lse[b, h, rows])
        assert beyond_rounding(go, Or) <= BF16_O, (b, h)
        assert np.abs(gl - Lr).max() <= BF16_LSE, (b, h)
        dQr, _ = attn_bwd_rows(x["q"], x["k"], x["v"], x["do"], scale, True, 0, 0, rows)
        dKk, dVk = attn_bwd_keys(x["q"], x["k"], x["v"], x["do"], scale, True, 0, 0, keys)
        for name, g, r in (("dQ", dq[b, h, rows], dQr), ("dK", dk[b, h, keys], dKk), ("dV", dv[b, h, keys], dVk)):
            e_inf, e_fro = grad_errors(host(g), r)
            print(f"head ({b}, {h}) {name}: {e_inf:.2e} / {e_fro:.2e}")
            assert e_inf <= GRAD and e_fro <= GRAD, (b, h, name, e_inf, e_fro)


def test_longest_head():
    """One head at the per-head limit: 2^21 - 32 rows of d = 256."""
    _check_launch(1, 1, (1 << 21) - 32, 256, [(0, 0)], seed=900)


def test_largest_tensors():
    """2^31 - 524288 elements per tensor: heads at the start, the middle and the end."""
    _check_launch(2, 64, (1 << 17) - 32, 128, [(0, 0), (0, 63), (1, 7), (1, 63)], seed=910)


@pytest.mark.parametrize("Nq,splits", [(1, 0), (17, 0), (64, 7)])
def test_key_split_longest_cache(Nq, splits):
    """Nq queries (the cache's last positions under the causal mask) against 2^21 - 32 keys of
    d = 256, with the automatic or a given split count; every query row against the oracle."""
    B, H, Nk, d = 1, 2, (1 << 21) - 32, 256
    print(f"key-split size-limit launch: B{B} H{H} Nq {Nq} Nk {Nk} d {d}, splits {splits}", flush=True)
    cq = inputs.grid_codes((B, H, Nq, d), 920 + Nq)
    ck, cv = inputs.grid_codes((B, H, Nk, d), 921), inputs.grid_codes((B, H, Nk, d), 922)
    q, k, v = (torch.from_numpy(c).to(DEV).to(torch.bfloat16).mul_(inputs.GRID_STEP) for c in (cq, ck, cv))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=DEV)
    flash_attn_fwd_kvsplit(q, k, v, d ** -0.5, True, splits, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    for h in range(H):
        x = [c[:, h:h + 1].astype(np.float64) * inputs.GRID_STEP for c in (cq, ck, cv)]
        O, L = attn_fwd_kv(x[0], x[1], x[2], d ** -0.5, True)
        assert beyond_rounding(host(o[:, h:h + 1]), O) <= BF16_O, h
        assert np.abs(host(lse[:, h:h + 1]) - L).max() <= BF16_LSE, h
