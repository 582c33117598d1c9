"""GPU parity on a seeded sweep of small shapes (the dense 16-bit forward and backward against the
float64 oracle): batch, heads, ragged lengths, every head dim, causal or not, bf16 or fp16, and
scales other than 1/sqrt(d) (larger, smaller, negative). Complements the fixed-shape tests with
combinations none of them picks. Gates: O beyond the rounding of the stored output <= 1e-2 (the
sharper rows of a large scale reach |O| where half a 16-bit ulp alone nears the gate), LSE <= 1e-3,
gradients <= 5e-2 relative."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import flash_attn_bwd, flash_attn_fwd, inputs
from oracle import attn_bwd, attn_fwd
from tests.test_parity_gpu import BF16_LSE, BF16_O, GRAD, beyond_rounding, dev, grad_errors, host

pytestmark = pytest.mark.gpu

TDT = {"bf16": torch.bfloat16, "fp16": torch.float16}


def _configs(n=96, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([32, 64, 96, 128, 256]))
        B = int(rng.integers(1, 4))
        H = int(rng.choice([1, 2, 3, 5, 8]))
        N = int(rng.choice([1, 2, 31, 64, 65, 127, 200, 333, 512, 700]))
        causal = bool(rng.integers(0, 2))
        dtype = str(rng.choice(["bf16", "fp16"]))
        scale = float(rng.choice([1.0, 0.5, 2.0, -1.0])) * d ** -0.5
        out.append((i, B, H, N, d, causal, dtype, scale))
    return out


@pytest.mark.parametrize("i,B,H,N,d,causal,dtype,scale", _configs())
def test_random_shape_fwd_bwd(i, B, H, N, d, causal, dtype, scale):
    x = {n: inputs.random_tensor((B, H, N, d), 1000 + 10 * i + j, dtype) for j, n in enumerate(("q", "k", "v", "do"))}
    q, k, v, do = (dev(x[n], TDT[dtype]) for n in ("q", "k", "v", "do"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, N), float("nan"), device=q.device)
    flash_attn_fwd(q, k, v, scale, causal, out=o, lse=lse)
    dq, dk, dv = flash_attn_bwd(do, q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], scale, causal)
    ho, hl = host(o), host(lse)
    assert np.isfinite(ho).all() and np.isfinite(hl).all()
    assert beyond_rounding(ho, O) <= BF16_O
    assert np.abs(hl - L).max() <= BF16_LSE
    dQ, dK, dV, _ = attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, causal)
    for name, g, r in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
        g = host(g)
        assert np.isfinite(g).all(), name
        e_inf, e_fro = grad_errors(g, r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)
