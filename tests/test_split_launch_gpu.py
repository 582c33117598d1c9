"""GPU parity of small causal backward launches, where the backward kernels split their longest
tiles across two half-size workgroups:
  * dK/dV: the longest key tiles of each head (keys 0-63 and 64-127 of the tile); each wave takes
    one of the two 32-row blocks of every query tile, and the two waves that share keys add their
    partial sums at the end. The host splits about 3/8 of a head's key tiles when the launch has
    at least 8 key tiles per head and its workgroups all fit on the chip at once (so the launch
    would otherwise last as long as key tile 0), and only as many as still fit.
  * dQ (d <= 64, launches that fill at most half of the chip's slots): the longest query tiles
    (rows 0-63 and 64-127 of the tile); each wave takes one of the two 32-key blocks of every key
    tile, and the two waves that share rows add their partial sums at the end.
The shapes below cover head dims 32 to 128, bf16 and fp16, ragged lengths, and a launch where the
fit bounds the dK/dV split count (12 heads of 16 key tiles at d = 128, one workgroup per CU).
Every element of dQ, dK and dV is compared with the float64 oracle; outputs are poisoned with NaN
beforehand."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd, flash_attn_bwd_dkdv, flash_attn_bwd_dq, flash_attn_fwd,
                                               inputs)
from oracle import attn_bwd
from tests.test_parity_gpu import GRAD, dev, grad_errors, host

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "fp16": torch.float16}


@pytest.mark.parametrize("dtype,d,B,H,N", [
    ("bf16", 64, 1, 2, 1024),
    ("bf16", 64, 1, 2, 2100),
    ("bf16", 32, 1, 3, 1000),
    ("bf16", 96, 1, 2, 1500),
    ("bf16", 128, 1, 2, 1024),
    ("bf16", 128, 1, 12, 2048),
    ("fp16", 64, 2, 2, 1100),
])
def test_bwd_small_causal_launch(dtype, d, B, H, N):
    print(f"split dK/dV launch {dtype} B{B} H{H} N{N} d{d} causal", flush=True)
    w = inputs.Workload("t", dtype, B, H, N, d, True, True)
    x = inputs.make_inputs(w, seed=7 * N + d + H)
    q, k, v, do = (dev(x[n], DT[dtype]) for n in ("q", "k", "v", "do"))
    o, lse = flash_attn_fwd(q, k, v, w.scale, True)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    flash_attn_bwd(do, q, k, v, o, lse, w.scale, True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    dQ, dK, dV, _ = attn_bwd(x["q"], x["k"], x["v"], x["do"], w.scale, True)
    for name, g, r in (("dQ", dq, dQ), ("dK", dk, dK), ("dV", dv, dV)):
        assert bool(torch.isfinite(g).all()), name
        e_inf, e_fro = grad_errors(host(g), r)
        print(f"  {name}: {e_inf:.2e} / {e_fro:.2e}")
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)


def test_bwd_small_causal_launch_deterministic_and_staged():
    """Repeated calls give the same bits, the staged dQ then dK/dV calls reproduce the fused
    backward bit for bit, and the delta rows the split dQ launch writes (one wave of each pair
    writes them) equal rowsum(dO * O) in float64."""
    w = inputs.Workload("t", "bf16", 1, 2, 2048, 64, True, True)
    x = inputs.make_inputs(w, seed=41)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = flash_attn_fwd(q, k, v, w.scale, True)
    ref = flash_attn_bwd(do, q, k, v, o, lse, w.scale, True)
    for _ in range(3):
        got = flash_attn_bwd(do, q, k, v, o, lse, w.scale, True)
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
    dq2, delta = flash_attn_bwd_dq(q, k, v, o, lse, do, w.scale, True)
    dk2, dv2 = flash_attn_bwd_dkdv(q, k, v, lse, do, delta, w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], dq2) and torch.equal(ref[1], dk2) and torch.equal(ref[2], dv2)
    want = np.sum(host(o) * x["do"].astype(np.float64), axis=-1)
    assert np.abs(host(delta) - want).max() <= 1e-4 * max(1.0, np.abs(want).max())
