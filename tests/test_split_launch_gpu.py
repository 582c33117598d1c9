"""GPU parity of small launches (their workgroups fit on the chip at once), where the kernels split
their longest work in two:
  * dK/dV: the longest key tiles of each head (keys 0-63 and 64-127 of the tile); each wave takes
    one of the two 32-row blocks of every query tile, and the two waves that share keys add their
    partial sums at the end. The host splits about 3/8 of a head's key tiles when the launch has
    at least 8 key tiles per head and its workgroups all fit on the chip at once (so the launch
    would otherwise last as long as key tile 0), and only as many as still fit. Smaller launches,
    whose 64-key workgroups all fit at once (N >= 512), instead give every workgroup 64 keys and
    its wave pairs the even and the odd query tiles, exchanging dK and dV partials at the end.
  * dQ (causal, d <= 128, when the 64-row workgroups all fit at once; N >= 512): 64-row
    workgroups whose wave pairs take the even and the odd key tiles of the rows; the odd pair hands
    its dQ partial sums to the even pair, which adds them.
  * forward (dense, d <= 128, no more 128-row tiles than CUs (half as many at d > 64; causal
    launches with long rows up to twice that), N >= 256):
    64-row workgroups whose wave pairs take the even and the odd 64-key tiles of the rows; the
    odd pair hands its running max, row sums and O accumulator to the even pair, which merges
    them by the online-softmax rule.
The shapes below cover head dims 32 to 128, bf16 and fp16, ragged lengths, causal and not, a
launch where the fit bounds the dK/dV split count (12 heads of 16 key tiles at d = 128, one
workgroup per CU), and forward rows whose odd tiles score far above their even ones (the merge
must rescale the even part). Every output element is compared with the float64 oracle; outputs
are poisoned with NaN beforehand."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd, flash_attn_bwd_dkdv, flash_attn_bwd_dq, flash_attn_fwd,
                                               inputs)
from oracle import attn_bwd, attn_fwd
from tests.test_parity_gpu import BF16_LSE, BF16_O, GRAD, beyond_rounding, dev, grad_errors, host

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
    ("bf16", 64, 1, 24, 1500),  # too many 64-key workgroups for the stream split: the key-tile split
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


@pytest.mark.parametrize("dtype,d,B,H,N,causal", [
    ("bf16", 64, 1, 2, 1024, True),
    ("bf16", 64, 1, 2, 2100, True),
    ("bf16", 64, 1, 3, 1000, False),
    ("bf16", 32, 2, 2, 1500, True),
    ("bf16", 32, 1, 2, 333, False),
    ("fp16", 64, 1, 2, 1100, True),
    ("bf16", 64, 1, 2, 256, True),
    ("bf16", 128, 1, 2, 1024, True),
    ("bf16", 128, 1, 3, 700, False),
    ("bf16", 96, 1, 2, 1000, True),
    ("fp16", 128, 1, 2, 600, True),
    ("bf16", 128, 1, 12, 2048, True),  # causal with long rows: up to twice the tiles
    ("bf16", 64, 1, 16, 4096, True),
])
def test_fwd_small_launch(dtype, d, B, H, N, causal):
    print(f"split forward launch {dtype} B{B} H{H} N{N} d{d} causal {causal}", flush=True)
    w = inputs.Workload("t", dtype, B, H, N, d, causal, False)
    x = inputs.make_inputs(w, seed=3 * N + d + H)
    q, k, v = (dev(x[n], DT[dtype]) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=q.device)
    flash_attn_fwd(q, k, v, w.scale, causal, out=o, lse=lse)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], w.scale, causal)
    err, lerr = float(np.abs(host(o) - O).max()), float(np.abs(host(lse) - L).max())
    print(f"  O err {err:.3e} (beyond output rounding {beyond_rounding(host(o), O):.3e}), LSE err {lerr:.3e}")
    assert err <= BF16_O and lerr <= BF16_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_small_launch_odd_tiles_score_higher(causal):
    """Keys of the odd 64-key tiles scaled up so that their scores exceed the even tiles' by far
    more than the 2^16 guard: the odd pair's running max ends far above the even pair's, and the
    merge must scale the even part down by exp2(m_even - m) (underflowing to zero where the gap is
    that large) without losing the odd part."""
    B, H, N, d = 1, 2, 1024, 64
    w = inputs.Workload("t", "bf16", B, H, N, d, causal, False)
    x = inputs.make_inputs(w, seed=77)
    factor = np.where((np.arange(N) // 64) % 2 == 1, 6.0, 1.0).astype(np.float32)
    x["k"] = inputs.round_to_bf16(x["k"] * factor[None, None, :, None])
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o, lse = flash_attn_fwd(q, k, v, w.scale, causal)
    torch.cuda.synchronize()
    O, L = attn_fwd(x["q"], x["k"], x["v"], w.scale, causal)
    beyond, lerr = beyond_rounding(host(o), O), float(np.abs(host(lse) - L).max())
    print(f"causal {causal}: O beyond output rounding {beyond:.3e}, LSE err {lerr:.3e}")
    assert beyond <= BF16_O and lerr <= BF16_LSE
