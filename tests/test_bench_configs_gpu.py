"""GPU parity at the exact shapes and launch configurations of the benchmark's extra lines (block-sparse
and variable-length forwards, the dropout step, key-split decode), checked on sampled rows against
the float64 oracle, plus the extremes of the dropout threshold. The inputs are rebuilt with the
benchmark's own seeds and recipe (seeded N(0, 1), rounded to bf16)."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd_masked, flash_attn_dropout_mask, flash_attn_fwd_kvsplit,
                                               flash_attn_fwd_masked, inputs)
from oracle import attn_fwd_dropout, attn_fwd_kv, attn_fwd_masked, keep_mask, keep_threshold, padded_batch_visible
from oracle.dropout import random_bytes
from tests.test_parity_gpu import BF16_LSE, BF16_O, DEV, GRAD, beyond_rounding, dev, grad_errors, half_ulp_bf16, host

pytestmark = pytest.mark.gpu

ROWS = [0, 1, 127, 128, 1000, 2047, 2048, 3071, 4095]


def _bench_qkv(B, H, N, d, base):
    """The benchmark's inputs: inputs.random_tensor with seeds base, base + 1, base + 2."""
    return [inputs.random_tensor((B, H, N, d), base + i, "bf16") for i in range(3)]


def _rows_oracle(q, k, v, scale, vis, b, h, rows):
    """Oracle rows of one (b, h): the masked definition restricted to the sampled rows."""
    O, L = attn_fwd_masked(q[b:b + 1, h:h + 1, rows], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], scale,
                           vis[b:b + 1, h:h + 1, rows])
    return O[0, 0], L[0, 0]


@pytest.mark.parametrize("kind", ["blocksparse", "varlen"])
def test_masked_forward_bench_configs(kind):
    """bench.py time_masked_forward: B2 H32 N4096 d128 causal with a ~50% block map (diagonal on), or
    B8 H16 N4096 d128 causal with lengths uniform in [N/4, N] (seed 43)."""
    B, H, N, d = (2, 32, 4096, 128) if kind == "blocksparse" else (8, 16, 4096, 128)
    q, k, v = _bench_qkv(B, H, N, d, 41)
    rng = np.random.default_rng(43)
    nb = -(-N // 128)
    bmap = lens = None
    if kind == "blocksparse":
        bmap = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
        bmap[:, :, np.arange(nb), np.arange(nb)] = 1
    else:
        lens = rng.integers(N // 4, N + 1, size=B).astype(np.int32)
    tq, tk, tv = (dev(x, torch.bfloat16) for x in (q, k, v))
    sl = None if lens is None else torch.from_numpy(lens).to(DEV)
    bm = None if bmap is None else torch.from_numpy(bmap).to(DEV)
    o, lse = flash_attn_fwd_masked(tq, tk, tv, None, True, seqlens=sl, block_mask=bm)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (B // 2, 3)):
        # the visibility of this (b, h) only (the whole batch's would be B*H*N*N bytes)
        vis = padded_batch_visible(1, 1, N, True, None if lens is None else [int(lens[b])],
                                   None if bmap is None else bmap[b:b + 1, h:h + 1], 128)
        O, L = _rows_oracle(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], d ** -0.5, vis, 0, 0,
                            ROWS)
        go, gl = host(o[b, h, ROWS]), host(lse[b, h, ROWS])
        full = np.isfinite(L)
        assert (go[~full] == 0).all() and np.isneginf(gl[~full]).all()
        assert np.abs(go[full] - O[full]).max(initial=0) <= BF16_O
        assert np.abs(gl[full] - L[full]).max(initial=0) <= BF16_LSE


def test_dropout_step_bench_config():
    """bench.py time_dropout_step: B4 H16 N2048 d64 causal, p = 0.1, inputs seeds 51..54; the keep
    mask of the timed seeds, and forward rows plus full gradients of two heads."""
    B, H, N, d, p, seed = 4, 16, 2048, 64, 0.1, 100
    q, k, v, do = (inputs.random_tensor((B, H, N, d), 51 + i, "bf16") for i in range(4))
    tq, tk, tv, tdo = (dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = flash_attn_fwd_masked(tq, tk, tv, None, True, dropout_p=p, seed=seed)
    dq, dk, dv = flash_attn_bwd_masked(tdo, tq, tk, tv, o, lse, None, True, dropout_p=p, seed=seed)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 15)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        vis = padded_batch_visible(1, 1, N, True, None)
        keep = (random_bytes(B, H, N, N, seed, heads=[b * H + h]) < keep_threshold(p))[None]
        O, L = attn_fwd_dropout(q[sl], k[sl], v[sl], d ** -0.5, vis, keep, p)
        assert beyond_rounding(host(o[sl]), O) <= BF16_O
        assert np.abs(host(lse[sl]) - L).max() <= BF16_LSE
        from oracle import attn_bwd_dropout
        ref = attn_bwd_dropout(q[sl], k[sl], v[sl], do[sl], d ** -0.5, vis, keep, p)
        for name, g, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref[:3]):
            e_inf, e_fro = grad_errors(host(g[sl]), r)
            assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)


def test_decode_bench_config():
    """bench.py time_decode: B8 H32, one query against 8192 keys, d128, auto split count, seeds 31..33."""
    B, H, Nk, d = 8, 32, 8192, 128
    q = inputs.random_tensor((B, H, 1, d), 31, "bf16")
    k = inputs.random_tensor((B, H, Nk, d), 32, "bf16")
    v = inputs.random_tensor((B, H, Nk, d), 33, "bf16")
    o, lse = flash_attn_fwd_kvsplit(*(dev(x, torch.bfloat16) for x in (q, k, v)), None, False, 0)
    torch.cuda.synchronize()
    O, L = attn_fwd_kv(q, k, v, d ** -0.5, False)
    assert np.abs(host(o) - O).max() <= BF16_O
    assert np.abs(host(lse) - L).max() <= BF16_LSE


@pytest.mark.parametrize("p", [0.998, 1.0 / 512, 0.0039])
def test_dropout_threshold_extremes(p):
    """T = 1 (keep 1/256, weights x256), T = 256 (p rounds to 0: no dropout) and T = 255.

    O is checked on the scale of the kept weights: dividing O by 256 / T gives sum over kept keys of
    (P_ij) V_j, a sub-convex combination of V rows like an undropped output, and the error beyond
    the rounding of the stored output, measured on that scale, is held to the bf16 O gate. The kept
    weights themselves are checked exactly by a run with V = 1: every column of O is then
    (256 / T) * (sum of the kept probabilities of the row)."""
    B, H, N, d = 1, 2, 300, 64
    x = {n: inputs.random_tensor((B, H, N, d), 60 + i, "bf16") for i, n in enumerate(("q", "k", "v", "do"))}
    tq, tk, tv, tdo = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    got_keep = flash_attn_dropout_mask(B, H, N, N, p, 7, device=DEV).cpu().numpy().astype(bool)
    keep = keep_mask(B, H, N, N, p, 7)
    np.testing.assert_array_equal(got_keep, keep)
    o, lse = flash_attn_fwd_masked(tq, tk, tv, None, False, dropout_p=p, seed=7)
    g = flash_attn_bwd_masked(tdo, tq, tk, tv, o, lse, None, False, dropout_p=p, seed=7)
    torch.cuda.synchronize()
    vis = padded_batch_visible(B, H, N, False, None)
    O, L = attn_fwd_dropout(x["q"], x["k"], x["v"], d ** -0.5, vis, keep, p)
    T = keep_threshold(p)
    go = host(o)
    err_scaled = float(np.max(np.abs(go - O) - half_ulp_bf16(O))) * T / 256
    print(f"p={p} T={T}: O error beyond output rounding, on the kept-weight scale {err_scaled:.3e}")
    assert err_scaled <= BF16_O
    assert np.abs(host(lse) - L).max() <= BF16_LSE
    # kept-weight sums: V = 1 makes every output column (256 / T) * sum_j keep_ij P_ij
    ones = torch.ones_like(tv)
    o1, _ = flash_attn_fwd_masked(tq, tk, ones, None, False, dropout_p=p, seed=7)
    torch.cuda.synchronize()
    O1, _ = attn_fwd_dropout(x["q"], x["k"], np.ones_like(x["v"]), d ** -0.5, vis, keep, p)
    g1 = host(o1) * T / 256
    r1 = O1 * T / 256
    assert (r1 >= 0).all() and (r1 <= 1 + 1e-12).all()
    # each kept weight P_ij / l carries the bf16 rounding of P_ij (2^-9 relative) and of the
    # normaliser's terms (at most 2^-9 relative), and the stored output one more rounding (2^-9 of a
    # value <= 1): at most 3 * 2^-9 in all
    err1 = np.abs(g1 - r1).max()
    print(f"kept-weight sum error {err1:.3e}")
    assert err1 <= 3 * 2.0 ** -9, err1
    assert np.array_equal(g1 == 0, r1 == 0)  # rows with no kept key are exactly zero
    from oracle import attn_bwd_dropout
    ref = attn_bwd_dropout(x["q"], x["k"], x["v"], x["do"], d ** -0.5, vis, keep, p)
    for name, gg, r in zip(("dQ", "dK", "dV"), g, ref[:3]):
        e_inf, e_fro = grad_errors(host(gg), r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)
