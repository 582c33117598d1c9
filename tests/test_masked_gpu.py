"""GPU parity of the masked paths (padding / variable length, block-sparse maps, per-sequence cache
lengths) against the float64 masked oracle, through the C ABI.

Gates are the dense path's (O <= 1e-2, LSE <= 1e-3 max-abs on rows that see a key; gradients
<= 5e-2 relative to their norm). Rows that see no key must be exactly O = 0, LSE = -inf, and
their gradients exactly 0. With every block enabled and full lengths the masked kernels walk the
same tiles in the same order as the dense ones, so their results must be bitwise identical.
"""
import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd, flash_attn_bwd_masked, flash_attn_fwd,
                                               flash_attn_fwd_kvsplit, flash_attn_fwd_masked, inputs)
from oracle import attn_bwd_masked, attn_fwd_masked, kv_cache_visible, padded_batch_visible
from tests.test_parity_gpu import BF16_LSE, BF16_O, DEV, GRAD, beyond_rounding, dev, grad_errors, host

pytestmark = pytest.mark.gpu

BLK = 128


def _inputs(B, H, N, d, seed, dtype="bf16", with_do=False):
    names = ("q", "k", "v", "do") if with_do else ("q", "k", "v")
    return {n: inputs.random_tensor((B, H, N, d), seed + i, dtype) for i, n in enumerate(names)}


def _random_map(B, H, N, seed, density):
    nb = -(-N // BLK)
    return (np.random.default_rng(seed).random((B, H, nb, nb)) < density).astype(np.uint8)


def _fwd(x, scale, causal, seqlens, bmap, tdt=torch.bfloat16):
    q, k, v = (dev(x[n], tdt) for n in ("q", "k", "v"))
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    bm = None if bmap is None else torch.from_numpy(bmap).to(DEV)
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    o, lse = flash_attn_fwd_masked(q, k, v, scale, causal, seqlens=sl, block_mask=bm, out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def _check_fwd(o, lse, O, L, beyond_output_rounding=False):
    """Every row written (outputs start as NaN), rows that see no key exactly (0, -inf), the rest
    within the bf16 gates: plain max-abs O error, or with beyond_output_rounding the error beyond
    the rounding of the stored bf16 output (half an ulp is 0.0156 at |O| in [4, 8), above the
    1e-2 gate by itself; rows that see few keys reach such values)."""
    o, lse = host(o), host(lse)
    full = np.isfinite(L)
    assert np.isfinite(o).all()
    assert (o[~full] == 0).all() and np.isneginf(lse[~full]).all()
    err = np.abs(o[full] - O[full]).max(initial=0)
    if beyond_output_rounding:
        beyond = beyond_rounding(o[full], O[full]) if full.any() else 0.0
        print(f"O error {err:.3e}, beyond the output's rounding {beyond:.3e}")
        assert beyond <= BF16_O
    else:
        assert err <= BF16_O
    assert np.abs(lse[full] - L[full]).max(initial=0) <= BF16_LSE


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,seqlens", [(300, [300, 1, 0, 129]), (1000, [999, 640, 128, 257]), (77, [77, 50, 5, 0])])
def test_fwd_padded(N, seqlens, causal, d):
    B, H = len(seqlens), 2
    x = _inputs(B, H, N, d, seed=N + d)
    o, lse = _fwd(x, d ** -0.5, causal, seqlens, None)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], d ** -0.5, padded_batch_visible(B, H, N, causal, seqlens))
    _check_fwd(o, lse, O, L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,seqlens", [(300, [300, 1, 0, 129]), (1000, [999, 640, 0, 257, 1000, 128])])
def test_fwd_padded_eight_heads(N, seqlens, causal, d):
    """Eight heads per sequence: the launch runs the tiles with work before the padding tiles and
    has the tiles with work write the padding rows (O = 0, LSE = -inf). Outputs start as NaN, so a
    tile that no workgroup writes, or writes wrongly, fails."""
    B, H = len(seqlens), 8
    x = _inputs(B, H, N, d, seed=3 * N + d)
    o, lse = _fwd(x, d ** -0.5, causal, seqlens, None)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], d ** -0.5, padded_batch_visible(B, H, N, causal, seqlens))
    _check_fwd(o, lse, O, L, beyond_output_rounding=True)


def test_fwd_padded_eight_heads_with_block_map():
    """Lengths and a block map together, eight heads per sequence (a tile with work whose map row
    enables no key block still writes its share of the padding rows)."""
    B, H, N = 3, 8, 700
    seqlens = [700, 300, 0]
    bmap = _random_map(B, H, N, seed=21, density=0.3)
    x = _inputs(B, H, N, 128, seed=22)
    o, lse = _fwd(x, 128 ** -0.5, True, seqlens, bmap)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], 128 ** -0.5, padded_batch_visible(B, H, N, True, seqlens, bmap, BLK))
    _check_fwd(o, lse, O, L, beyond_output_rounding=True)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,N", [(64, 8, 100), (3, 16, 333), (2, 24, 257)])
def test_fwd_padded_head_layouts(B, H, N, causal):
    """The padding-last order at its limits: exactly 64 sequences (one per lane of a wave), 16 and
    24 heads per sequence; non-causal launches take its head-major branch. Lengths include 0 and N."""
    rng = np.random.default_rng(B * H + N)
    seqlens = [int(v) for v in rng.integers(0, N + 1, size=B)]
    seqlens[0], seqlens[-1] = N, 0
    x = _inputs(B, H, N, 64, seed=B + H + N)
    o, lse = _fwd(x, 0.125, causal, seqlens, None)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], 0.125, padded_batch_visible(B, H, N, causal, seqlens))
    _check_fwd(o, lse, O, L, beyond_output_rounding=True)


def test_fwd_padded_many_sequences():
    """65 sequences of eight heads (more than one wave's lanes): the launch keeps the plain tile
    order, still correct."""
    B, H, N = 65, 8, 130
    seqlens = [int(v) for v in np.random.default_rng(31).integers(0, N + 1, size=B)]
    x = _inputs(B, H, N, 64, seed=32)
    o, lse = _fwd(x, 0.125, True, seqlens, None)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], 0.125, padded_batch_visible(B, H, N, True, seqlens))
    _check_fwd(o, lse, O, L, beyond_output_rounding=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,density", [(700, 0.5), (1100, 0.3), (256, 0.0), (513, 0.8)])
def test_fwd_block_sparse(N, density, causal, d):
    B, H = 2, 2
    x = _inputs(B, H, N, d, seed=2 * N + d)
    bmap = _random_map(B, H, N, seed=N, density=density)
    if density > 0:
        bmap[0, 0, -1, :] = 0  # one query block with no enabled block at all
    seqlens = [N, N - 130] if N > 200 else None
    o, lse = _fwd(x, d ** -0.5, causal, seqlens, bmap)
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], d ** -0.5,
                           padded_batch_visible(B, H, N, causal, seqlens, bmap, BLK))
    _check_fwd(o, lse, O, L)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_forward_without_masks_is_the_dense_forward(causal, d):
    """All blocks enabled and full lengths: the same tiles in the same order, bitwise. (48 heads of
    8 query tiles: more tiles than CUs, so the dense forward takes its plain launch; smaller dense
    launches split each row's key loop over two wave pairs, which changes the summation order.)"""
    B, H, N = 2, 24, 900
    x = _inputs(B, H, N, d, seed=5)
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    ref = flash_attn_fwd(q, k, v, 0.1, causal)
    nb = -(-N // BLK)
    ones = torch.ones((B, H, nb, nb), dtype=torch.uint8, device=DEV)
    full = torch.full((B,), N, dtype=torch.int32, device=DEV)
    for sl, bm in ((None, None), (full, None), (None, ones), (full, ones)):
        got = flash_attn_fwd_masked(q, k, v, 0.1, causal, seqlens=sl, block_mask=bm)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])


def _bwd_case(B, H, N, d, causal, seqlens, bmap, seed, tdt=torch.bfloat16, dtype="bf16"):
    x = _inputs(B, H, N, d, seed=seed, dtype=dtype, with_do=True)
    q, k, v, do = (dev(x[n], tdt) for n in ("q", "k", "v", "do"))
    sl = None if seqlens is None else torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    bm = None if bmap is None else torch.from_numpy(bmap).to(DEV)
    scale = d ** -0.5
    o, lse = flash_attn_fwd_masked(q, k, v, scale, causal, seqlens=sl, block_mask=bm)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    flash_attn_bwd_masked(do, q, k, v, o, lse, scale, causal, seqlens=sl, block_mask=bm, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    vis = padded_batch_visible(B, H, N, causal, seqlens, bmap, BLK)
    dQ, dK, dV, _ = attn_bwd_masked(x["q"], x["k"], x["v"], x["do"], scale, vis)
    rows_seen = vis.any(axis=-1)   # queries that see a key
    keys_seen = vis.any(axis=-2)   # keys some query sees
    for name, g, r, live in (("dQ", dq, dQ, rows_seen), ("dK", dk, dK, keys_seen), ("dV", dv, dV, keys_seen)):
        g = host(g)
        assert np.isfinite(g).all(), name
        assert (g[~live] == 0).all(), name
        e_inf, e_fro = grad_errors(g, r)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,seqlens", [(300, [300, 1, 0, 129]), (640, [500, 640, 64, 200])])
def test_bwd_padded(N, seqlens, causal, d):
    _bwd_case(len(seqlens), 2, N, d, causal, seqlens, None, seed=7 * N + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,density,padded", [(700, 0.5, False), (1000, 0.4, True), (300, 0.0, False)])
def test_bwd_block_sparse(N, density, padded, causal, d):
    B, H = 2, 2
    bmap = _random_map(B, H, N, seed=N + 1, density=density)
    if density > 0:
        bmap[1, 0, 1, :] = 0  # a query block with nothing enabled
        bmap[0, 1, :, 2] = 0  # a key block no query sees
    _bwd_case(B, H, N, d, causal, [N - 37, N - 300] if padded else None, bmap, seed=N + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,seqlens", [(300, [300, 1, 0, 129]), (700, [700, 455, 0, 64, 699])])
def test_bwd_padded_eight_heads(N, seqlens, causal, d):
    """Eight heads per sequence: dQ and dK/dV run their padding tiles after every tile with work
    (gradients start as NaN, so a tile left unwritten fails)."""
    _bwd_case(len(seqlens), 8, N, d, causal, seqlens, None, seed=N + d + 7)


def test_bwd_padded_large_causal_launch():
    """B8 H16 N1024 d64 causal with lengths: a launch that large pairs dQ's tiles when it has no
    lengths; with them every tile runs on its own, padding tiles last. Every gradient is written
    (NaN-filled beforehand, exact zeros for rows and keys that see nothing); three heads are
    checked against the oracle."""
    B, H, N, d = 8, 16, 1024, 64
    seqlens = [int(v) for v in np.random.default_rng(8).integers(N // 4, N + 1, size=B)]
    seqlens[3] = 0
    x = _inputs(B, H, N, d, seed=81, with_do=True)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    scale = d ** -0.5
    o, lse = flash_attn_fwd_masked(q, k, v, scale, True, seqlens=sl)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    flash_attn_bwd_masked(do, q, k, v, o, lse, scale, True, seqlens=sl, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    gq, gk, gv = host(dq), host(dk), host(dv)
    assert np.isfinite(gq).all() and np.isfinite(gk).all() and np.isfinite(gv).all()
    for b in range(B):  # padding rows and keys of every sequence are exactly zero
        for g in (gq, gk, gv):
            assert (g[b, :, seqlens[b]:] == 0).all()
    for b, h in ((0, 0), (3, 5), (B - 1, H - 1)):
        sl_ = (slice(b, b + 1), slice(h, h + 1))
        vis = padded_batch_visible(1, 1, N, True, [seqlens[b]])
        ref = attn_bwd_masked(x["q"][sl_], x["k"][sl_], x["v"][sl_], x["do"][sl_], scale, vis)
        for name, g, r in (("dQ", gq, ref[0]), ("dK", gk, ref[1]), ("dV", gv, ref[2])):
            e_inf, e_fro = grad_errors(g[sl_], r)
            assert e_inf <= GRAD and e_fro <= GRAD, (name, b, h, e_inf, e_fro)


def test_bwd_masked_fp16():
    bmap = _random_map(2, 2, 600, seed=3, density=0.6)
    _bwd_case(2, 2, 600, 128, True, [600, 333], bmap, seed=11, tdt=torch.float16, dtype="fp16")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_backward_without_masks_is_the_dense_backward(causal, d):
    """All blocks enabled and full lengths give the dense backward's bits. (48 heads: enough
    workgroups that the dense dQ takes its plain launch; small dense launches split each row's key
    loop over two wave pairs, which changes the summation order.)"""
    B, H, N = 2, 24, 700
    x = _inputs(B, H, N, d, seed=9, with_do=True)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    o, lse = flash_attn_fwd(q, k, v, 0.1, causal)
    ref = flash_attn_bwd(do, q, k, v, o, lse, 0.1, causal)
    nb = -(-N // BLK)
    ones = torch.ones((B, H, nb, nb), dtype=torch.uint8, device=DEV)
    full = torch.full((B,), N, dtype=torch.int32, device=DEV)
    got = flash_attn_bwd_masked(do, q, k, v, o, lse, 0.1, causal, seqlens=full, block_mask=ones)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_masked_deterministic():
    B, H, N = 2, 4, 1500
    x = _inputs(B, H, N, 128, seed=12, with_do=True)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    sl = torch.tensor([1500, 777], dtype=torch.int32, device=DEV)
    bm = torch.from_numpy(_random_map(B, H, N, seed=4, density=0.5)).to(DEV)
    first = None
    for _ in range(3):
        o, lse = flash_attn_fwd_masked(q, k, v, 0.09, True, seqlens=sl, block_mask=bm)
        g = flash_attn_bwd_masked(do, q, k, v, o, lse, 0.09, True, seqlens=sl, block_mask=bm)
        torch.cuda.synchronize()
        cur = (o, lse) + tuple(g)
        if first is None:
            first = cur
        else:
            assert all(torch.equal(a, b) for a, b in zip(cur, first))


# ---------------------------------------------------------------------------------------------
# key-split forward with per-sequence cache lengths
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,lens,splits", [(1, 4097, [4097, 1, 0, 2000], 0), (1, 1000, [999, 64, 65, 500], 3),
                                               (200, 1000, [1000, 150, 200, 901], 0), (64, 640, [640, 0, 10, 300], 4),
                                               # one split: the workgroups write O and LSE themselves (no merge),
                                               # including rows before a short cache's first key and an empty cache
                                               (200, 1000, [1000, 150, 0, 901], 1), (1, 700, [700, 0, 1, 333], 1)])
def test_kvsplit_cache_lengths(Nq, Nk, lens, splits, causal, d):
    B, H = len(lens), 2
    x = {"q": inputs.random_tensor((B, H, Nq, d), Nq + d, "bf16"),
         "k": inputs.random_tensor((B, H, Nk, d), Nk + d, "bf16"),
         "v": inputs.random_tensor((B, H, Nk, d), Nk + d + 1, "bf16")}
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = flash_attn_fwd_kvsplit(q, k, v, d ** -0.5, causal, splits, out=o, lse=lse, seqlens_k=sl)
    torch.cuda.synchronize()
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], d ** -0.5, kv_cache_visible(B, H, Nq, Nk, causal, lens))
    _check_fwd(o, lse, O, L)


@pytest.mark.parametrize("d", [32, 96, 256])
def test_kvsplit_single_split_head_dims(d):
    """One split at every other head dim (d = 256 keeps the merge kernel; the others write O and LSE
    in the split kernel), causal, with cache lengths that leave some rows and one sequence empty."""
    B, H, Nq, Nk, lens = 3, 2, 130, 777, [777, 100, 0]
    x = {"q": inputs.random_tensor((B, H, Nq, d), 50 + d, "bf16"),
         "k": inputs.random_tensor((B, H, Nk, d), 51 + d, "bf16"),
         "v": inputs.random_tensor((B, H, Nk, d), 52 + d, "bf16")}
    q, k, v = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    o, lse = flash_attn_fwd_kvsplit(q, k, v, d ** -0.5, True, 1, out=o, lse=lse, seqlens_k=sl)
    torch.cuda.synchronize()
    O, L = attn_fwd_masked(x["q"], x["k"], x["v"], d ** -0.5, kv_cache_visible(B, H, Nq, Nk, True, lens))
    _check_fwd(o, lse, O, L, beyond_output_rounding=True)


def test_autograd_wrapper_routes_masks_and_dropout():
    """flash_attention(...) with lengths, a map and dropout: its gradients are the masked backward's
    with the same seed, and its output the masked forward's."""
    from io_aware_flashattention_flash_amd import flash_attention

    B, H, N, d = 2, 2, 500, 64
    x = _inputs(B, H, N, d, seed=21, with_do=True)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    sl = torch.tensor([500, 260], dtype=torch.int32, device=DEV)
    bm = torch.from_numpy(_random_map(B, H, N, seed=8, density=0.7)).to(DEV)
    qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
    out = flash_attention(qa, ka, va, 0.125, True, seqlens=sl, block_mask=bm, dropout_p=0.2, seed=99)
    out.backward(do)
    o, lse = flash_attn_fwd_masked(q, k, v, 0.125, True, seqlens=sl, block_mask=bm, dropout_p=0.2, seed=99)
    ref = flash_attn_bwd_masked(do, q, k, v, o, lse, 0.125, True, seqlens=sl, block_mask=bm, dropout_p=0.2, seed=99)
    torch.cuda.synchronize()
    assert torch.equal(out.detach(), o)
    for g, r in zip((qa.grad, ka.grad, va.grad), ref):
        assert torch.equal(g, r)


def test_block_map_at_capacity():
    """N = 131072: 1024 key blocks per map row, the most a map may hold. Causal, one full-length and
    one shorter sequence, a random map (30% of blocks) in which one head's last query tile has
    all 1024 blocks enabled and another head has an empty map row. The full N x N oracle is out of
    reach on the host, so it runs on sampled rows alone: O, LSE and dQ of query rows at the start,
    in the empty map row, around the shorter sequence's end and at the end; dK and dV of each
    sequence's last block of keys (and the padding keys after it), which under the causal mask only
    that sequence's last query block sees, so the oracle on those rows gives them exactly. Every
    output element must come back finite (they start as NaN)."""
    B, H, N, d = 2, 2, 131072, 64
    seqlens = [N, 100000]
    print(f"block map at capacity: B{B} H{H} N{N} d{d}, lengths {seqlens}", flush=True)
    bmap = _random_map(B, H, N, 950, 0.3)
    assert bmap.shape[-1] == 1024
    bmap[0, 0, -1, :] = 1  # head (0, 0): the last query tile walks every block
    bmap[0, 1, 5, :] = 0   # head (0, 1): rows 640..767 see no key
    x = _inputs(B, H, N, d, seed=951, with_do=True)
    scale = d ** -0.5
    o, lse = _fwd(x, scale, True, seqlens, bmap)
    q, k, v, do = (dev(x[n], torch.bfloat16) for n in ("q", "k", "v", "do"))
    sl = torch.tensor(seqlens, dtype=torch.int32, device=DEV)
    bm = torch.from_numpy(bmap).to(DEV)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    flash_attn_bwd_masked(do, q, k, v, o, lse, scale, True, seqlens=sl, block_mask=bm, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for name, t in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t).all()), name
    rows = [0, 1, 127, 128, 640, 700, 767, 50000, 99967, 99968, 99999, 100000, 100001, N - 129, N - 128, N - 1]
    vis = padded_batch_visible(B, H, N, True, seqlens, bmap, rows=rows)
    O, L = attn_fwd_masked(x["q"][:, :, rows], x["k"], x["v"], scale, vis)
    _check_fwd(o[:, :, rows], lse[:, :, rows], O, L, beyond_output_rounding=True)
    dQ = attn_bwd_masked(x["q"][:, :, rows], x["k"], x["v"], x["do"][:, :, rows], scale, vis)[0]
    g = host(dq[:, :, rows])
    seen = vis.any(axis=-1)
    assert (g[~seen] == 0).all()
    e_inf, e_fro = grad_errors(g, dQ)
    print(f"dQ rows: {e_inf:.2e} / {e_fro:.2e}")
    assert e_inf <= GRAD and e_fro <= GRAD
    for b, Lb in enumerate(seqlens):
        r0 = (Lb - 1) // BLK * BLK  # the last query block with valid rows; it alone sees keys >= r0
        R = np.arange(r0, Lb)
        vr = padded_batch_visible(B, H, N, True, seqlens, bmap, rows=R)
        _, dK, dV, _ = attn_bwd_masked(x["q"][:, :, R], x["k"], x["v"], x["do"][:, :, R], scale, vr)
        for name, t, ref in (("dK", dk, dK), ("dV", dv, dV)):
            gk = host(t[b, :, r0:])
            rk = ref[b, :, r0:]
            assert (gk[:, Lb - r0:] == 0).all(), (b, name)  # padding keys
            e_inf, e_fro = grad_errors(gk, rk)
            print(f"sequence {b} {name}, keys {r0}..{N - 1}: {e_inf:.2e} / {e_fro:.2e}")
            assert e_inf <= GRAD and e_fro <= GRAD, (b, name)
