"""CPU pins of the masked-attention oracle (padding / variable length, key-value cache lengths,
block-sparse maps) against facts that do not come from its own code: torch's float64
scaled_dot_product_attention under the same boolean mask, truncation to the valid part of each
sequence (the unmasked oracle, itself pinned), independence from padding contents, block-diagonal
maps as independent attentions, brute-force loops, finite differences. Planted mistakes in copies
of the mask builders, on the CPU, must fail at least one pin."""
import math

import numpy as np
import pytest

from oracle import attn_bwd, attn_fwd, attn_fwd_kv
from oracle import masked as om

RNG = np.random.default_rng


def _qkv(B, H, N, d, seed, Nk=None):
    r = RNG(seed)
    Nk = N if Nk is None else Nk
    return r.standard_normal((B, H, N, d)), r.standard_normal((B, H, Nk, d)), r.standard_normal((B, H, Nk, d))


def _random_block_mask(B, H, nb, seed, density=0.5):
    return (RNG(seed).random((B, H, nb, nb)) < density).astype(np.uint8)


# ---------------------------------------------------------------------------------------------
# pins, each taking the mask builder and the attention functions under test
# ---------------------------------------------------------------------------------------------
def pin_torch_sdpa(padded, fwd):
    """torch float64 SDPA with the same boolean mask on the rows that see a key; empty rows are
    O = 0, LSE = -inf; LSE equals torch.logsumexp of the masked scores."""
    import torch

    B, H, N, d, blk = 2, 3, 37, 5, 8
    q, k, v = _qkv(B, H, N, d, 1)
    seqlens = np.array([37, 20])
    bm = _random_block_mask(B, H, -(-N // blk), 2)
    for causal in (False, True):
        vis = padded(B, H, N, causal, seqlens, bm, blk)
        O, L = fwd(q, k, v, 0.6, vis)
        tq, tk, tv, tm = (torch.tensor(x) for x in (q, k, v, vis))
        s = (0.6 * (tq @ tk.transpose(-1, -2))).masked_fill(~tm, float("-inf"))
        ref_L = torch.logsumexp(s, dim=-1).numpy()
        ref_O = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=0.6).numpy()
        # expected visibility written out per element (independent of the builder)
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        for b in range(B):
            for h in range(H):
                exp_vis = (i < seqlens[b]) & (j < seqlens[b]) & (bm[b, h][i // blk, j // blk] != 0)
                if causal:
                    exp_vis &= j <= i
                np.testing.assert_array_equal(vis[b, h], exp_vis)
                full = exp_vis.any(axis=1)
                np.testing.assert_allclose(O[b, h, full], ref_O[b, h, full], atol=1e-12)
                np.testing.assert_allclose(L[b, h, full], ref_L[b, h, full], atol=1e-12)
                assert (O[b, h, ~full] == 0).all() and np.isneginf(L[b, h, ~full]).all()


def pin_truncation(padded, fwd):
    """Padded batch: the valid rows of sequence b equal plain attention over its first L_b rows;
    the padding rows are 0 / -inf."""
    B, H, N, d = 3, 2, 29, 4
    q, k, v = _qkv(B, H, N, d, 3)
    seqlens = np.array([29, 11, 1])
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.9, padded(B, H, N, causal, seqlens))
        for b, Lb in enumerate(seqlens):
            Ot, Lt = attn_fwd(q[b:b + 1, :, :Lb], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], 0.9, causal)
            np.testing.assert_allclose(O[b, :, :Lb], Ot[0], atol=1e-13)
            np.testing.assert_allclose(L[b, :, :Lb], Lt[0], atol=1e-13)
            assert (O[b, :, Lb:] == 0).all() and np.isneginf(L[b, :, Lb:]).all()


def pin_padding_contents_ignored(padded, fwd):
    B, H, N, d = 2, 2, 23, 4
    q, k, v = _qkv(B, H, N, d, 4)
    seqlens = np.array([15, 9])
    vis = padded(B, H, N, True, seqlens)
    O1, L1 = fwd(q, k, v, 0.5, vis)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for b, Lb in enumerate(seqlens):
        for x in (q2, k2, v2):
            x[b, :, Lb:] = 1e3 * RNG(5).standard_normal(x[b, :, Lb:].shape)
    O2, L2 = fwd(q2, k2, v2, 0.5, vis)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(L1, L2)


def pin_block_diagonal(padded, fwd):
    """A block-diagonal map makes each block of rows attend only to its own block of keys: the same
    as independent attention on each slice (also under the causal mask and a ragged last block)."""
    B, H, N, d, blk = 1, 2, 21, 3, 8
    q, k, v = _qkv(B, H, N, d, 6)
    nb = -(-N // blk)
    bm = np.broadcast_to(np.eye(nb, dtype=np.uint8), (B, H, nb, nb))
    for causal in (False, True):
        O, L = fwd(q, k, v, 1.1, padded(B, H, N, causal, None, bm, blk))
        for s in range(0, N, blk):
            e = min(N, s + blk)
            Ot, Lt = attn_fwd(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], 1.1, causal)
            np.testing.assert_allclose(O[:, :, s:e], Ot, atol=1e-13)
            np.testing.assert_allclose(L[:, :, s:e], Lt, atol=1e-13)


def pin_block_map_all_ones_and_empty_rows(padded, fwd):
    B, H, N, d, blk = 1, 1, 19, 3, 4
    q, k, v = _qkv(B, H, N, d, 7)
    nb = -(-N // blk)
    ones = np.ones((B, H, nb, nb), dtype=np.uint8)
    O, L = fwd(q, k, v, 0.7, padded(B, H, N, False, None, ones, blk))
    Od, Ld = attn_fwd(q, k, v, 0.7, False)
    np.testing.assert_allclose(O, Od, atol=1e-13)
    np.testing.assert_allclose(L, Ld, atol=1e-13)
    # query block 2 sees nothing (its whole map row is zero); block 0 sees only key block 3,
    # so under the causal mask its rows see nothing either
    bm = ones.copy()
    bm[0, 0, 2, :] = 0
    bm[0, 0, 0, :] = 0
    bm[0, 0, 0, 3] = 1
    O, L = fwd(q, k, v, 0.7, padded(B, H, N, True, None, bm, blk))
    for r in list(range(0, 4)) + list(range(8, 12)):
        assert (O[0, 0, r] == 0).all() and np.isneginf(L[0, 0, r])
    assert np.isfinite(L[0, 0, 4:8]).all() and np.isfinite(L[0, 0, 12:]).all()


def pin_brute_force(padded, fwd):
    """math.fsum loops over the visible keys of a random element-wise mask."""
    B, H, N, d = 1, 2, 7, 3
    q, k, v = _qkv(B, H, N, d, 8)
    vis = RNG(9).random((B, H, N, N)) < 0.5
    vis[0, 0, 3] = False  # one empty row
    O, L = fwd(q, k, v, 0.8, vis)
    for h in range(H):
        for i in range(N):
            keys = [j for j in range(N) if vis[0, h, i, j]]
            if not keys:
                assert (O[0, h, i] == 0).all() and L[0, h, i] == -math.inf
                continue
            s = {j: 0.8 * math.fsum(q[0, h, i, c] * k[0, h, j, c] for c in range(d)) for j in keys}
            lse = max(s.values()) + math.log(math.fsum(math.exp(s[j] - max(s.values())) for j in keys))
            assert abs(L[0, h, i] - lse) < 1e-13
            for c in range(d):
                assert abs(O[0, h, i, c] - math.fsum(math.exp(s[j] - lse) * v[0, h, j, c] for j in keys)) < 1e-13


def pin_kv_cache_lengths(kvvis, fwd):
    """Per-sequence cache length L_b: sequence b's result is the unpadded key/value problem over its
    first L_b keys (the pinned attn_fwd_kv, bottom-right causal); keys beyond L_b do not matter."""
    B, H, Nq, Nk, d = 3, 2, 4, 30, 5
    q, k, v = _qkv(B, H, Nq, d, 10, Nk=Nk)
    Ls = np.array([30, 17, 4])
    for causal in (False, True):
        O, L = fwd(q, k, v, 0.4, kvvis(B, H, Nq, Nk, causal, Ls))
        for b, Lb in enumerate(Ls):
            Ot, Lt = attn_fwd_kv(q[b:b + 1], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], 0.4, causal)
            np.testing.assert_allclose(O[b], Ot[0], atol=1e-13)
            np.testing.assert_allclose(L[b], Lt[0], atol=1e-13)
    # a cache shorter than the query count: under the causal mask the first Nq - L_b queries see
    # nothing
    O, L = fwd(q, k, v, 0.4, kvvis(B, H, Nq, Nk, True, np.array([2, 3, 30])))
    assert (O[0, :, :2] == 0).all() and np.isneginf(L[0, :, :2]).all() and np.isfinite(L[0, :, 2:]).all()
    assert (O[1, :, :1] == 0).all() and np.isneginf(L[1, :, :1]).all() and np.isfinite(L[1, :, 1:]).all()


PADDED_PINS = [pin_torch_sdpa, pin_truncation, pin_padding_contents_ignored, pin_block_diagonal,
               pin_block_map_all_ones_and_empty_rows]


@pytest.mark.parametrize("pin", PADDED_PINS, ids=lambda f: f.__name__)
def test_padded_pin(pin):
    pin(om.padded_batch_visible, om.attn_fwd_masked)


def test_brute_force_pin():
    pin_brute_force(None, om.attn_fwd_masked)


def test_kv_cache_pin():
    pin_kv_cache_lengths(om.kv_cache_visible, om.attn_fwd_masked)


def test_row_restricted_visibility_is_a_slice():
    """The builder's `rows` option (used where the full N x N array is too large) returns exactly
    those rows of the full array, and the masked forward and dQ of those rows alone equal the
    full results' rows."""
    B, H, N, d = 2, 2, 300, 8
    q, k, v = _qkv(B, H, N, d, 80)
    do = RNG(81).standard_normal((B, H, N, d))
    bm = _random_block_mask(B, H, 3, 82, 0.6)
    rows = [0, 1, 127, 128, 200, 255, 256, 299]
    for causal in (False, True):
        for seqlens, bmap in ((None, None), ([300, 130], None), (None, bm), ([255, 299], bm)):
            full = om.padded_batch_visible(B, H, N, causal, seqlens, bmap)
            part = om.padded_batch_visible(B, H, N, causal, seqlens, bmap, rows=rows)
            np.testing.assert_array_equal(part, full[:, :, rows])
            O, L = om.attn_fwd_masked(q, k, v, 0.4, full)
            Or, Lr = om.attn_fwd_masked(q[:, :, rows], k, v, 0.4, part)
            np.testing.assert_allclose(Or, O[:, :, rows], rtol=0, atol=1e-13)  # BLAS order only
            np.testing.assert_allclose(Lr, L[:, :, rows], rtol=0, atol=1e-13)
            dQ = om.attn_bwd_masked(q, k, v, do, 0.4, full)[0]
            dQr = om.attn_bwd_masked(q[:, :, rows], k, v, do[:, :, rows], 0.4, part)[0]
            np.testing.assert_allclose(dQr, dQ[:, :, rows], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------------------------
def test_masked_backward_finite_differences():
    """Every input element of a tiny problem with padding, a sparse map, the causal mask and an
    empty row, against central differences of sum(O * dO)."""
    B, H, N, d, blk = 1, 1, 7, 2, 2
    q, k, v = _qkv(B, H, N, d, 11)
    do = RNG(12).standard_normal((B, H, N, d))
    bm = np.ones((1, 1, 4, 4), dtype=np.uint8)
    bm[0, 0, 1, 0] = 0
    bm[0, 0, 1, 1] = 0  # rows 2, 3 see nothing under the causal mask
    vis = om.padded_batch_visible(B, H, N, True, np.array([6]), bm, blk)
    assert not vis[0, 0, 2].any() and not vis[0, 0, 3].any()
    dQ, dK, dV, D = om.attn_bwd_masked(q, k, v, do, 0.9, vis)
    loss = lambda q_, k_, v_: float(np.sum(om.attn_fwd_masked(q_, k_, v_, 0.9, vis)[0] * do))
    eps = 1e-6
    for X, G, name in ((q, dQ, "q"), (k, dK, "k"), (v, dV, "v")):
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = {"q": (Xp, k, v), "k": (q, Xp, v), "v": (q, k, Xp)}[name]
            args_m = {"q": (Xm, k, v), "k": (q, Xm, v), "v": (q, k, Xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - G[idx]) < 1e-7, (name, idx, fd, G[idx])
    assert (dQ[0, 0, 2:4] == 0).all() and (dQ[0, 0, 6] == 0).all() and (dK[0, 0, 6] == 0).all() and (dV[0, 0, 6] == 0).all()
    np.testing.assert_allclose(D, np.sum(do * om.attn_fwd_masked(q, k, v, 0.9, vis)[0], axis=-1), atol=1e-13)


def test_masked_backward_matches_torch_autograd_and_truncation():
    import torch

    B, H, N, d, blk = 2, 2, 26, 4, 8
    q, k, v = _qkv(B, H, N, d, 13)
    do = RNG(14).standard_normal((B, H, N, d))
    seqlens = np.array([26, 13])
    bm = _random_block_mask(B, H, 4, 15, density=0.7)
    bm[:, :, np.arange(4), np.arange(4)] = 1  # every row sees its own block
    vis = om.padded_batch_visible(B, H, N, True, seqlens, bm, blk)
    dQ, dK, dV, _ = om.attn_bwd_masked(q, k, v, do, 0.6, vis)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.tensor(vis), scale=0.6)
    valid = torch.tensor(vis.any(axis=-1))[..., None]
    (torch.where(valid, out, 0.0) * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)
    # padding only (no map): sequence b's gradients are the unpadded ones over its first L_b rows
    vis = om.padded_batch_visible(B, H, N, False, seqlens)
    dQ, dK, dV, _ = om.attn_bwd_masked(q, k, v, do, 0.6, vis)
    b, Lb = 1, 13
    g = attn_bwd(q[b:b + 1, :, :Lb], k[b:b + 1, :, :Lb], v[b:b + 1, :, :Lb], do[b:b + 1, :, :Lb], 0.6, False)
    for got, ref in zip((dQ, dK, dV), g[:3]):
        np.testing.assert_allclose(got[b, :, :Lb], ref[0], atol=1e-13)
        assert (got[b, :, Lb:] == 0).all()


# ---------------------------------------------------------------------------------------------
# planted mistakes in the mask builders (CPU only)
# ---------------------------------------------------------------------------------------------
def _padded_mutant(kind):
    def build(B, H, N, causal, seqlens=None, block_mask=None, block=om.BLOCK):
        i = np.arange(N)[:, None]
        j = np.arange(N)[None, :]
        vis = np.ones((B, H, N, N), dtype=bool)
        if causal:
            vis &= ((j < i) if kind == "causal_strict" else (j <= i))[None, None]
        if seqlens is not None:
            L = np.asarray(seqlens).reshape(B, 1, 1, 1)
            if kind == "lengths_keys_only":
                vis &= j[None, None] < L
            elif kind == "lengths_off_by_one":
                vis &= (i[None, None] <= L) & (j[None, None] <= L)
            else:
                vis &= (i[None, None] < L) & (j[None, None] < L)
        if block_mask is not None:
            bm = np.asarray(block_mask) != 0
            if kind == "block_map_transposed":
                vis &= bm[:, :, j // block, i // block]
            elif kind == "block_index_by_row_only":
                vis &= bm[:, :, i // block, i // block]
            else:
                vis &= bm[:, :, i // block, j // block]
        return vis
    return build


def _fwd_mutant(kind):
    def fwd(q, k, v, scale, visible):
        if kind == "empty_rows_mean":  # empty rows fall back to uniform attention
            visible = np.where(visible.any(axis=-1, keepdims=True), visible, True)
        return om.attn_fwd_masked(q, k, v, scale, visible)
    return fwd


def _kv_mutant(kind):
    def build(B, H, Nq, Nk, causal, seqlens_k=None):
        L = (np.full(B, Nk) if seqlens_k is None else np.asarray(seqlens_k)).reshape(B, 1, 1, 1)
        i = np.arange(Nq)[None, None, :, None]
        j = np.arange(Nk)[None, None, None, :]
        vis = j < L
        if causal:
            vis = vis & ((j <= i + Nk - Nq) if kind == "align_to_capacity" else (j <= i + L - Nq + 1))
        return np.broadcast_to(vis, (B, H, Nq, Nk)).copy()
    return build


@pytest.mark.parametrize("kind", ["causal_strict", "lengths_keys_only", "lengths_off_by_one", "block_map_transposed",
                                  "block_index_by_row_only"])
def test_padded_mutant_is_caught(kind):
    caught = 0
    for pin in PADDED_PINS:
        try:
            pin(_padded_mutant(kind), om.attn_fwd_masked)
        except AssertionError:
            caught += 1
    assert caught >= 1, kind


def test_empty_row_mutant_is_caught():
    with pytest.raises(AssertionError):
        pin_brute_force(None, _fwd_mutant("empty_rows_mean"))
    with pytest.raises(AssertionError):
        pin_block_map_all_ones_and_empty_rows(om.padded_batch_visible, _fwd_mutant("empty_rows_mean"))


@pytest.mark.parametrize("kind", ["align_to_capacity", "diagonal_shifted"])
def test_kv_mutant_is_caught(kind):
    with pytest.raises(AssertionError):
        pin_kv_cache_lengths(_kv_mutant(kind), om.attn_fwd_masked)
