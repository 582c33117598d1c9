"""CPU pins of the dropout oracle: the Philox4x32-10 generator against the authors' published
known-answer vectors, the element -> (counter, word, byte) contract against a scalar pure-Python
statement of it, keep-rate and byte-uniformity statistics, and attention with dropout against
torch float64 autograd and finite differences with the same keep mask."""
import math

import numpy as np
import pytest

from oracle import attn_fwd_masked, padded_batch_visible
from oracle import dropout as od

RNG = np.random.default_rng

# Known-answer vectors of Philox4x32-10 published with the Random123 library by the generator's
# authors (Salmon, Moraes, Dror, Shaw): (counter, key) -> output, 32-bit words.
KAT = [
    ((0x00000000, 0x00000000, 0x00000000, 0x00000000), (0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("ctr,key,out", KAT)
def test_philox_known_answers(ctr, key, out):
    got = od.philox4x32_10(np.array([ctr], dtype=np.uint64), key)[0]
    assert [int(x) for x in got] == list(out)


def _scalar_philox(ctr, key):
    """The same generator on Python ints, one round at a time (a second statement)."""
    c = list(ctr)
    k0, k1 = key
    for _ in range(10):
        p0, p1 = 0xD2511F53 * c[0], 0xCD9E8D57 * c[2]
        c = [((p1 >> 32) ^ c[1] ^ k0) & 0xFFFFFFFF, p1 & 0xFFFFFFFF, ((p0 >> 32) ^ c[3] ^ k1) & 0xFFFFFFFF,
             p0 & 0xFFFFFFFF]
        k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return c


def test_scalar_statement_agrees_with_known_answers():
    for ctr, key, out in KAT:
        assert _scalar_philox(ctr, key) == list(out)


def test_random_bytes_follow_the_element_contract():
    """Every element's byte, recomputed one element at a time from the contract's wording."""
    B, H, Nq, Nk, seed = 2, 3, 5, 77, 0x1234_5678_9ABC_DEF0
    got = od.random_bytes(B, H, Nq, Nk, seed)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                for j in range(Nk):
                    words = _scalar_philox((i, j // 32, b * H + h, (j // 4) % 2), key)
                    byte = (words[(j % 32) // 8] >> (8 * (j % 4))) & 0xFF
                    assert got[b, h, i, j] == byte, (b, h, i, j)


def test_threshold_and_keep_rate():
    assert od.keep_threshold(0.0) == 256 and od.keep_threshold(0.1) == 230 and od.keep_threshold(0.5) == 128
    for p in (0.1, 0.3, 0.5, 0.9):
        keep = od.keep_mask(2, 4, 64, 512, p, seed=7)
        rate, n = keep.mean(), keep.size
        expect = od.keep_threshold(p) / 256.0
        assert abs(rate - expect) < 5 * math.sqrt(expect * (1 - expect) / n), (p, rate, expect)
    assert od.keep_mask(1, 1, 8, 64, 0.0, seed=3).all()


def test_bytes_are_uniform_and_seed_dependent():
    by = od.random_bytes(2, 2, 64, 1024, seed=11).ravel()
    counts = np.bincount(by, minlength=256)
    e = by.size / 256
    chi2 = float(((counts - e) ** 2 / e).sum())
    assert chi2 < 255 + 6 * math.sqrt(2 * 255), chi2   # 255 degrees of freedom
    other = od.random_bytes(2, 2, 64, 1024, seed=12).ravel()
    assert (by == other).mean() < 0.01                 # ~1/256 coincide by chance


def test_p_zero_is_attention_without_dropout():
    B, H, N, d = 2, 2, 40, 8
    q, k, v = (RNG(s).standard_normal((B, H, N, d)) for s in (1, 2, 3))
    vis = padded_batch_visible(B, H, N, True, [40, 23])
    O, L = od.attn_fwd_dropout(q, k, v, 0.3, vis, od.keep_mask(B, H, N, N, 0.0, 5), 0.0)
    Om, Lm = attn_fwd_masked(q, k, v, 0.3, vis)
    np.testing.assert_allclose(O, Om, atol=1e-14)
    np.testing.assert_array_equal(L, Lm)


def test_dropout_forward_and_backward_match_torch_autograd():
    import torch

    B, H, N, d, p = 2, 2, 45, 6, 0.3
    q, k, v, do = (RNG(s).standard_normal((B, H, N, d)) for s in (4, 5, 6, 7))
    vis = padded_batch_visible(B, H, N, True, [45, 30])
    keep = od.keep_mask(B, H, N, N, p, seed=99)
    O, L = od.attn_fwd_dropout(q, k, v, 0.4, vis, keep, p)
    dQ, dK, dV, D = od.attn_bwd_dropout(q, k, v, do, 0.4, vis, keep, p)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = (0.4 * tq @ tk.transpose(-1, -2)).masked_fill(~torch.tensor(vis), float("-inf"))
    rows = torch.tensor(vis.any(-1))[..., None]
    P = torch.where(rows, torch.softmax(torch.where(rows, s, 0.0), dim=-1), 0.0)
    out = (P * torch.tensor(keep) * (256.0 / od.keep_threshold(p))) @ tv
    (out * torch.tensor(do)).sum().backward()
    np.testing.assert_allclose(O, out.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(dQ, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV, tv.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(D, np.sum(do * O, axis=-1), atol=1e-12)
    fin = np.isfinite(L)
    np.testing.assert_allclose(L[fin], torch.logsumexp(s, -1).detach().numpy()[fin], atol=1e-12)


def test_dropout_backward_finite_differences():
    B, H, N, d, p = 1, 1, 6, 2, 0.5
    q, k, v, do = (RNG(s).standard_normal((B, H, N, d)) for s in (8, 9, 10, 11))
    vis = padded_batch_visible(B, H, N, False, None)
    keep = od.keep_mask(B, H, N, N, p, seed=1)
    assert 0 < keep.mean() < 1
    dQ, dK, dV, _ = od.attn_bwd_dropout(q, k, v, do, 0.8, vis, keep, p)
    loss = lambda a, b_, c: float(np.sum(od.attn_fwd_dropout(a, b_, c, 0.8, vis, keep, p)[0] * do))
    eps = 1e-6
    for X, G, pos in ((q, dQ, 0), (k, dK, 1), (v, dV, 2)):
        for idx in np.ndindex(X.shape):
            args_p, args_m = [q, k, v], [q, k, v]
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p[pos], args_m[pos] = Xp, Xm
            assert abs((loss(*args_p) - loss(*args_m)) / (2 * eps) - G[idx]) < 1e-7


def test_dropout_is_unbiased_on_average():
    """Averaged over seeds, the dropped output approaches the undropped one (the 256 / T scale)."""
    B, H, N, d, p = 1, 1, 16, 4, 0.4
    q, k, v = (RNG(s).standard_normal((B, H, N, d)) for s in (12, 13, 14))
    vis = padded_batch_visible(B, H, N, False, None)
    ref, _ = attn_fwd_masked(q, k, v, 0.5, vis)
    acc = np.zeros_like(ref)
    n = 400
    for s in range(n):
        acc += od.attn_fwd_dropout(q, k, v, 0.5, vis, od.keep_mask(B, H, N, N, p, seed=1000 + s), p)[0]
    assert np.abs(acc / n - ref).max() < 0.1


def test_planted_generator_mistakes_are_caught():
    """A round short, swapped multipliers, or the key not advanced: the known answers fail."""
    def variant(kind):
        def f(ctr, key):
            c = list(ctr)
            k0, k1 = key
            m0, m1 = (0xCD9E8D57, 0xD2511F53) if kind == "swapped" else (0xD2511F53, 0xCD9E8D57)
            for _ in range(9 if kind == "nine_rounds" else 10):
                p0, p1 = m0 * c[0], m1 * c[2]
                c = [((p1 >> 32) ^ c[1] ^ k0) & 0xFFFFFFFF, p1 & 0xFFFFFFFF, ((p0 >> 32) ^ c[3] ^ k1) & 0xFFFFFFFF,
                     p0 & 0xFFFFFFFF]
                if kind != "fixed_key":
                    k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
            return c
        return f
    for kind in ("nine_rounds", "swapped", "fixed_key"):
        f = variant(kind)
        assert any(f(c, k) != list(o) for c, k, o in KAT), kind


def test_head_subset_equals_slice_of_full():
    full = od.random_bytes(2, 3, 9, 70, seed=5)
    sub = od.random_bytes(2, 3, 9, 70, seed=5, heads=[0, 4, 5])
    np.testing.assert_array_equal(sub, full.reshape(6, 9, 70)[[0, 4, 5]])
