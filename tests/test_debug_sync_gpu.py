"""Race guard: the library built with a full wait and a workgroup barrier after every pipeline stage
(libflashattn_debugsync.so, FA_DEBUG_SYNC) against the normal build, bit for bit.

The stages compute the same values in both builds; only the ordering guarantees differ. The normal
build overlaps each tile's load with the previous tile's compute behind one barrier per tile (the
double buffer whose reuse the yunthe.com kernel sketch, section 4, leaves unguarded). A missing
wait or barrier there would let a read see a half-written tile in the normal build only, and the
outputs would then differ from the fully synchronised build's."""
import contextlib
import ctypes
import os

import numpy as np
import pytest
import torch

from io_aware_flashattention_flash_amd import flash_attn as fa
from io_aware_flashattention_flash_amd import inputs
from io_aware_flashattention_flash_amd.build import DEBUGSYNC_LIB_PATH
from tests.test_parity_gpu import DEV, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def debug_lib():
    if not os.path.exists(DEBUGSYNC_LIB_PATH):
        raise RuntimeError(f"{DEBUGSYNC_LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(DEBUGSYNC_LIB_PATH)
    for name, (res, args) in fa.SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


@contextlib.contextmanager
def using(lib):
    """Route the binding's calls to `lib` (the binding keeps one library handle)."""
    saved = fa.load_library()
    fa._lib_handle = lib
    try:
        yield
    finally:
        fa._lib_handle = saved


def both(debug_lib, call):
    """call() with the normal build, then with the race-guard build; returns both results on the host."""
    a = call()
    with using(debug_lib):
        b = call()
    torch.cuda.synchronize()
    return [t.cpu() for t in a], [t.cpu() for t in b]


def assert_bitwise(a, b):
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.uint8) if x.dtype != torch.uint8 else x,
                           y.view(torch.uint8) if y.dtype != torch.uint8 else y), "builds differ"


def qkv(B, H, N, d, dtype, seed, do=False):
    w = inputs.Workload("t", dtype, B, H, N, d, True, do)
    x = inputs.make_inputs(w, seed=seed)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[dtype]
    return [dev(x[n], dt) for n in (("q", "k", "v", "do") if do else ("q", "k", "v"))]


@pytest.mark.parametrize("dtype,d,N,causal", [("bf16", 64, 1000, True), ("bf16", 128, 333, False),
                                              ("bf16", 128, 2048, True), ("fp16", 96, 700, True),
                                              ("bf16", 32, 513, False), ("bf16", 256, 300, True)])
def test_forward_and_backward_match_the_race_guard_build(debug_lib, dtype, d, N, causal):
    q, k, v, do = qkv(2, 8, N, d, dtype, seed=N + d, do=True)

    def run():
        o, lse = fa.flash_attn_fwd(q, k, v, None, causal)
        dq, dk, dv = fa.flash_attn_bwd(do, q, k, v, o, lse, None, causal)
        return o, lse, dq, dk, dv

    a, b = both(debug_lib, run)
    assert_bitwise(a, b)


@pytest.mark.parametrize("B,H,N", [(2, 16, 600), (1, 3, 300)])
def test_fp32_forward_matches_the_race_guard_build(debug_lib, B, H, N):
    q, k, v = qkv(B, H, N, 64, "fp32", seed=5)
    a, b = both(debug_lib, lambda: fa.flash_attn_fwd(q, k, v, None, True))
    assert_bitwise(a, b)


def test_masked_dropout_and_keysplit_match_the_race_guard_build(debug_lib):
    B, H, N, d = 2, 4, 900, 64
    q, k, v, do = qkv(B, H, N, d, "bf16", seed=77, do=True)
    lens = torch.tensor([900, 517], dtype=torch.int32, device=DEV)
    nb = -(-N // 128)
    bmap = (torch.rand(B, H, nb, nb, generator=torch.Generator().manual_seed(3)) < 0.6).to(torch.uint8)
    bmap[:, :, torch.arange(nb), torch.arange(nb)] = 1
    bmap = bmap.to(DEV)

    def run():
        o, lse = fa.flash_attn_fwd_masked(q, k, v, None, True, seqlens=lens, block_mask=bmap, dropout_p=0.2, seed=9)
        g = fa.flash_attn_bwd_masked(do, q, k, v, o, lse, None, True, seqlens=lens, block_mask=bmap,
                                     dropout_p=0.2, seed=9)
        o2, lse2 = fa.flash_attn_fwd_kvsplit(q[:, :, -3:].contiguous(), k, v, None, True, 0)
        # one split: the split kernel writes O and LSE itself (with a single query tile per head its
        # K/V loads also carry the non-temporal hint)
        o3, lse3 = fa.flash_attn_fwd_kvsplit(q[:, :, -3:].contiguous(), k, v, None, True, 1)
        o4, lse4 = fa.flash_attn_fwd_kvsplit(q[:, :, -300:].contiguous(), k, v, None, True, 1, seqlens_k=lens)
        return (o, lse, *g, o2, lse2, o3, lse3, o4, lse4)

    a, b = both(debug_lib, run)
    assert_bitwise(a, b)
