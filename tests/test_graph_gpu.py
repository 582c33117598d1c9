"""HIP graph capture of the library's launches. Once its outputs and workspace are passed in, no
entry point allocates, sets memory or synchronises, so a caller can record a whole attention step
into a graph (torch.cuda.CUDAGraph records HIP graphs on ROCm) and replay it. Each test captures
one sequence of calls once, then replays it several times on new inputs copied into the captured
tensors, with other GPU work and host synchronisations between the replays. Every replay must equal
an eager call of the same functions on the same inputs bit for bit (the same kernels, and each
kernel's result does not depend on launch timing); the eager calls themselves are checked against
the oracle by the other GPU tests."""
import pytest
import torch

from io_aware_flashattention_flash_amd import (flash_attn_bwd, flash_attn_bwd_masked, flash_attn_bwd_workspace_size,
                                               flash_attn_fwd, flash_attn_fwd_kvsplit, flash_attn_fwd_kvsplit_noalloc,
                                               flash_attn_fwd_kvsplit_workspace_size, flash_attn_fwd_masked, inputs)
from tests.test_parity_gpu import DEV

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _fill(tensors, seed):
    """New seeded standard-normal contents, rounded to the tensors' 16-bit type, copied in place."""
    for i, t in enumerate(tensors):
        a = inputs.random_tensor(tuple(t.shape), seed + i, "bf16")
        t.copy_(torch.from_numpy(a).to(DEV).to(t.dtype))


def _other_work():
    """Unrelated GPU work and a host synchronisation between replays."""
    x = torch.randn(1 << 20, device=DEV)
    y = (x * 2.0).sum()
    torch.cuda.synchronize()
    return float(y)


def _replay_and_compare(graph, static_in, static_out, eager, seed):
    for r in range(REPLAYS):
        _fill(static_in, seed + 10 * r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in static_out]
        want = eager()
        torch.cuda.synchronize()
        for i, (g, w) in enumerate(zip(got, want)):
            assert torch.equal(g, w), (r, i)
        _other_work()


@pytest.mark.parametrize("N", [333, 1100])
def test_graph_dense_forward_backward(N):
    """N = 1100 (small launch) runs the split forward, dQ and dK/dV kernels."""
    B, H, d, causal = 2, 4, 64, True
    scale = d ** -0.5
    q, k, v, do = (torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=DEV)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(1, flash_attn_bwd_workspace_size(B, H, N, d)), dtype=torch.uint8, device=DEV)
    _fill((q, k, v, do), 100)

    def step(o_, lse_, dq_, dk_, dv_):
        flash_attn_fwd(q, k, v, scale, causal, out=o_, lse=lse_)
        flash_attn_bwd(do, q, k, v, o_, lse_, scale, causal, dq=dq_, dk=dk_, dv=dv_, workspace=ws)

    step(o, lse, dq, dk, dv)  # eager first call (library load, device queries)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(o, lse, dq, dk, dv)

    def eager():
        outs = (torch.empty_like(o), torch.empty_like(lse), torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv))
        step(*outs)
        return outs

    _replay_and_compare(g, (q, k, v, do), (o, lse, dq, dk, dv), eager, 200)


def test_graph_masked_dropout_forward_backward():
    """Padding lengths, a block map and dropout (a fixed seed: the keep mask is the same on every
    replay, as in the eager call)."""
    B, H, N, d, causal = 2, 2, 300, 128, True
    scale = d ** -0.5
    q, k, v, do = (torch.empty(B, H, N, d, dtype=torch.bfloat16, device=DEV) for _ in range(4))
    sl = torch.tensor([300, 170], dtype=torch.int32, device=DEV)
    nb = -(-N // 128)
    bm = torch.ones(B, H, nb, nb, dtype=torch.uint8, device=DEV)
    bm[0, 1, 2, 0] = 0
    bm[1, 0, 1, 1] = 0
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=DEV)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(1, flash_attn_bwd_workspace_size(B, H, N, d)), dtype=torch.uint8, device=DEV)
    _fill((q, k, v, do), 300)
    kw = dict(seqlens=sl, block_mask=bm, dropout_p=0.2, seed=1234)

    def step(o_, lse_, dq_, dk_, dv_):
        flash_attn_fwd_masked(q, k, v, scale, causal, out=o_, lse=lse_, **kw)
        flash_attn_bwd_masked(do, q, k, v, o_, lse_, scale, causal, dq=dq_, dk=dk_, dv=dv_, workspace=ws, **kw)

    step(o, lse, dq, dk, dv)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(o, lse, dq, dk, dv)

    def eager():
        outs = (torch.empty_like(o), torch.empty_like(lse), torch.empty_like(dq), torch.empty_like(dk), torch.empty_like(dv))
        step(*outs)
        return outs

    _replay_and_compare(g, (q, k, v, do), (o, lse, dq, dk, dv), eager, 400)


@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_key_split_decode(noalloc):
    """A decoding step: 3 queries against 5000 cached keys per (batch, head), per-sequence cache
    lengths, with a workspace or through the no-allocation entry point."""
    B, H, Nq, Nk, d = 2, 4, 3, 5000, 128
    scale = d ** -0.5
    q = torch.empty(B, H, Nq, d, dtype=torch.bfloat16, device=DEV)
    k, v = (torch.empty(B, H, Nk, d, dtype=torch.bfloat16, device=DEV) for _ in range(2))
    lens = torch.tensor([5000, 3001], dtype=torch.int32, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, Nq, device=DEV)
    ws = torch.empty(max(1, flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d)), dtype=torch.uint8, device=DEV)
    _fill((q, k, v), 500)

    def step(o_, lse_):
        if noalloc:
            flash_attn_fwd_kvsplit_noalloc(q, k, v, o_, lse_, scale, True, 0, seqlens_k=lens)
        else:
            flash_attn_fwd_kvsplit(q, k, v, scale, True, 0, out=o_, lse=lse_, workspace=ws, seqlens_k=lens)

    step(o, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(o, lse)

    def eager():
        outs = (torch.empty_like(o), torch.empty_like(lse))
        step(*outs)
        return outs

    _replay_and_compare(g, (q, k, v), (o, lse), eager, 600)
