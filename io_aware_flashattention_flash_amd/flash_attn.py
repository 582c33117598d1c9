"""Python binding of libflashattn.so (argument marshalling only).

The functions carry the C ABI's names. They check what only Python can see
(device, dtype, contiguity, matching shapes), allocate outputs and the
backward workspace with torch (PyTorch supplies device memory and the current
stream), pass raw device pointers to the library and raise RuntimeError with
the library's status string on any error. Every step of the attention runs in
the library's HIP kernels; there is no fallback path. If the shared library
has not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashattn.so")

FA_DTYPE_FP32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_FP16 = 2
FA_MASK_BLOCK = 128  # rows and keys per block-sparse map entry
_DTYPES = {torch.float32: FA_DTYPE_FP32, torch.bfloat16: FA_DTYPE_BF16, torch.float16: FA_DTYPE_FP16}

# Names and C signatures of every exported entry point (mirrors include/flash_attn.h).
_vp, _int, _float, _size, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_uint64
SIGNATURES = {
    "flash_attn_fwd": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _float, _int, _int, _vp]),
    "flash_attn_bwd_workspace_size": (_size, [_int, _int, _int, _int, _int]),
    "flash_attn_bwd": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size,
                              _int, _int, _int, _int, _float, _int, _int, _vp]),
    "flash_attn_bwd_delta": (_int, [_vp, _vp, _vp, _int, _int, _int, _int, _int, _vp]),
    "flash_attn_bwd_dkdv": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _int, _int, _int, _int, _float, _int, _int, _vp]),
    "flash_attn_bwd_dq": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _int, _int, _int, _int, _float, _int, _int, _vp]),
    "flash_attn_fwd_kvsplit_workspace_size": (_size, [_int, _int, _int, _int, _int, _int, _int]),
    "flash_attn_fwd_kvsplit": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _float, _int, _vp,
                                      _int, _vp, _size, _int, _vp]),
    "flash_attn_fwd_masked": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _float, _int, _vp, _vp,
                                     _float, _u64, _int, _vp]),
    "flash_attn_bwd_masked": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _size,
                                     _int, _int, _int, _int, _float, _int, _vp, _vp, _float, _u64, _int, _vp]),
    "flash_attn_dropout_mask": (_int, [_vp, _int, _int, _int, _int, _float, _u64, _vp]),
    "flash_attn_fwd_kvsplit_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _int, _int, _int, _int, _int, _float, _int,
                                              _vp, _int, _int, _vp]),
    "flash_attn_status_string": (ctypes.c_char_p, [_int]),
}
FA_NOALLOC_SCRATCH_BYTES = 16 << 20  # the library's fixed scratch per GPU (include/flash_attn.h)

_lib_handle = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once and declare its signatures. Raises if it is not built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(path):
            raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                               "or python -m io_aware_flashattention_flash_amd.build")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = lib
    return _lib_handle


def flash_attn_status_string(status: int) -> str:
    return load_library().flash_attn_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise RuntimeError(flash_attn_status_string(status))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_tensor(name: str, t: torch.Tensor, like: Optional[torch.Tensor] = None) -> None:
    # (cheap accessors only: these checks run on every call, in front of microsecond kernels)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if like is None:
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got {tuple(t.shape)}")
        if t.dtype not in _DTYPES:
            raise ValueError(f"{name} must be bfloat16, float16 or float32, got {t.dtype}")
    elif t.shape != like.shape or t.dtype != like.dtype or t.get_device() != like.get_device():
        # (like has passed these checks itself: matching it makes t 4-D with a supported dtype)
        raise ValueError(f"{name} must match q in shape, dtype and device")


def _check_workspace(workspace: torch.Tensor, q: torch.Tensor) -> int:
    """A caller-supplied workspace must be a contiguous tensor on q's device (its address is passed
    to kernels that write it); returns its size in bytes."""
    if not isinstance(workspace, torch.Tensor):
        raise TypeError("workspace must be a torch.Tensor")
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on q's device")
    return workspace.numel() * workspace.element_size()


def _stream_handle(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.get_device()).cuda_stream


def flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                   causal: bool = False, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, want_lse: bool = True
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """O = softmax(scale * Q K^T [causal]) V and the natural-log LSE, on the current stream."""
    _check_tensor("q", q)
    _check_tensor("k", k, q)
    _check_tensor("v", v, q)
    B, H, N, d = q.shape
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous()
                            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    st = load_library().flash_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                       int(bool(causal)), _DTYPES[q.dtype], _stream_handle(q))
    _check(st)
    return out, lse


def flash_attn_fwd_kvsplit_workspace_size(B: int, H: int, Nq: int, Nk: int, d: int, num_splits: int = 0,
                                          dtype: int = FA_DTYPE_BF16) -> int:
    return int(load_library().flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d, num_splits, dtype))


def _check_seqlens(name: str, t: Optional[torch.Tensor], B: int, ref: torch.Tensor) -> None:
    if t is None:
        return
    if t.dtype != torch.int32 or tuple(t.shape) != (B,) or not t.is_contiguous() or t.device != ref.device:
        raise ValueError(f"{name} must be a contiguous int32 [B] tensor on q's device")


def _check_block_mask(t: Optional[torch.Tensor], B: int, H: int, N: int, ref: torch.Tensor) -> None:
    if t is None:
        return
    nb = (N + FA_MASK_BLOCK - 1) // FA_MASK_BLOCK
    if t.dtype not in (torch.uint8, torch.bool) or tuple(t.shape) != (B, H, nb, nb) or not t.is_contiguous() \
            or t.device != ref.device:
        raise ValueError(f"block_mask must be a contiguous uint8 or bool [B, H, {nb}, {nb}] tensor on q's device")


def flash_attn_fwd_masked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                          causal: bool = False, seqlens: Optional[torch.Tensor] = None,
                          block_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, want_lse: bool = True, dropout_p: float = 0.0,
                          seed: int = 0) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Forward with per-sequence lengths (int32 [B]: rows >= L_b of Q, K, V are padding), a
    block-sparse map (uint8 / bool [B, H, ceil(N/128), ceil(N/128)], zero = block skipped) and/or
    attention dropout (probability dropout_p, Philox key `seed`). Rows that see no key get O = 0,
    LSE = -inf."""
    _check_tensor("q", q)
    _check_tensor("k", k, q)
    _check_tensor("v", v, q)
    B, H, N, d = q.shape
    _check_seqlens("seqlens", seqlens, B, q)
    _check_block_mask(block_mask, B, H, N, q)
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_rows("lse", lse, q)
    st = load_library().flash_attn_fwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                                              int(bool(causal)), _ptr(seqlens), _ptr(block_mask), float(dropout_p),
                                              int(seed) & (2 ** 64 - 1), _DTYPES[q.dtype], _stream_handle(q))
    _check(st)
    return out, lse


def flash_attn_bwd_masked(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                          lse: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
                          seqlens: Optional[torch.Tensor] = None, block_mask: Optional[torch.Tensor] = None,
                          dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                          dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                          dropout_p: float = 0.0, seed: int = 0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Backward of flash_attn_fwd_masked (same seqlens, block_mask, dropout_p and seed)."""
    _check_tensor("q", q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q)
    B, H, N, d = q.shape
    _check_rows("lse", lse, q)
    _check_seqlens("seqlens", seqlens, B, q)
    _check_block_mask(block_mask, B, H, N, q)
    scale = float(d) ** -0.5 if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q)
    dt = _DTYPES[q.dtype]
    need = flash_attn_bwd_workspace_size(B, H, N, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q)
    st = load_library().flash_attn_bwd_masked(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                              _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d, scale,
                                              int(bool(causal)), _ptr(seqlens), _ptr(block_mask), float(dropout_p),
                                              int(seed) & (2 ** 64 - 1), dt, _stream_handle(q))
    _check(st)
    return dq, dk, dv


def flash_attn_dropout_mask(B: int, H: int, Nq: int, Nk: int, dropout_p: float, seed: int,
                            device="cuda", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The keep mask (uint8 [B, H, Nq, Nk], 1 = kept) that flash_attn_fwd_masked applies for
    (dropout_p, seed)."""
    if out is None:
        out = torch.empty((B, H, Nq, Nk), dtype=torch.uint8, device=device)
    if out.dtype != torch.uint8 or tuple(out.shape) != (B, H, Nq, Nk) or not out.is_contiguous() \
            or out.device.type != "cuda":
        raise ValueError("out must be a contiguous uint8 [B, H, Nq, Nk] GPU tensor")
    st = load_library().flash_attn_dropout_mask(_ptr(out), B, H, Nq, Nk, float(dropout_p), int(seed) & (2 ** 64 - 1),
                                                _stream_handle(out))
    _check(st)
    return out


def flash_attn_fwd_kvsplit(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: Optional[float] = None,
                           causal: bool = False, num_splits: int = 0, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, want_lse: bool = True,
                           workspace: Optional[torch.Tensor] = None, seqlens_k: Optional[torch.Tensor] = None
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Attention of q [B, H, Nq, d] against k, v [B, H, Nk, d] with Nq <= Nk (decode / chunked
    prefill), the key range split across workgroups and the partial softmaxes merged. Causal
    aligns the queries with the last Nq key positions. seqlens_k (int32 [B]) gives each
    sequence's valid cache length L_b <= Nk; its queries are then positions L_b - Nq .. L_b - 1."""
    _check_tensor("q", q)
    _check_tensor("k", k)
    _check_tensor("v", v, k)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H, d, dtype and device")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous()
                            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    _check_seqlens("seqlens_k", seqlens_k, B, q)
    dt = _DTYPES[q.dtype]
    need = flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d, num_splits, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q)
    st = load_library().flash_attn_fwd_kvsplit(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk, d,
                                               scale, int(bool(causal)), _ptr(seqlens_k), int(num_splits),
                                               _ptr(workspace), ws_bytes, dt, _stream_handle(q))
    _check(st)
    return out, lse


def flash_attn_fwd_kvsplit_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor,
                                   lse: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                                   causal: bool = False, num_splits: int = 0,
                                   seqlens_k: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """flash_attn_fwd_kvsplit with its partials in the library's fixed scratch array instead of a
    workspace: the caller passes the outputs (out [B, H, Nq, d], optional lse [B, H, Nq]), and neither
    this function nor the library allocates anything. Calls that may overlap on one GPU race on the
    shared scratch."""
    _check_tensor("q", q)
    _check_tensor("k", k)
    _check_tensor("v", v, k)
    _check_tensor("out", out, q)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H, d, dtype and device")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous()
                            or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, Nq] tensor on q's device")
    _check_seqlens("seqlens_k", seqlens_k, B, q)
    scale = float(d) ** -0.5 if scale is None else float(scale)
    st = load_library().flash_attn_fwd_kvsplit_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Nq, Nk,
                                                       d, scale, int(bool(causal)), _ptr(seqlens_k), int(num_splits),
                                                       _DTYPES[q.dtype], _stream_handle(q))
    _check(st)
    return out, lse


def flash_attn_bwd_workspace_size(B: int, H: int, N: int, d: int, dtype: int = FA_DTYPE_BF16) -> int:
    return int(load_library().flash_attn_bwd_workspace_size(B, H, N, d, dtype))


def flash_attn_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                   lse: torch.Tensor, scale: Optional[float] = None, causal: bool = False,
                   dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                   dv: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None
                   ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """dQ, dK, dV of sum(O * dout), recomputing P from the forward's O and LSE."""
    _check_tensor("q", q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q)
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 [B, H, N] tensor on q's device")
    scale = float(d) ** -0.5 if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, q)
    dt = _DTYPES[q.dtype]
    need = flash_attn_bwd_workspace_size(B, H, N, d, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = _check_workspace(workspace, q)
    st = load_library().flash_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                       _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, H, N, d, scale,
                                       int(bool(causal)), dt, _stream_handle(q))
    _check(st)
    return dq, dk, dv


def _check_rows(name: str, t: torch.Tensor, q: torch.Tensor) -> None:
    B, H, N, _ = q.shape
    if t.dtype != torch.float32 or tuple(t.shape) != (B, H, N) or not t.is_contiguous() or t.device != q.device:
        raise ValueError(f"{name} must be a contiguous float32 [B, H, N] tensor on q's device")


def flash_attn_bwd_delta(o: torch.Tensor, dout: torch.Tensor, delta: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Backward stage 1: delta = rowsum(dout * o), float32 [B, H, N]."""
    _check_tensor("o", o)
    _check_tensor("dout", dout, o)
    B, H, N, d = o.shape
    if delta is None:
        delta = torch.empty((B, H, N), dtype=torch.float32, device=o.device)
    _check_rows("delta", delta, o)
    _check(load_library().flash_attn_bwd_delta(_ptr(o), _ptr(dout), _ptr(delta), B, H, N, d, _DTYPES[o.dtype],
                                               _stream_handle(o)))
    return delta


def flash_attn_bwd_dkdv(q, k, v, lse, dout, delta, scale=None, causal=False, dk=None, dv=None):
    """Backward stage 2 (key-outer recompute): dK and dV."""
    _check_tensor("q", q)
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _check_tensor(name, t, q)
    _check_rows("lse", lse, q)
    _check_rows("delta", delta, q)
    B, H, N, d = q.shape
    scale = float(d) ** -0.5 if scale is None else float(scale)
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_tensor("dk", dk, q)
    _check_tensor("dv", dv, q)
    _check(load_library().flash_attn_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(lse), _ptr(dout), _ptr(delta),
                                              _ptr(dk), _ptr(dv), B, H, N, d, scale, int(bool(causal)),
                                              _DTYPES[q.dtype], _stream_handle(q)))
    return dk, dv


def flash_attn_bwd_dq(q, k, v, o, lse, dout, scale=None, causal=False, dq=None, delta=None):
    """Backward query-outer stage: dQ, plus delta = rowsum(dout * o) for the dK/dV stage."""
    _check_tensor("q", q)
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_tensor(name, t, q)
    _check_rows("lse", lse, q)
    B, H, N, d = q.shape
    scale = float(d) ** -0.5 if scale is None else float(scale)
    dq = torch.empty_like(q) if dq is None else dq
    delta = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if delta is None else delta
    _check_tensor("dq", dq, q)
    _check_rows("delta", delta, q)
    _check(load_library().flash_attn_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(delta),
                                            _ptr(dq), B, H, N, d, scale, int(bool(causal)), _DTYPES[q.dtype],
                                            _stream_handle(q)))
    return dq, delta


class FlashAttnFunction(torch.autograd.Function):
    """autograd wrapper: forward saves (q, k, v, o, lse); backward recomputes through the library.
    With lengths, a block map or dropout it uses the masked entry points, and the dropout seed is
    kept so the backward regenerates the same keep mask."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, causal=False, seqlens=None, block_mask=None, dropout_p=0.0, seed=0):
        ctx.masked = seqlens is not None or block_mask is not None or dropout_p > 0.0
        if ctx.masked:
            o, lse = flash_attn_fwd_masked(q, k, v, scale, causal, seqlens=seqlens, block_mask=block_mask,
                                           dropout_p=dropout_p, seed=seed)
        else:
            o, lse = flash_attn_fwd(q, k, v, scale, causal)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale, ctx.causal = scale, causal
        ctx.seqlens, ctx.block_mask, ctx.dropout_p, ctx.seed = seqlens, block_mask, dropout_p, seed
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if ctx.masked:
            dq, dk, dv = flash_attn_bwd_masked(do.contiguous(), q, k, v, o, lse, ctx.scale, ctx.causal,
                                               seqlens=ctx.seqlens, block_mask=ctx.block_mask,
                                               dropout_p=ctx.dropout_p, seed=ctx.seed)
        else:
            dq, dk, dv = flash_attn_bwd(do.contiguous(), q, k, v, o, lse, ctx.scale, ctx.causal)
        return dq, dk, dv, None, None, None, None, None, None


def flash_attention(q, k, v, scale=None, causal=False, seqlens=None, block_mask=None, dropout_p=0.0, seed=None):
    """Differentiable exact attention on [B, H, N, d] tensors. seqlens (int32 [B]) and block_mask
    (uint8 [B, H, ceil(N/128), ceil(N/128)]) mask as in flash_attn_fwd_masked; dropout_p > 0 drops
    attention probabilities with a Philox seed (drawn from torch's CPU generator when None)."""
    if dropout_p > 0.0 and seed is None:
        seed = int(torch.randint(0, 2 ** 62, (1,)).item())
    return FlashAttnFunction.apply(q, k, v, scale, causal, seqlens, block_mask, float(dropout_p),
                                   0 if seed is None else int(seed))
