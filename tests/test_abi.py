"""CPU-side tests of the C ABI: the library loads, exports every symbol the header declares,
and rejects each invalid argument with its status before anything is launched.

Every call here fails validation (NULL or fake host addresses are never dereferenced: the
library returns before any HIP call), so these tests need no GPU."""
import ctypes
import math
import os
import re

import pytest

from io_aware_flashattention_flash_amd import flash_attn as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flash_attn.h")

OK, NULLP, SHAPE, UNSUP, SCALE, ALIGN, WS, HIP, DROP, SCRATCH = range(10)
A = 0x10000  # a 16-byte-aligned fake address; never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libflashattn.so not built (run __graft_entry__.build())")
    return fa.load_library()


def _header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status_t|size_t|const char\*)\s+(flash_attn_\w+)\s*\(", text, re.M)))


def test_header_declares_every_bound_entry_point():
    assert _header_functions() == sorted(fa.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    for name in _header_functions():
        assert hasattr(lib, name), name


def test_exports_have_c_linkage():
    """The shared object's dynamic symbol table carries the plain C names (no C++ mangling)."""
    import subprocess
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("not built")
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    names = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _header_functions():
        assert name in names, name


def test_status_strings(lib):
    for s in range(10):
        txt = fa.flash_attn_status_string(s)
        assert txt.startswith("FA_"), txt
    assert "unknown" in fa.flash_attn_status_string(99)


def _fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=8, d=64, scale=0.125, causal=0, dtype=1):
    return lib.flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, None)


def _bwd(lib, ptrs=None, ws=A, ws_bytes=1 << 20, B=1, H=1, N=8, d=64, scale=0.125, causal=0, dtype=1):
    p = dict(q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A)
    p.update(ptrs or {})
    return lib.flash_attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"], p["dv"],
                              ws, ws_bytes, B, H, N, d, scale, causal, dtype, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o"])
def test_fwd_null_pointer(lib, which):
    assert _fwd(lib, **{which: None}) == NULLP


@pytest.mark.parametrize("shape", [(0, 1, 8, 64), (1, 0, 8, 64), (1, 1, 0, 64), (1, 1, 8, 0), (-1, 1, 8, 64),
                                   (1 << 10, 1 << 10, 1 << 10, 64), (1, 1, 1 << 23, 64)])
def test_fwd_bad_shape(lib, shape):
    B, H, N, d = shape
    assert _fwd(lib, B=B, H=H, N=N, d=d) == SHAPE


@pytest.mark.parametrize("d,dtype", [(48, 1), (80, 2), (160, 1), (512, 1), (32, 0), (96, 0), (256, 0), (80, 0),
                                     (64, 3), (64, -1)])
def test_fwd_unsupported(lib, d, dtype):
    assert _fwd(lib, d=d, dtype=dtype) == UNSUP


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
@pytest.mark.parametrize("dtype", [1, 2])
def test_16bit_head_dims_pass_the_support_check(lib, d, dtype):
    """Every 16-bit entry point accepts d in {32, 64, 96, 128, 256}: these calls fail at the
    alignment check that follows (the fake pointers never reach a launch)."""
    assert _fwd(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert _bwd(lib, ptrs={"q": A + 8}, d=d, dtype=dtype) == ALIGN
    assert _kvs(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert _fm(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert _bm(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert _dq(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert _dkdv(lib, d=d, dtype=dtype, q=A + 8) == ALIGN
    assert lib.flash_attn_bwd_delta(A, A, A + 2, 1, 1, 8, d, dtype, None) == ALIGN


@pytest.mark.parametrize("scale", [math.nan, math.inf, -math.inf])
def test_fwd_bad_scale(lib, scale):
    assert _fwd(lib, scale=scale) == SCALE


@pytest.mark.parametrize("which,addr", [("q", A + 8), ("k", A + 4), ("v", A + 2), ("o", A + 1), ("lse", A + 2)])
def test_fwd_misaligned(lib, which, addr):
    assert _fwd(lib, **{which: addr}) == ALIGN


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"])
def test_bwd_null_pointer(lib, which):
    assert _bwd(lib, {which: None}) == NULLP


def test_bwd_unsupported_fp32_and_head_dim(lib):
    assert _bwd(lib, dtype=0) == UNSUP
    assert _bwd(lib, d=80) == UNSUP


def test_bwd_bad_scale_and_shape(lib):
    assert _bwd(lib, scale=math.nan) == SCALE
    assert _bwd(lib, N=0) == SHAPE


def test_bwd_workspace(lib):
    need = lib.flash_attn_bwd_workspace_size(2, 3, 100, 64, 1)
    assert need >= 2 * 3 * 100 * 4 and need % 256 == 0
    assert need < 2 * 3 * 100 * 100 * 4  # linear in N: no N x N scratch
    assert _bwd(lib, ws=None, B=2, H=3, N=100) == WS
    assert _bwd(lib, ws_bytes=need - 1, B=2, H=3, N=100) == WS
    assert _bwd(lib, ws=A + 4, ws_bytes=need, B=2, H=3, N=100) == ALIGN


def test_workspace_size_invalid_shape_is_zero(lib):
    assert lib.flash_attn_bwd_workspace_size(0, 1, 1, 64, 1) == 0


@pytest.mark.parametrize("which", ["q", "o", "do", "dq", "dk", "dv"])
def test_bwd_misaligned(lib, which):
    assert _bwd(lib, {which: A + 8}) == ALIGN


def test_python_binding_rejects_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.flash_attn_fwd(x, x, x)


def test_signature_table_matches_header_parameter_counts():
    text = open(HEADER).read()
    for name, (_, args) in fa.SIGNATURES.items():
        m = re.search(r"^\s*(?:fa_status_t|size_t|const char\*)\s+" + name + r"\s*\(([^)]*)\)", text, re.M)
        assert m, name
        nparams = len([p for p in m.group(1).split(",") if p.strip()])
        assert nparams == len(args), (name, nparams, len(args))


def _stage_args(**kw):
    a = dict(q=A, k=A, v=A, o=A, lse=A, do=A, delta=A, dk=A, dv=A, dq=A, B=1, H=1, N=8, d=64, scale=0.125, causal=0,
             dtype=1)
    a.update(kw)
    return a


def _dkdv(lib, **kw):
    a = _stage_args(**kw)
    return lib.flash_attn_bwd_dkdv(a["q"], a["k"], a["v"], a["lse"], a["do"], a["delta"], a["dk"], a["dv"], a["B"],
                                   a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)


def _dq(lib, **kw):
    a = _stage_args(**kw)
    return lib.flash_attn_bwd_dq(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["delta"], a["dq"], a["B"],
                                 a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], None)


def _kvs(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=1, Nk=8, d=64, scale=0.125, causal=0, splits=0, ws=A,
         ws_bytes=1 << 20, dtype=1, seqlens_k=None):
    return lib.flash_attn_fwd_kvsplit(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, seqlens_k, splits, ws, ws_bytes,
                                      dtype, None)


def test_kvsplit_validation(lib):
    assert _kvs(lib, q=None) == NULLP
    assert _kvs(lib, Nq=9, Nk=8) == SHAPE          # more queries than keys
    assert _kvs(lib, splits=65) == SHAPE
    assert _kvs(lib, splits=-1) == SHAPE
    assert _kvs(lib, Nq=0) == SHAPE
    assert _kvs(lib, dtype=0) == UNSUP              # 16-bit types only
    assert _kvs(lib, d=80) == UNSUP
    assert _kvs(lib, scale=math.inf) == SCALE
    assert _kvs(lib, k=A + 8) == ALIGN
    assert _kvs(lib, ws=None) == WS
    assert _kvs(lib, ws_bytes=16) == WS
    assert _kvs(lib, ws=A + 4) == ALIGN
    assert _kvs(lib, dtype=2, v=A + 2) == ALIGN      # fp16 gets past the dtype check
    assert _kvs(lib, seqlens_k=A + 2) == ALIGN       # int32 lengths: 4-byte aligned


def _fm(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, N=8, d=64, scale=0.125, causal=0, seqlens=None, bm=None, p=0.0,
        seed=0, dtype=1):
    return lib.flash_attn_fwd_masked(q, k, v, o, lse, B, H, N, d, scale, causal, seqlens, bm, p, seed, dtype, None)


def _bm(lib, q=A, k=A, v=A, o=A, lse=A, do=A, dq=A, dk=A, dv=A, ws=A, ws_bytes=1 << 20, B=1, H=1, N=8, d=64,
        scale=0.125, causal=0, seqlens=None, bmask=None, p=0.0, seed=0, dtype=1):
    return lib.flash_attn_bwd_masked(q, k, v, o, lse, do, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, causal, seqlens,
                                     bmask, p, seed, dtype, None)


def test_masked_validation(lib):
    for call in (_fm, _bm):
        assert call(lib, q=None) == NULLP
        assert call(lib, N=0) == SHAPE
        assert call(lib, dtype=0) == UNSUP            # 16-bit types only
        assert call(lib, d=80) == UNSUP
        assert call(lib, scale=math.nan) == SCALE
        assert call(lib, k=A + 8) == ALIGN
        assert call(lib, seqlens=A + 2) == ALIGN
        assert call(lib, dtype=2, q=A + 8) == ALIGN   # fp16 gets past the dtype check
    # a block map row may hold at most FA_MAX_MASK_BLOCKS = 1024 blocks of 128 keys
    assert _fm(lib, N=1024 * 128 + 1, B=1, H=1, bm=A) == UNSUP
    assert _bm(lib, N=1024 * 128 + 1, bmask=A) == UNSUP
    assert _fm(lib, N=1024 * 128 + 1, q=A + 8) == ALIGN  # without a map the length is fine
    assert _bm(lib, ws=None) == WS
    assert _bm(lib, lse=None) == NULLP
    for call in (_fm, _bm):
        for bad in (-0.1, 1.0, 0.999, math.nan, math.inf):
            assert call(lib, p=bad, k=A + 8 if call is _fm else A) in (DROP, ALIGN), bad
        assert call(lib, p=-0.1) == DROP and call(lib, p=1.0) == DROP and call(lib, p=math.nan) == DROP
        assert call(lib, p=0.998, q=A + 8) == ALIGN   # T = round(256 * 0.002) = 1 is allowed
        assert call(lib, p=0.5, seed=2 ** 64 - 1, q=A + 8) == ALIGN


def test_dropout_mask_validation(lib):
    assert lib.flash_attn_dropout_mask(None, 1, 1, 4, 4, 0.5, 1, None) == NULLP
    assert lib.flash_attn_dropout_mask(A, 0, 1, 4, 4, 0.5, 1, None) == SHAPE
    assert lib.flash_attn_dropout_mask(A, 1, 1, 4, 0, 0.5, 1, None) == SHAPE
    assert lib.flash_attn_dropout_mask(A, 1, 1, 4, 4, 1.5, 1, None) == DROP


def test_kvsplit_workspace_size(lib):
    assert lib.flash_attn_fwd_kvsplit_workspace_size(1, 1, 9, 8, 64, 0, 1) == 0      # Nq > Nk
    one = lib.flash_attn_fwd_kvsplit_workspace_size(2, 4, 3, 1000, 128, 1, 1)
    four = lib.flash_attn_fwd_kvsplit_workspace_size(2, 4, 3, 1000, 128, 4, 1)
    assert one >= 2 * 4 * 3 * 129 * 4 and four >= 4 * 2 * 4 * 3 * 129 * 4 and four > one
    assert one < 2 * 4 * 3 * 1000 * 4  # linear in Nq, independent of Nk: no score matrix


def test_fp16_passes_the_dtype_check(lib):
    """dtype 2 (fp16) is in the support matrix of every entry point: its calls get past the dtype
    check to the later ones (these fake pointers never reach a launch)."""
    assert _fwd(lib, dtype=2, q=A + 8) == ALIGN
    assert _bwd(lib, dtype=2, scale=math.nan) == SCALE
    assert _dq(lib, dtype=2, k=A + 8) == ALIGN
    assert _dkdv(lib, dtype=2, lse=A + 1) == ALIGN
    assert lib.flash_attn_bwd_delta(A, A, A + 2, 1, 1, 8, 64, 2, None) == ALIGN


def test_bwd_stage_validation(lib):
    assert lib.flash_attn_bwd_delta(None, A, A, 1, 1, 8, 64, 1, None) == NULLP
    assert lib.flash_attn_bwd_delta(A, A, A + 2, 1, 1, 8, 64, 1, None) == ALIGN
    assert lib.flash_attn_bwd_delta(A, A, A, 1, 1, 8, 80, 1, None) == UNSUP
    assert lib.flash_attn_bwd_delta(A, A, A, 1, 1, 0, 64, 1, None) == SHAPE
    for fn in (_dkdv, _dq):
        assert fn(lib, q=None) == NULLP
        assert fn(lib, delta=None) == NULLP
        assert fn(lib, dtype=0) == UNSUP
        assert fn(lib, d=200) == UNSUP
        assert fn(lib, scale=math.inf) == SCALE
        assert fn(lib, N=0) == SHAPE
        assert fn(lib, k=A + 8) == ALIGN
        assert fn(lib, lse=A + 1) == ALIGN
    assert _dkdv(lib, dv=None) == NULLP
    assert _dq(lib, dq=A + 8) == ALIGN
    assert _dq(lib, o=None) == NULLP
    assert _dq(lib, o=A + 4) == ALIGN


def _support_matrix():
    """{dtype code: set of head dims} from the header's 'Support' paragraph."""
    text = open(HEADER).read()
    m16 = re.search(r"bf16, fp16:\s*d in \{([0-9, ]+)\}", text)
    m32 = re.search(r"fp32:\s*d in \{([0-9, ]+)\};\s*flash_attn_fwd only", text)
    assert m16 and m32, "support lines not found in the header"
    d16 = {int(x) for x in m16.group(1).split(",")}
    d32 = {int(x) for x in m32.group(1).split(",")}
    return {0: d32, 1: d16, 2: d16}


def test_header_support_matrix_matches_the_abi(lib):
    """Every entry point accepts exactly the (dtype, d) pairs the header lists: a supported pair
    gets past the support check to the alignment check (the fake pointers never reach a launch),
    any other pair is FA_ERR_UNSUPPORTED. fp32 is listed for flash_attn_fwd only."""
    support = _support_matrix()
    assert support[1] == {32, 64, 96, 128, 256} and support[0] == {64, 128}
    for dtype in (0, 1, 2):
        for d in range(1, 300):
            ok16 = dtype in (1, 2) and d in support[dtype]
            ok_fwd = d in support[dtype]
            want = lambda ok: ALIGN if ok else UNSUP  # noqa: E731
            assert _fwd(lib, d=d, dtype=dtype, q=A + 8) == want(ok_fwd), (dtype, d)
            assert _kvs(lib, d=d, dtype=dtype, q=A + 8) == want(ok16), (dtype, d)
            assert _fm(lib, d=d, dtype=dtype, q=A + 8) == want(ok16), (dtype, d)
            assert _bwd(lib, ptrs={"q": A + 8}, d=d, dtype=dtype) == want(ok16), (dtype, d)
            assert _bm(lib, d=d, dtype=dtype, q=A + 8) == want(ok16), (dtype, d)
            assert _dq(lib, d=d, dtype=dtype, q=A + 8) == want(ok16), (dtype, d)
            assert _dkdv(lib, d=d, dtype=dtype, q=A + 8) == want(ok16), (dtype, d)
            assert lib.flash_attn_bwd_delta(A, A, A + 2, 1, 1, 8, d, dtype, None) == want(ok16), (dtype, d)


class _StubLib:
    """Stands in for the library in binding-only tests: sizes are answered, compute calls fail."""

    def flash_attn_fwd_kvsplit_workspace_size(self, *args):
        return 4096

    def flash_attn_bwd_workspace_size(self, *args):
        return 4096

    def __getattr__(self, name):
        raise AssertionError(f"{name} must not be reached: the binding should have rejected the call")


@pytest.mark.parametrize("entry", ["kvsplit", "bwd", "bwd_masked"])
@pytest.mark.parametrize("bad", ["other_device", "non_contiguous", "not_a_tensor"])
def test_binding_rejects_a_bad_workspace_before_any_library_call(monkeypatch, entry, bad):
    """A workspace on another device than q (here: q on the host, workspace on the meta device), a
    non-contiguous one, or a non-tensor is rejected in Python; the library's compute entry point is
    never called, so no foreign address reaches a kernel."""
    import torch
    monkeypatch.setattr(fa, "load_library", lambda *a: _StubLib())
    monkeypatch.setattr(fa, "_check_tensor", lambda name, t, like=None: None)  # accept host tensors here
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    if bad == "other_device":
        ws = torch.empty(4096, dtype=torch.uint8, device="meta")
    elif bad == "non_contiguous":
        ws = torch.empty(2, 4096, dtype=torch.uint8)[:, ::2]
    else:
        ws = 12345
    with pytest.raises((ValueError, TypeError), match="workspace"):
        if entry == "kvsplit":
            fa.flash_attn_fwd_kvsplit(q, q, q, workspace=ws)
        elif entry == "bwd":
            lse = torch.zeros(1, 2, 8)
            fa.flash_attn_bwd(q, q, q, q, q, lse, workspace=ws)
        else:
            lse = torch.zeros(1, 2, 8)
            fa.flash_attn_bwd_masked(q, q, q, q, q, lse, workspace=ws)


def _kvs_na(lib, q=A, k=A, v=A, o=A, lse=A, B=1, H=1, Nq=1, Nk=8, d=64, scale=0.125, causal=0, splits=0, dtype=1,
            seqlens_k=None):
    return lib.flash_attn_fwd_kvsplit_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, seqlens_k, splits,
                                              dtype, None)


def test_kvsplit_noalloc_validation(lib):
    """The no-allocation key-split forward checks its arguments like flash_attn_fwd_kvsplit (before
    anything else), and a call whose partials would not fit the fixed scratch is refused with
    FA_ERR_SCRATCH_LIMIT before any HIP call."""
    assert _kvs_na(lib, q=None) == NULLP
    assert _kvs_na(lib, Nq=9, Nk=8) == SHAPE
    assert _kvs_na(lib, splits=65) == SHAPE
    assert _kvs_na(lib, dtype=0) == UNSUP
    assert _kvs_na(lib, d=80) == UNSUP
    assert _kvs_na(lib, scale=math.inf) == SCALE
    assert _kvs_na(lib, k=A + 8) == ALIGN
    assert _kvs_na(lib, seqlens_k=A + 2) == ALIGN
    limit = fa.FA_NOALLOC_SCRATCH_BYTES
    # 64 splits of B*H*Nq = 1024 rows of d = 128: 64 * 1024 * 129 * 4 bytes > 16 MiB
    B, H, Nq, Nk, d, S = 8, 32, 4, 8192, 128, 64
    assert lib.flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d, S, 1) > limit
    assert _kvs_na(lib, B=B, H=H, Nq=Nq, Nk=Nk, d=d, splits=S) == SCRATCH
    assert "SCRATCH" in fa.flash_attn_status_string(SCRATCH)


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.FA_NOALLOC_SCRATCH_BYTES
