"""The C ABI from a host program of its own (tests/c_abi/abi_roundtrip, built with the library): no
Python binding and no torch between the caller and the library. The program reads bf16 inputs from
a file, runs the forward, the backward and the masked forward with dropout on a stream it creates,
and writes the outputs; they are checked against the float64 oracle with the usual bf16 gates."""
import os
import subprocess

import numpy as np
import pytest

from io_aware_flashattention_flash_amd import inputs
from oracle import attn_bwd, attn_fwd, attn_fwd_dropout, keep_mask, padded_batch_visible
from tests.test_parity_gpu import BF16_LSE, BF16_O, GRAD, beyond_rounding, grad_errors

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_roundtrip")


def _bf16_bits(x):
    """Bits of float32 values that are exactly bf16 (the input recipe rounds them so)."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _from_bf16(bits, shape):
    return (bits.astype(np.uint32) << 16).view(np.float32).reshape(shape).astype(np.float64)


@pytest.mark.parametrize("causal", [0, 1])
def test_standalone_program_through_the_c_abi(tmp_path, causal):
    if not os.path.exists(BIN):
        pytest.fail("tests/c_abi/abi_roundtrip is not built (run __graft_entry__.build())")
    B, H, N, d = 2, 3, 333, 64
    x = {n: inputs.random_tensor((B, H, N, d), 90 + i, "bf16") for i, n in enumerate(("q", "k", "v", "do"))}
    seqlens = np.array([333, 200], dtype=np.int32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for n in ("q", "k", "v", "do"):
            f.write(_bf16_bits(x[n]).tobytes())
        f.write(seqlens.tobytes())
    print(f"abi_roundtrip B={B} H={H} N={N} d={d} causal={causal}", flush=True)
    r = subprocess.run([BIN, str(src), str(dst), str(B), str(H), str(N), str(d), str(causal)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    raw = open(dst, "rb").read()
    shape, rows = (B, H, N, d), B * H * N
    e, off = B * H * N * d, 0
    out = {}
    for name, kind in (("o", 16), ("lse", 32), ("dq", 16), ("dk", 16), ("dv", 16), ("om", 16), ("lsem", 32)):
        if kind == 16:
            out[name] = _from_bf16(np.frombuffer(raw, np.uint16, e, off), shape)
            off += 2 * e
        else:
            out[name] = np.frombuffer(raw, np.float32, rows, off).reshape(B, H, N).astype(np.float64)
            off += 4 * rows
    assert off == len(raw)
    scale = d ** -0.5
    O, L = attn_fwd(x["q"], x["k"], x["v"], scale, bool(causal))
    assert np.abs(out["o"] - O).max() <= BF16_O and np.abs(out["lse"] - L).max() <= BF16_LSE
    dQ, dK, dV, _ = attn_bwd(x["q"], x["k"], x["v"], x["do"], scale, bool(causal))
    for name, r_ in (("dq", dQ), ("dk", dK), ("dv", dV)):
        e_inf, e_fro = grad_errors(out[name], r_)
        assert e_inf <= GRAD and e_fro <= GRAD, (name, e_inf, e_fro)
    # masked forward with lengths and dropout 0.25, seed 0x5eed (as the program passes them)
    vis = padded_batch_visible(B, H, N, bool(causal), list(seqlens))
    Om, Lm = attn_fwd_dropout(x["q"], x["k"], x["v"], scale, vis, keep_mask(B, H, N, N, 0.25, 0x5EED), 0.25)
    full = np.isfinite(Lm)
    assert (out["om"][~full] == 0).all() and np.isneginf(out["lsem"][~full]).all()
    assert beyond_rounding(out["om"][full], Om[full]) <= BF16_O
    assert np.abs(out["lsem"][full] - Lm[full]).max() <= BF16_LSE
