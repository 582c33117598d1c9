"""Seeded synthetic inputs and the workload registry.

This module is shared by the tests, the benchmark and the smoke check: it
draws the tensors that both the HIP path and the CPU oracle consume. It holds
none of the attention arithmetic, only random draws, the fp32 -> bf16
rounding of those draws, and the table of workloads.

Recipe (the pages name no generator, seed or distribution beyond "Q/K/V"
being N x d matrices, so this is a reading of them):
  * ``rng = numpy.random.default_rng(seed)``;
  * draw, in this order, Q, K, V and (for a backward workload) dO, each as
    ``rng.standard_normal([B, H, N, d])`` cast to float32;
  * a workload with ``q_mult`` multiplies Q by that factor in float32 (a
    power of two, so exact);
  * bf16 workloads round every tensor to bf16 round-to-nearest-even; the
    rounded values are kept as float32 arrays whose low 16 bits are zero, so
    the same numbers reach the GPU (as bf16) and the oracle (as float64).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "fp32", "bf16" or "fp16": storage type of Q, K, V, O, dO
    B: int
    H: int
    N: int
    d: int
    causal: bool
    backward: bool      # True when the workload also runs the recompute backward
    q_mult: float = 1.0
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def fwd_flops(self) -> float:
        """4*B*H*N^2*d, halved for a causal mask (the counting convention of the
        workload definitions; masked work is not counted)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        return f * 0.5 if self.causal else f

    def bwd_flops(self) -> float:
        """Five N x N x d products in the backward (recomputed S, dV, dP, dQ, dK):
        2.5 times the forward count."""
        return 2.5 * self.fwd_flops()


# The five synthetic workloads: a small fp32 case, a short-sequence bf16 case,
# two long causal bf16 cases and a causal forward+backward case.
WORKLOADS: Dict[str, Workload] = {
    "fwd_fp32_b1h1n128d64": Workload("fwd_fp32_b1h1n128d64", "fp32", 1, 1, 128, 64, False, False),
    "fwd_bf16_b4h16n1024d64": Workload("fwd_bf16_b4h16n1024d64", "bf16", 4, 16, 1024, 64, False, False),
    "fwd_bf16_b2h32n4096d128_causal": Workload("fwd_bf16_b2h32n4096d128_causal", "bf16", 2, 32, 4096, 128, True, False),
    "fwd_bf16_b1h16n16384d128_causal_q2": Workload("fwd_bf16_b1h16n16384d128_causal_q2", "bf16", 1, 16, 16384, 128, True,
                                                   False, q_mult=2.0),
    "fwdbwd_bf16_b4h16n2048d64_causal": Workload("fwdbwd_bf16_b4h16n2048d64_causal", "bf16", 4, 16, 2048, 64, True, True),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returned as float32
    whose low 16 bits are zero. Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (r.astype(np.uint32) << 16).view(np.float32)


def round_to_fp16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest IEEE binary16 (ties to even, NumPy's cast); returned as
    float32. Values beyond the binary16 range become infinite."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage type `dtype` ("fp32" leaves them unchanged)."""
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "fp16":
        return round_to_fp16(x)
    return np.ascontiguousarray(x, dtype=np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None, shape=None) -> Dict[str, np.ndarray]:
    """Draw Q, K, V (and dO for a backward workload) for workload ``w``.

    ``shape`` overrides [B, H, N, d] (used for reduced-size parity cases that
    keep the workload's dtype, mask and value distribution)."""
    seed = w.seed if seed is None else seed
    shape = tuple(shape) if shape is not None else w.shape
    rng = np.random.default_rng(seed)
    names = ["q", "k", "v"] + (["do"] if w.backward else [])
    out = {}
    for nm in names:
        t = rng.standard_normal(shape).astype(np.float32)
        if nm == "q" and w.q_mult != 1.0:
            t = t * np.float32(w.q_mult)
        out[nm] = round_to(t, w.dtype)
    return out


def random_tensor(shape, seed: int, dtype: str = "bf16", mult: float = 1.0) -> np.ndarray:
    """One standard-normal tensor from its own seed (for edge-case tests)."""
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal(shape) * mult).astype(np.float32)
    return round_to(t, dtype)


GRID_STEP = 1.0 / 64.0


def grid_codes(shape, seed: int) -> np.ndarray:
    """Integer codes c, uniform on [-128, 128), as int8; the tensor's values are c * GRID_STEP,
    uniform on [-2, 2) in steps of 1/64. Every such value is exact in bf16 and fp16 (at most 8
    significant bits), so the codes can be widened on either side without rounding. One byte per
    element and no float draws: cheap enough for tensors of ~2^31 elements (the size-limit tests),
    where standard-normal draws would dominate the run."""
    return np.random.default_rng(seed).integers(-128, 128, size=shape, dtype=np.int8)
