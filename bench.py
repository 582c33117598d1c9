#!/usr/bin/env python3
"""Attention throughput on one MI355X: TFLOPS (fwd, fwd+bwd) and % of the dense bf16 MFMA peak.

One step is one pass of the whole hot path over one batch of resident synthetic input: the fused
forward (O, LSE) followed by the two backward stages (dQ with delta, then dK/dV) of the causal bf16
workload B=4 H=16 N=2048 d=64. FLOPs follow the workload definition: 4*B*H*N^2*d for the
forward, halved for the causal mask, and 2.5x that for the backward (five N x N x d products).

Prints ONE JSON line. Besides the headline it carries:
  roofline      for the kernel with the largest measured time: algorithmic flops per launch /
                its average duration (HIP events around each kernel of every 5th timed step, on the
                launch stream: an event between two kernels holds the second back by ~5 us, so the
                other timed steps carry none),
                against 2516.6 TFLOP/s dense bf16; traffic = HBM bytes per launch from the
                committed rocprofv3 counter summary, or null if that kernel's source changed since
  cpu_baseline  the float64 CPU oracle timed on the host cores over a bounded sample of heads
  workloads     forward-only TFLOPS of the other bf16 workloads and the fp32 workload's latency
                (timed before the headline, followed by the fp16 fwd+bwd extra line at the
                headline's shape, so the headline's warm-up and timed steps run on a GPU whose clock
                has settled for this kind of load; it takes ~100 steps from a change of load)
  shader clock  the gfx clock sampled from the host (amdsmi) during each timed region, or null
  extras        the same kernels on fp16 storage (the long causal forward and the fwd+bwd step), the
                key-split decoding step (one query against 8192 keys, HBM-bound: GB/s), block-sparse
                and variable-length forwards, the step with dropout, head dims 32 / 96 / 256, and two
                small launches (B1 H16 d64, B1 H8 d128, N 2048 causal: the split kernels)
"""
from __future__ import annotations

import argparse
import contextlib
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 flop/clk/CU (dense)
PEAK_FP32_TFLOPS = 157.3
HEADLINE = "fwdbwd_bf16_b4h16n2048d64_causal"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--workload", default=None,
                    help="time only this workload (any name in inputs.WORKLOADS) and print its own JSON line; "
                         "used to profile one kernel at a time")
    ap.add_argument("--decode", action="store_true",
                    help="time only the key-split decoding line (B8 H32, 1 query x 8192 keys, d128) for --steps "
                         "calls and print its JSON line; used to profile the HBM-bound kernel")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run --steps plain device copies of 256 MiB (reference for the HBM byte counters)")
    return ap.parse_args()


def traffic_for(workload: str, kernel: str):
    """HBM bytes per launch from the committed counter summary, if it matches the current source."""
    from io_aware_flashattention_flash_amd.profiling import source_digest

    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get("workloads", {}).get(workload, {}).get(kernel)
    except (OSError, ValueError, AttributeError):
        return None
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


class ClockSampler:
    """Samples the GPU's current shader (gfx) clock in MHz from a host thread while a timed region
    runs (amdsmi's read-only clock query, every 10 ms). The device is matched to torch's by PCI bus
    id. If the query is unavailable the summary is None; nothing else depends on it.

    The figure is the one the power-management firmware reports, not a clock measured on the
    engines. It reads 2.0-2.4 GHz during the long workloads and the headline step, but the idle
    level (~170 MHz) throughout the short d = 64 and fp32 workloads, even over 0.2-0.3 s of
    back-to-back launches whose throughput shows the engines running at full clock. The summary uses
    only samples taken at least SKIP_S after the window opened, and timed_calls keeps the GPU loaded
    for at least WINDOW_MS while a sampler is open."""

    WINDOW_MS = 300.0
    SKIP_S = 0.15

    def __init__(self, props):
        self.samples, self._stop, self._thread, self._handle = [], None, None, None
        try:
            import amdsmi

            amdsmi.amdsmi_init()
            want = getattr(props, "pci_bus_id", None)
            handles = amdsmi.amdsmi_get_processor_handles()
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)
                if (want is None and len(handles) == 1) or (want is not None and int(bdf.split(":")[1], 16) == want):
                    self._handle = h
                    break
            self._amdsmi = amdsmi
        except Exception:
            self._handle = None

    def _read(self):
        info = self._amdsmi.amdsmi_get_clock_info(self._handle, self._amdsmi.AmdSmiClkType.GFX)
        return float(info["clk"])

    def __enter__(self):
        import threading

        self.samples = []
        if self._handle is None:
            return self
        self._stop = threading.Event()

        t0 = time.perf_counter()

        def run():
            while not self._stop.is_set():
                try:
                    self.samples.append((time.perf_counter() - t0, self._read()))
                except Exception:
                    return
                self._stop.wait(0.01)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        t = sorted(mhz for when, mhz in self.samples if when >= self.SKIP_S)
        if not t:
            return None
        return {"median_mhz": t[len(t) // 2], "min_mhz": t[0], "max_mhz": t[-1], "samples": len(t),
                "window_s": round(self.samples[-1][0], 3)}


TORCH_DTYPE = {"bf16": "bfloat16", "fp16": "float16", "fp32": "float32"}
# Extra lines (not workloads of the metric): the fp16 storage path on the same shapes.
EXTRAS = ("fwd_fp16_b2h32n4096d128_causal", "fwdbwd_fp16_b4h16n2048d64_causal")


def extra_workload(name):
    from io_aware_flashattention_flash_amd import inputs

    base = inputs.WORKLOADS[name.replace("fp16", "bf16")]
    return inputs.Workload(name, "fp16", base.B, base.H, base.N, base.d, base.causal, base.backward, base.q_mult)


SETTLE_MS = 30.0  # GPU time of untimed calls enqueued right before every timed run


def timed_calls(call, reps, warmup, clock=None):
    """Average ms per call of `reps` back-to-back calls between two HIP events (reps=None: about
    0.3 s of calls). Before them, untimed calls covering SETTLE_MS of GPU time are enqueued with no
    host synchronisation in between: after an idle gap of >= 5 ms the GPU runs its first ~10 ms of
    work in a slower transient, which the timed calls would otherwise include. Returns (ms, reps)."""
    import torch

    for _ in range(warmup):
        call()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    call()
    b.record()
    torch.cuda.synchronize()
    one = max(a.elapsed_time(b), 1e-3)
    if reps is None:
        reps = int(min(2000, max(20, 300.0 / one)))
    settle_ms = SETTLE_MS
    if clock is not None:  # the sampler needs a longer loaded window than short workloads' timed calls
        settle_ms = max(settle_ms, ClockSampler.WINDOW_MS - reps * one)
    settle = int(min(50000, max(1, settle_ms / one)))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with (clock if clock is not None else contextlib.nullcontext()):
        for _ in range(settle):
            call()
        a.record()
        for _ in range(reps):
            call()
        b.record()
        torch.cuda.synchronize()
    return a.elapsed_time(b) / reps, reps


def time_forward(name, reps, warmup, dev, to_dev, wl=None, cold=False, clock=None):
    """Forward-only timing of one workload (HIP events around `reps` back-to-back launches; the
    shader clock is sampled over them when a ClockSampler is given)."""
    import torch

    from io_aware_flashattention_flash_amd import flash_attn_fwd, inputs

    wl = inputs.WORKLOADS[name] if wl is None else wl
    xi = inputs.make_inputs(wl)
    dt = getattr(torch, TORCH_DTYPE[wl.dtype])
    qi, ki, vi = (to_dev(xi[n], dt) for n in ("q", "k", "v"))
    oi = torch.empty_like(qi)
    li = torch.empty(wl.B, wl.H, wl.N, device=dev)
    def call():
        flash_attn_fwd(qi, ki, vi, wl.scale, wl.causal, out=oi, lse=li)

    ms, reps = timed_calls(call, reps, warmup, clock)
    us = ms * 1e3
    tf = wl.fwd_flops() / (us * 1e-6) / 1e12
    peak = PEAK_FP32_TFLOPS if wl.dtype == "fp32" else PEAK_BF16_TFLOPS  # fp16 dense MFMA peak = bf16's
    nbytes = wl.B * wl.H * (4 * wl.N * wl.d * (4 if wl.dtype == "fp32" else 2) + 4 * wl.N)
    out = {"workload": name, "pass": "fwd", "reps": reps, "us": round(us, 2), "tflops": round(tf, 1),
           "pct_of_peak": round(100 * tf / peak, 2), "gbps_algorithmic": round(nbytes / (us * 1e-6) / 1e9, 1)}
    if clock is not None:
        out["shader_clock"] = clock.summary()

    # per-call distribution: each of 50 calls bracketed by its own events (warm caches)
    p10, p50, p90 = percentiles_us(call, 50)
    out.update({"p10_us": p10, "p50_us": p50, "p90_us": p90})
    if cold:
        # cold caches: before each timed call, a fill kernel writes 1 GiB (more than the 256 MB
        # MALL plus the L2s), evicting Q, K, V; only the attention call is inside the events
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        c10, c50, c90 = percentiles_us(call, 20, before=flush.zero_)
        out.update({"cold_p50_us": c50, "cold_p10_us": c10, "cold_p90_us": c90,
                    "cold_tflops": round(wl.fwd_flops() / (c50 * 1e-6) / 1e12, 2)})
        del flush
    return out


def percentiles_us(call, n, before=None):
    """(p10, p50, p90) in microseconds of `call`, each run bracketed by its own HIP events on the
    current stream; `before` (untimed) runs ahead of each call."""
    import torch

    evs = []
    for _ in range(n):
        if before is not None:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        call()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    pick = lambda q: round(t[min(len(t) - 1, int(q * len(t)))], 2)
    return pick(0.1), pick(0.5), pick(0.9)


def time_decode(B, H, Nk, d, reps, dev):
    """Key-split forward of one query per (batch, head) against Nk keys (auto split count): the
    HBM-bound decoding step. Algorithmic bytes: K and V once, plus Q, O and LSE."""
    import torch

    from io_aware_flashattention_flash_amd import flash_attn_fwd_kvsplit, flash_attn_fwd_kvsplit_workspace_size, inputs

    q = torch.from_numpy(inputs.random_tensor((B, H, 1, d), 31)).to(dev).to(torch.bfloat16)
    k = torch.from_numpy(inputs.random_tensor((B, H, Nk, d), 32)).to(dev).to(torch.bfloat16)
    v = torch.from_numpy(inputs.random_tensor((B, H, Nk, d), 33)).to(dev).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, 1, device=dev)
    ws = torch.empty(flash_attn_fwd_kvsplit_workspace_size(B, H, 1, Nk, d, 0, 1), dtype=torch.uint8, device=dev)
    ms, reps = timed_calls(lambda: flash_attn_fwd_kvsplit(q, k, v, None, False, 0, out=o, lse=lse, workspace=ws),
                           reps, 10)
    us = ms * 1e3
    nbytes = B * H * (2 * Nk * d * 2 + 2 * d * 2 + 4)
    return {"workload": f"decode_bf16_b{B}h{H}nq1nk{Nk}d{d}", "pass": "fwd (key-split + merge)", "reps": reps,
            "us": round(us, 2), "gbps_algorithmic": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 8e12, 2)}


def time_masked_forward(kind, B, H, N, d, dev, reps=100):
    """Forward under a mask: "blocksparse" (causal; a seeded map enabling about half of the 128 x 128
    blocks, diagonal blocks always on) or "varlen" (causal; seeded lengths uniform in [N/4, N]).
    TFLOPS counts 4 d flops per visible (query, key) pair only."""
    import numpy as np
    import torch

    from io_aware_flashattention_flash_amd import flash_attn_fwd_masked, inputs

    q, k, v = (torch.from_numpy(inputs.random_tensor((B, H, N, d), 41 + i)).to(dev).to(torch.bfloat16)
               for i in range(3))
    rng = np.random.default_rng(43)
    nb = -(-N // 128)
    sl = bm = None
    if kind == "blocksparse":
        bmap = (rng.random((B, H, nb, nb)) < 0.5).astype(np.uint8)
        bmap[:, :, np.arange(nb), np.arange(nb)] = 1
        # visible pairs: enabled blocks on or below the diagonal, causal inside diagonal blocks
        rows = np.minimum(128, N - 128 * np.arange(nb))  # rows (= keys) per block
        diag = np.array([r * (r + 1) // 2 for r in rows])
        below = np.tril(np.ones((nb, nb), dtype=bool), -1)
        pairs = int(np.einsum("bhrc,r,c->", ((bmap != 0) & below).astype(np.int64), rows, rows) + B * H * diag.sum())
        bm = torch.from_numpy(bmap).to(dev)
    else:
        lens = rng.integers(N // 4, N + 1, size=B).astype(np.int32)
        pairs = int(H * sum(int(L) * (int(L) + 1) // 2 for L in lens))
        sl = torch.from_numpy(lens).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    ms, reps = timed_calls(lambda: flash_attn_fwd_masked(q, k, v, None, True, seqlens=sl, block_mask=bm, out=o,
                                                         lse=lse), reps, 10)
    us = ms * 1e3
    tf = 4.0 * d * pairs / (us * 1e-6) / 1e12
    return {"workload": f"fwd_bf16_b{B}h{H}n{N}d{d}_causal_{kind}", "pass": "fwd (masked)", "reps": reps,
            "us": round(us, 2), "visible_pairs": pairs, "tflops_visible": round(tf, 1),
            "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}


def time_dropout_step(B, H, N, d, p, dev, reps=50):
    """Forward + backward (dQ, then dK/dV) of causal attention with dropout probability p, through
    the masked entry points; flops counted as for the dense step (dropout adds none)."""
    import torch

    from io_aware_flashattention_flash_amd import flash_attn_bwd_masked, flash_attn_fwd_masked, inputs

    q, k, v, do = (torch.from_numpy(inputs.random_tensor((B, H, N, d), 51 + i)).to(dev).to(torch.bfloat16)
                   for i in range(4))
    o = torch.empty_like(q)
    lse = torch.empty(B, H, N, device=dev)
    grads = [torch.empty_like(q) for _ in range(3)]
    ws = torch.empty(4 * B * H * N + 256, dtype=torch.uint8, device=dev)

    def step(seed):
        flash_attn_fwd_masked(q, k, v, None, True, out=o, lse=lse, dropout_p=p, seed=seed)
        flash_attn_bwd_masked(do, q, k, v, o, lse, None, True, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws,
                              dropout_p=p, seed=seed)

    seeds = itertools.count()
    ms, reps = timed_calls(lambda: step(next(seeds)), reps, 5)
    us = ms * 1e3
    flops = 3.5 * 4.0 * B * H * N * N * d / 2
    return {"workload": f"fwdbwd_bf16_b{B}h{H}n{N}d{d}_causal_dropout{p}", "pass": "fwd+bwd (dropout)", "reps": reps,
            "us": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 1)}


def prepare_fwdbwd(w, x, dev, to_dev):
    """Device tensors for the fwd+bwd step of a 16-bit workload, and the step itself (forward, dQ
    with delta, dK/dV) with optional HIP events between the stages."""
    import torch

    from io_aware_flashattention_flash_amd import flash_attn_bwd_dkdv, flash_attn_bwd_dq, flash_attn_fwd

    dt = getattr(torch, TORCH_DTYPE[w.dtype])
    q, k, v, do = (to_dev(x[n], dt) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step(evs=None):
        if evs is not None:
            evs[0].record()
        flash_attn_fwd(q, k, v, w.scale, w.causal, out=o, lse=lse)
        if evs is not None:
            evs[1].record()
        flash_attn_bwd_dq(q, k, v, o, lse, do, w.scale, w.causal, dq=dq, delta=delta)
        if evs is not None:
            evs[2].record()
        flash_attn_bwd_dkdv(q, k, v, lse, do, delta, w.scale, w.causal, dk=dk, dv=dv)
        if evs is not None:
            evs[3].record()

    step.outputs = (o, dq)
    return step


def one_step_ms(step, warmup):
    """GPU time of one call of `step` (events around it), after `warmup` untimed calls."""
    import torch

    for _ in range(warmup):
        step()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    step()
    b.record()
    torch.cuda.synchronize()
    return max(a.elapsed_time(b), 1e-3)


def auto_steps(step, warmup, seconds=0.3):
    """Steps of `step` that take about `seconds` (after `warmup` untimed ones)."""
    return int(min(3000, max(20, seconds * 1e3 / one_step_ms(step, warmup))))


class KernelEvent:
    """A HIP timing event created with hipEventDisableSystemFence, for the events between kernels:
    recording a default event performs a system-scope cache write-back and invalidation, which
    holds the next kernel back and adds ~2 us to each duration measured between such events.
    Same interface as torch.cuda.Event (record on torch's current stream, elapsed_time in ms). The
    calls go to the HIP runtime torch has loaded (a second copy of the runtime would not know torch's
    streams). The events live until the process ends."""

    DISABLE_SYSTEM_FENCE = 0x20000000
    _hip = None

    @classmethod
    def runtime(cls):
        if cls._hip is None:
            import ctypes

            with open("/proc/self/maps") as f:
                paths = [ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln]
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            cls._hip = ctypes.CDLL(paths[0])
        return cls._hip

    def __init__(self):
        import ctypes

        self._h = ctypes.c_void_p()
        if self.runtime().hipEventCreateWithFlags(ctypes.byref(self._h), ctypes.c_uint(self.DISABLE_SYSTEM_FENCE)):
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        import ctypes

        import torch

        if self.runtime().hipEventRecord(self._h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)):
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, other):
        import ctypes

        ms = ctypes.c_float()
        if self.runtime().hipEventElapsedTime(ctypes.byref(ms), self._h, other._h):
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value


class TimedSteps:
    """K steps of a fwd+bwd step between two HIP events on the stream, enqueued without waiting.
    Every `sample_every`-th step also records fence-free events (KernelEvent) between its three
    kernels (forward, dQ, dK/dV); each still costs the next kernel a little, so sampling a subset
    keeps that off most steps while timing each kernel inside the timed region."""

    NAMES = ("fwd", "bwd_dq", "bwd_dkdv")

    def __init__(self, step, steps, sample_every=1):
        import torch

        self.step, self.steps = step, steps
        self.sampled = [i for i in range(steps) if i % sample_every == sample_every - 1] or [steps - 1]
        try:
            make = KernelEvent
            make()
            self.event_kind = "HIP events (hipEventDisableSystemFence)"
        except (RuntimeError, OSError, AttributeError):  # the HIP runtime's entry points are not reachable
            make = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
            self.event_kind = "HIP events (torch, default flags)"
        self.kev = {i: [make() for _ in range(4)] for i in self.sampled}
        self.t0 = torch.cuda.Event(enable_timing=True)
        self.t1 = torch.cuda.Event(enable_timing=True)

    def enqueue(self):
        self.t0.record()
        for i in range(self.steps):
            self.step(self.kev.get(i))
        self.t1.record()

    def result(self):
        """(ms per step, {kernel: average ms over the sampled steps}); waits for the GPU."""
        import torch

        torch.cuda.synchronize()
        ms_step = self.t0.elapsed_time(self.t1) / self.steps
        kern = {n: sum(e[j].elapsed_time(e[j + 1]) for e in self.kev.values()) / len(self.kev)
                for j, n in enumerate(self.NAMES)}
        o, dq = self.step.outputs
        if not (torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()):
            raise RuntimeError("non-finite output in the benchmark step")
        return ms_step, kern


def run_fwdbwd(step, steps, warmup, clock=None, sample_every=1):
    """Times `steps` steps (steps=None: about 0.3 s of steps) after `warmup` untimed ones and
    SETTLE_MS of untimed steps enqueued right before them (see timed_calls). Returns (ms per step,
    {stage: average ms})."""
    one_ms = one_step_ms(step, warmup)
    if steps is None:
        steps = int(min(3000, max(20, 300.0 / one_ms)))
    timed = TimedSteps(step, steps, sample_every)
    with (clock if clock is not None else contextlib.nullcontext()):
        for _ in range(int(min(2000, max(1, SETTLE_MS / one_ms)))):
            step()
        timed.enqueue()
        return timed.result()


def time_fwdbwd(w, x, steps, warmup, dev, to_dev, clock=None):
    """prepare_fwdbwd + run_fwdbwd for one 16-bit workload."""
    return run_fwdbwd(prepare_fwdbwd(w, x, dev, to_dev), steps, warmup, clock)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus must be 1 (no multi-GPU path exists)"}))
        sys.exit(2)

    import torch

    from io_aware_flashattention_flash_amd import inputs, load_library

    load_library()  # raises if the HIP library is not built
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)

    def to_dev(a, dt):
        return torch.from_numpy(a).to(dev).to(dt)

    if args.copy_calibration:
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": max(1, args.steps)}))
        return

    if args.decode:
        print(json.dumps(time_decode(8, 32, 8192, 128, args.steps, dev)))
        return
    if args.workload is not None and args.workload != HEADLINE:
        print(json.dumps(time_forward(args.workload, args.steps, args.warmup, dev, to_dev)))
        return

    clock = ClockSampler(props)

    # ------------------------------------------------------------------ forward-only workloads
    # (timed first: their ~0.3 s runs of back-to-back launches also take the GPU out of its idle
    # clock state before the headline's warm-up steps)
    workloads = {}
    if not args.no_workloads:
        for name, wl in inputs.WORKLOADS.items():
            if not wl.backward:
                # the short workloads (N <= 1024) also get cold-cache timings
                workloads[name] = time_forward(name, None, 10, dev, to_dev, cold=wl.N <= 1024, clock=clock)
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ headline inputs
    # Everything the headline needs is built before the fp16 line runs, so the GPU goes from that
    # line straight into the headline. After an idle gap (host work) the GPU runs a few fast steps,
    # then 10-17% slower ones for ~50 steps, then settles (measured on this step); a short run of
    # 5 warm-up + 20 timed steps would sit in that transient.
    w = inputs.WORKLOADS[HEADLINE]
    x = inputs.make_inputs(w)
    headline_step = prepare_fwdbwd(w, x, dev, to_dev)

    # ------------------------------------------------------------------ fp16 fwd+bwd extra line
    # (the headline's shape on fp16 storage, about 0.3 s of steps, enqueued so that the headline's
    # warm-up steps follow it on the GPU without an idle gap)
    extras = {}
    fp16 = None
    fp16_step = None
    if not args.no_workloads:
        name = "fwdbwd_fp16_b4h16n2048d64_causal"
        wl16 = extra_workload(name)
        fp16_step = prepare_fwdbwd(wl16, inputs.make_inputs(wl16), dev, to_dev)

    # ------------------------------------------------------------------ headline: fwd + bwd
    # W untimed warm-up steps, a synchronisation, then exactly K timed steps between two events and
    # a final synchronisation. Every 5th timed step also times its three kernels (the roofline's
    # kernel durations, measured inside the timed region). The clock sampler opens before the fp16
    # line, whose ~0.3 s of steps keep the GPU loaded up to the headline (see ClockSampler).
    timed = TimedSteps(headline_step, args.steps, sample_every=5)
    with clock:
        if fp16_step is not None:
            fp16 = TimedSteps(fp16_step, auto_steps(fp16_step, 10))
            fp16.enqueue()
        for _ in range(args.warmup):
            headline_step()
        torch.cuda.synchronize()
        timed.enqueue()
        ms_step, kern_ms = timed.result()
    headline_clock = clock.summary()
    if fp16 is not None:
        ms, km = fp16.result()
        extras[name] = {"workload": name, "pass": "fwd+bwd", "us": round(ms * 1e3, 2),
                        "tflops": round((wl16.fwd_flops() + wl16.bwd_flops()) / (ms * 1e-3) / 1e12, 1),
                        "kernels_us": {n: round(t * 1e3, 2) for n, t in km.items()}}
        del fp16, fp16_step
    names = ["fwd", "bwd_dq", "bwd_dkdv"]

    f_fwd, f_bwd = w.fwd_flops(), w.bwd_flops()
    value = (f_fwd + f_bwd) / (ms_step * 1e-3) / 1e12
    kflops = {"fwd": f_fwd, "bwd_dkdv": 2.0 * f_fwd, "bwd_dq": 0.5 * f_fwd}
    kbytes = {  # algorithmic HBM bytes per launch (each tensor moved once)
        "fwd": w.B * w.H * (4 * w.N * w.d * 2 + 4 * w.N),
        "bwd_dkdv": w.B * w.H * (6 * w.N * w.d * 2 + 8 * w.N),
        "bwd_dq": w.B * w.H * (6 * w.N * w.d * 2 + 8 * w.N),  # also reads O and writes delta
    }
    dom = max(kern_ms, key=kern_ms.get)
    bound = "hbm" if kflops[dom] == 0 else "mfma"
    if bound == "mfma":
        achieved, peak, unit = kflops[dom] / (kern_ms[dom] * 1e-3) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, unit = kbytes[dom] / (kern_ms[dom] * 1e-3) / 1e9, 8000.0, "GB/s"
    roofline = {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": traffic_for(HEADLINE, dom),
                "algorithmic_flops_per_launch": kflops[dom], "algorithmic_bytes_per_launch": kbytes[dom],
                "avg_launch_us": round(kern_ms[dom] * 1e3, 2),
                "launch_timing": f"{timed.event_kind} around each kernel on "
                                 f"{len(timed.sampled)} of the {args.steps} timed steps (every 5th)"}
    kernels = {n: {"avg_us": round(kern_ms[n] * 1e3, 2),
                   "tflops": round(kflops[n] / (kern_ms[n] * 1e-3) / 1e12, 1) if kflops[n] else None,
                   "gbps_algorithmic": round(kbytes[n] / (kern_ms[n] * 1e-3) / 1e9, 1)} for n in names}
    bwd_ms = kern_ms["bwd_dkdv"] + kern_ms["bwd_dq"]

    # ------------------------------------------------------------------ the other extra lines
    if not args.no_workloads:
        for name in EXTRAS:
            wl = extra_workload(name)
            if not wl.backward:  # the fp16 fwd+bwd line was timed before the headline
                extras[name] = time_forward(name, None, 10, dev, to_dev, wl=wl)
        extras["decode_bf16_b8h32nq1nk8192d128"] = time_decode(8, 32, 8192, 128, 200, dev)
        for kind, shape in (("blocksparse", (2, 32, 4096, 128)), ("varlen", (8, 16, 4096, 128))):
            r = time_masked_forward(kind, *shape, dev)
            extras[r["workload"]] = r
        r = time_dropout_step(4, 16, 2048, 64, 0.1, dev)
        extras[r["workload"]] = r
        # head dims beyond 64 / 128: the causal forward at the 4096-token shape (same tokens x d as
        # the d = 128 workload) and the headline fwd+bwd step shape
        for d in (32, 96, 256):
            fw = inputs.Workload(f"fwd_bf16_b2h32n4096d{d}_causal", "bf16", 2, 32, 4096, d, True, False)
            extras[fw.name] = time_forward(fw.name, None, 10, dev, to_dev, wl=fw)
            bw = inputs.Workload(f"fwdbwd_bf16_b4h16n2048d{d}_causal", "bf16", 4, 16, 2048, d, True, True)
            ms, km = time_fwdbwd(bw, inputs.make_inputs(bw), 30, 5, dev, to_dev)
            extras[bw.name] = {"workload": bw.name, "pass": "fwd+bwd", "us": round(ms * 1e3, 2),
                               "tflops": round((bw.fwd_flops() + bw.bwd_flops()) / (ms * 1e-3) / 1e12, 1),
                               "kernels_us": {n: round(t * 1e3, 2) for n, t in km.items()}}
            torch.cuda.empty_cache()
        # small launches (their workgroups fit on the chip at once: the split kernels)
        for B, H, d in ((1, 16, 64), (1, 8, 128)):
            bw = inputs.Workload(f"fwdbwd_bf16_b{B}h{H}n2048d{d}_causal", "bf16", B, H, 2048, d, True, True)
            ms, km = time_fwdbwd(bw, inputs.make_inputs(bw), 30, 5, dev, to_dev)
            extras[bw.name] = {"workload": bw.name, "pass": "fwd+bwd", "us": round(ms * 1e3, 2),
                               "tflops": round((bw.fwd_flops() + bw.bwd_flops()) / (ms * 1e-3) / 1e12, 1),
                               "kernels_us": {n: round(t * 1e3, 2) for n, t in km.items()}}
        torch.cuda.empty_cache()

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attn_bwd, attn_fwd
        affinity = len(os.sched_getaffinity(0))
        try:
            from threadpoolctl import threadpool_info
            blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
        except Exception:
            blas = None
        cores = blas if blas is not None else affinity
        heads = [(b, h) for b in range(w.B) for h in range(w.H)]
        done = 0
        c0 = time.perf_counter()
        for b, h in heads:
            sl = (slice(b, b + 1), slice(h, h + 1))
            attn_fwd(x["q"][sl], x["k"][sl], x["v"][sl], w.scale, True)
            attn_bwd(x["q"][sl], x["k"][sl], x["v"][sl], x["do"][sl], w.scale, True)
            done += 1
            if time.perf_counter() - c0 >= args.cpu_seconds:
                break
        secs = time.perf_counter() - c0
        per_head = (f_fwd + f_bwd) / len(heads)
        cpu = {"value": round(per_head * done / secs / 1e12, 6), "unit": "TFLOPS", "cores": cores,
               "cores_meaning": "BLAS threads that ran the oracle's matrix products (NumPy's exp runs on one)",
               "blas_threads": blas, "affinity_cores": affinity, "kind": "oracle",
               "sample": f"float64 oracle forward+backward on {done} of {len(heads)} (batch, head) slices of "
                         f"{HEADLINE}, {secs:.1f} s; value scaled by the workload's flop count per head"}

    out = {
        "metric": "attention TFLOPS (fwd, fwd+bwd) and % of MI355X dense bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q, K, V, dO rounded to bf16 (numpy default_rng(0))",
        "config": {"workload": HEADLINE, "pass": "fwd+bwd", "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": True, "scale": w.scale},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(f_fwd / (kern_ms["fwd"] * 1e-3) / 1e12, 1),
        "bwd_tflops": round(f_bwd / (bwd_ms * 1e-3) / 1e12, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "workloads": workloads,
        "extras": extras,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""), "cus": props.multi_processor_count,
                   "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)},
        "shader_clock_headline": headline_clock,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
