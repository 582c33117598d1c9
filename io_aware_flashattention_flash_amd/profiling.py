"""Turn rocprofv3 output into the short text summaries kept under profiles/.

  python -m io_aware_flashattention_flash_amd.profiling trace STATS_CSV OUT_MD "COMMAND" "TITLE" [--bench-json F]
      kernel-trace summary (calls, average / min / max duration, share) of this library's kernels;
      with --bench-json, the traced bench.py run's own output line is appended for comparison, and
      with --plain-json that of the same command run without the profiler

  python -m io_aware_flashattention_flash_amd.profiling traffic --copy-fetch DIR --copy-write DIR \
      --copy-bytes N --run WORKLOAD FETCH_DIR WRITE_DIR KERNEL_STATS_CSV [--run ...] \
      --out-json JSON --out-md MD --commands "..."
      HBM traffic per launch of each attention kernel of each workload from FETCH_SIZE / WRITE_SIZE
      (KiB per dispatch), each scaled by what the same counter reports for a plain device copy of N
      bytes (bench.py --copy-calibration); set against the kernel's algorithmic bytes (each tensor
      moved once: the ratio of fetched to algorithmic read bytes is the re-read factor of K/V tiles
      that reach past L2) and, with the kernel's average duration from the same workload's kernel
      trace, as GB/s. Stored with a digest of the kernel's source so that a stale figure is never
      reported for a changed kernel.

  python -m io_aware_flashattention_flash_amd.profiling counters --run LABEL DIR WORKLOAD ... \
      --out-md MD --commands "..."
      MFMA / VALU / LDS counter summary, one counter pass per workload
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
from collections import defaultdict

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = {"fwd": "fa_fwd_16bit.hip", "fwd_fp32": "fa_fwd_fp32.hip", "bwd_dq": "fa_bwd_16bit.hip",
                  "bwd_dkdv": "fa_bwd_16bit.hip", "fwd_kvsplit": "fa_fwd_16bit.hip",
                  "kvsplit_merge": "fa_fwd_16bit.hip"}
KERNEL_PREFIX = {"fwd": ("fa::fwd16_kernel",), "fwd_fp32": ("fa::fwd_fp32_kernel", "fa::fwd_fp32_split_kernel"),
                 "bwd_dq": ("fa::bwd_dq_kernel",), "bwd_dkdv": ("fa::bwd_dkdv_kernel",),
                 "kvsplit_merge": ("fa::kvsplit_merge_kernel",)}
KSPLIT_MODE = 1  # the forward kernel's sixth template argument (its launch mode) in key-split launches


class Decode:
    """A key-split forward workload (Nq queries against Nk keys), as bench.py --decode times it."""

    def __init__(self, B, H, Nq, Nk, d):
        self.B, self.H, self.Nq, self.Nk, self.d = B, H, Nq, Nk, d


DECODE = {"decode_bf16_b8h32nq1nk8192d128": Decode(8, 32, 1, 8192, 128)}


def workload(name: str):
    from . import inputs

    return DECODE[name] if name in DECODE else inputs.WORKLOADS[name]


def source_digest(kernel: str) -> str:
    """Digest of the source file that defines `kernel` plus the shared device headers."""
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "fa_device.h", "fa_launch.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_TEMPLATE_ARG = re.compile(r"DF16b|DF16_|Li(-?\d+)E|Lb([01])E")


def readable_name(name: str) -> str:
    """This library's kernel names as `fa::kernel<args>`. The profiler reports some template
    instances undemangled (the bf16 / fp16 element types); their Itanium-mangled form
    _ZN2fa<len><name>I<args>E... is rendered here for the handful of argument kinds the
    kernels use (16-bit float types, int and bool constants)."""
    short = name.replace("void ", "").split("(")[0]
    m = re.match(r"_ZN2fa(\d+)", short)
    if not m:
        return short
    n = int(m.group(1))
    start = m.end()
    fn = short[start:start + n]
    rest = short[start + n:]
    if not rest.startswith("I"):
        return f"fa::{fn}"
    args = []
    for a in _TEMPLATE_ARG.finditer(rest[1:rest.index("EE") + 1] if "EE" in rest else rest[1:]):
        tok = a.group(0)
        args.append("bf16" if tok == "DF16b" else "f16" if tok == "DF16_" else
                    a.group(1) if a.group(1) is not None else ("true" if a.group(2) == "1" else "false"))
    return f"fa::{fn}<{', '.join(args)}>"


def kernel_key(name: str):
    short = readable_name(name)
    if short.startswith("fa::fwd16_kernel<"):
        args = short[len("fa::fwd16_kernel<"):-1].split(", ")
        if len(args) > 5 and args[5] == str(KSPLIT_MODE):
            return "fwd_kvsplit"
    for key, prefixes in KERNEL_PREFIX.items():
        if any(short.startswith(prefix + "<") for prefix in prefixes):
            return key
    return None


def algorithmic_bytes(w, kernel: str):
    """(read, write) bytes of one launch of `kernel` on workload w when every tensor crosses HBM once:
    forward reads Q, K, V and writes O and LSE; dQ reads Q, K, V, O, dO, LSE and writes dQ and delta;
    dK/dV reads Q, K, V, dO, LSE, delta and writes dK, dV. A key-split forward reads Q, K and V (its
    fp32 partials are scratch, not counted) and its merge writes O and LSE."""
    if isinstance(w, Decode):
        return {"fwd_kvsplit": (w.B * w.H * (w.Nq + 2 * w.Nk) * w.d * 2, 0),
                "kvsplit_merge": (0, w.B * w.H * w.Nq * (w.d * 2 + 4))}[kernel]
    s = 4 if w.dtype == "fp32" else 2
    t, r = w.B * w.H * w.N * w.d * s, w.B * w.H * w.N * 4
    return {"fwd": (3 * t, t + r), "fwd_fp32": (3 * t, t + r), "bwd_dq": (5 * t + r, t + r),
            "bwd_dkdv": (4 * t + 2 * r, 2 * t)}[kernel]


def kernel_names(directory: str) -> dict:
    """Kernel key -> the set of readable kernel names (template instances) in a counter pass."""
    path = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    names = defaultdict(set)
    for row in csv.DictReader(open(path[0])):
        k = kernel_key(row["Kernel_Name"])
        if k is not None:
            names[k].add(readable_name(row["Kernel_Name"]))
    return names


def kernel_avg_us(stats_csv: str, only=None) -> dict:
    """Average duration per attention kernel key from a --kernel-trace --stats kernel_stats.csv
    (calls-weighted over the instances of a key; with `only` (key -> names), over those instances)."""
    tot, calls = defaultdict(float), defaultdict(int)
    for r in csv.DictReader(open(stats_csv)):
        k = kernel_key(r["Name"])
        if k is None or (only is not None and readable_name(r["Name"]) not in only.get(k, ())):
            continue
        tot[k] += float(r["TotalDurationNs"])
        calls[k] += int(r["Calls"])
    return {k: tot[k] / calls[k] / 1e3 for k in tot}


def counter_per_dispatch(directory: str, counter: str, match) -> dict:
    """Average of `counter` per dispatch for every kernel name accepted by `match` (name -> key)."""
    path = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not path:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    total, dispatches = defaultdict(float), defaultdict(set)
    for row in csv.DictReader(open(path[0])):
        if row["Counter_Name"] != counter:
            continue
        key = match(row["Kernel_Name"])
        if key is None:
            continue
        total[key] += float(row["Counter_Value"])
        dispatches[key].add(row["Dispatch_Id"])
    return {k: total[k] / len(dispatches[k]) for k in total}


def _bench_json(bench_json: str) -> dict:
    with open(bench_json) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def _bench_line(bench_json: str) -> str:
    d = _bench_json(bench_json)
    if "roofline" not in d:  # a single timed line (bench.py --decode)
        return (f"{d['workload']}: {d['us']} µs per call ({d['reps']} calls back to back between two events), "
                f"{d['gbps_algorithmic']} GB/s algorithmic = {d['pct_of_hbm_peak']}% of the 8 TB/s HBM peak.")
    r = d["roofline"]
    kern = ", ".join(f"{n} {k['avg_us']:.2f} µs" for n, k in d["kernels"].items())
    return (f"value {d['value']} {d['unit']}, {d['ms_per_step']} ms per step; per-kernel event averages "
            f"({r.get('launch_timing', 'HIP events')}): {kern}; roofline kernel {r['kernel']}, {r['achieved']} "
            f"{r['unit']} of {r['peak']}, frac {r['frac']}.")


def bench_line_section(bench_json: str, plain_json: str = None) -> list:
    """The bench line printed by the traced run itself and, if given, that of the same command run
    without the profiler just before on the same box: throughput, per-kernel event averages and
    roofline fraction, for comparison with the trace's durations."""
    lines = ["", "## The traced run's bench line", "", _bench_line(bench_json)]
    if "roofline" in _bench_json(bench_json):
        lines += ["", "An event pair around one kernel also spans that launch's dispatch gap after the previous "
                  "kernel, which the profiler lengthens (it adds work to every dispatch); the trace's durations are "
                  "the kernels' own. The trace's averages of the headline's kernel instances also include its "
                  "warm-up steps."]
    else:
        lines += ["", "The events span both launches of each call (key-split forward and merge) and the gaps "
                  "between them, which the profiler lengthens."]
    if plain_json:
        lines += ["", "## The same command without the profiler (same box, just before)", "", _bench_line(plain_json)]
    return lines


def trace(stats_csv: str, out_md: str, command: str, title: str, bench_json: str = None,
          plain_json: str = None) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        short = readable_name(r["Name"])
        if not short.startswith("fa::"):
            continue
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
    if bench_json:
        lines += bench_line_section(bench_json, plain_json)
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def traffic(a) -> dict:
    # the runtime's device-to-device blit kernel that a same-device torch copy launches
    copy = lambda n: "copy" if "copybuffer" in n.lower() else None
    cf = counter_per_dispatch(a.copy_fetch, "FETCH_SIZE", copy).get("copy")
    cw = counter_per_dispatch(a.copy_write, "WRITE_SIZE", copy).get("copy")
    if not cf or not cw:
        raise RuntimeError("copy calibration kernel not found in the counter output")
    # a copy of N bytes fetches N and writes N: KiB reported per byte moved
    f_scale, w_scale = cf * 1024.0 / a.copy_bytes, cw * 1024.0 / a.copy_bytes
    out = {"_calibration": {"copy_bytes": a.copy_bytes, "fetch_kib_per_dispatch": cf, "write_kib_per_dispatch": cw,
                            "fetch_scale": f_scale, "write_scale": w_scale}, "workloads": {}}
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated), every workload", "",
             "Commands (run from the repository root on one MI355X; one counter per pass):", "", "```",
             a.commands, "```", "",
             f"Calibration: a device copy of {a.copy_bytes} bytes reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE "
             f"{cw:.0f} KiB per dispatch, i.e. {f_scale:.4f} / {w_scale:.4f} of the bytes moved; kernel figures "
             "below are divided by these factors. FETCH_SIZE counts L2 misses sent to the fabric, some of which "
             "the 256 MB Infinity Cache serves, so it bounds HBM reads from above. Algorithmic bytes move every "
             "tensor once; fetched / algorithmic read bytes is the factor by which K/V (and Q/dO) tiles are "
             "re-read past L2. GB/s divide the bytes by the kernel's average duration in the same workload's "
             "kernel trace.", "",
             "| workload | kernel | fetch MB | write MB | algorithmic read / write MB | fetch / algorithmic read | "
             "avg µs | counter GB/s | algorithmic GB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for wname, fdir, wdir, stats in a.run:
        w = workload(wname)
        fetch = counter_per_dispatch(fdir, "FETCH_SIZE", kernel_key)
        write = counter_per_dispatch(wdir, "WRITE_SIZE", kernel_key)
        # the trace's averages over the same kernel instances the counter pass ran
        avg = kernel_avg_us(stats, kernel_names(fdir)) if stats != "-" else {}
        entry = {}
        for k in sorted(set(fetch) & set(write)):
            fb, wb = fetch[k] * 1024.0 / f_scale, write[k] * 1024.0 / w_scale
            ar, aw = algorithmic_bytes(w, k)
            e = {"source_digest": source_digest(k), "fetch_bytes_per_launch": round(fb),
                 "write_bytes_per_launch": round(wb), "bytes_per_launch": round(fb + wb),
                 "algorithmic_read_bytes": ar, "algorithmic_write_bytes": aw,
                 "fetch_over_algorithmic_read": round(fb / ar, 3) if ar else None}
            us = avg.get(k)
            if us:
                e.update({"avg_us": round(us, 2), "counter_gbps": round((fb + wb) / (us * 1e-6) / 1e9, 1),
                          "algorithmic_gbps": round((ar + aw) / (us * 1e-6) / 1e9, 1)})
            entry[k] = e
            ratio = f"{fb / ar:.2f}" if ar else "–"
            lines.append(f"| {wname} | {k} | {fb / 1e6:.2f} | {wb / 1e6:.2f} | {ar / 1e6:.2f} / {aw / 1e6:.2f} | "
                         f"{ratio} | {e.get('avg_us', '–')} | {e.get('counter_gbps', '–')} | "
                         f"{e.get('algorithmic_gbps', '–')} |")
        out["workloads"][wname] = entry
    with open(a.out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


# One counter pass per workload (at most 8 SQ and 2 GRBM counters, so they fit a single pass). The
# fp32 workload counts SQ_INSTS_VALU_MFMA_MOPS_F32 in place of the bf16 matrix-op counter.
COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
            "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
COUNTERS_FP32 = COUNTERS.replace("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F32")
N_XCD, N_SIMD = 8, 1024  # MI355X: GRBM_GUI_ACTIVE is summed over the 8 XCDs; 256 CUs x 4 SIMDs


def counter_summary(directory: str, formula_flops: dict) -> list:
    """Per attention kernel in one counter pass: averages per dispatch and the derived figures.

    formula_flops: kernel key -> algorithmic MFMA flops per launch (the workload's counting
    convention). SQ_INSTS_VALU_MFMA_MOPS_BF16 counts matrix work in units of 512 flops, so
    512 x MOPS / formula is the executed-to-counted ratio: about 1 + tile / N for a causal forward
    whose above-diagonal tiles are skipped (2 if they were not), about 3 for dQ (it recomputes S
    and dP beside its one counted product), about 1 for dK/dV."""
    path = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not path:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    total, dispatches = defaultdict(lambda: defaultdict(float)), defaultdict(set)
    for row in csv.DictReader(open(path[0])):
        key = kernel_key(row["Kernel_Name"])
        if key is None:
            continue
        total[key][row["Counter_Name"]] += float(row["Counter_Value"])
        dispatches[key].add(row["Dispatch_Id"])
    out = []
    for key in sorted(total):
        c = {n: v / len(dispatches[key]) for n, v in total[key].items()}
        cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
        mfma_flops = 512.0 * (c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0))
        out.append({
            "kernel": key,
            "dispatches": len(dispatches[key]),
            "gpu_cycles": cycles,
            "mfma_busy_frac": c["SQ_VALU_MFMA_BUSY_CYCLES"] / N_SIMD / cycles,
            "mfma_flops": mfma_flops,
            "executed_over_formula": mfma_flops / formula_flops[key] if key in formula_flops else None,
            "valu_per_mfma": (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / c["SQ_INSTS_MFMA"],
            "lds_instr_per_mfma": c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"],
            "lds_bank_conflict_frac": c["SQ_LDS_BANK_CONFLICT"] / max(1.0, c["SQ_LDS_IDX_ACTIVE"]),
        })
    return out


def counters_md(runs: list, out_md: str, commands: str) -> str:
    """runs: [(workload label, counter directory, {kernel: formula flops})]."""
    lines = ["# MFMA, VALU and LDS counters per attention kernel (rocprofv3 --pmc, one pass per workload)", "",
             "Commands (run from the repository root on one MI355X):", "", "```", commands, "```", "",
             "Derived figures: MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 SIMDs / (GRBM_GUI_ACTIVE / 8 XCDs); "
             "executed / counted = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / the workload's flop formula (causal "
             "forward: about 1 + 128/N when tiles above the diagonal are skipped, 2 if they were not; dQ: "
             "about 3, it recomputes S and dP beside its one counted product); LDS bank conflicts = "
             "SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE. Counts are averages per dispatch.", "",
             "| workload | kernel | dispatches | MFMA busy | executed / counted flops | VALU instr per MFMA | "
             "LDS instr per MFMA | LDS bank-conflict cycles |", "|---|---|---|---|---|---|---|---|"]
    for label, directory, formula in runs:
        for r in counter_summary(directory, formula):
            ratio = "–" if r["executed_over_formula"] is None else f"{r['executed_over_formula']:.3f}"
            lines.append(f"| {label} | {r['kernel']} | {r['dispatches']} | {r['mfma_busy_frac']:.1%} | {ratio} | "
                         f"{r['valu_per_mfma']:.2f} | {r['lds_instr_per_mfma']:.2f} | "
                         f"{r['lds_bank_conflict_frac']:.2%} |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


STALL_COUNTERS = ("SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
                  "SQ_ACTIVE_INST_ANY SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE")


def stall_md(directory: str, out_md: str, title: str, commands: str) -> str:
    """Where each kernel's wave-cycles go, from one counter pass: waiting at s_waitcnt for memory
    or LDS results (SQ_WAIT_ANY), ready but not issued because other waves hold the issue slots
    (SQ_WAIT_INST_ANY; of which waiting to issue an LDS instruction: SQ_WAIT_INST_LDS), and issuing
    (SQ_ACTIVE_INST_ANY; of which VALU and LDS). The three parts add up to the wave-cycles."""
    path = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not path:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    tot, disp = defaultdict(lambda: defaultdict(float)), defaultdict(set)
    for row in csv.DictReader(open(path[0])):
        k = kernel_key(row["Kernel_Name"])
        if k is None:
            continue
        tot[k][row["Counter_Name"]] += float(row["Counter_Value"])
        disp[k].add(row["Dispatch_Id"])
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X; one counter pass):", "", "```",
             commands, "```", "",
             "Shares of each kernel's wave-cycles (SQ_WAVE_CYCLES): waiting at `s_waitcnt` for memory or LDS "
             "results (SQ_WAIT_ANY); ready but not issued while other waves use the issue slots "
             "(SQ_WAIT_INST_ANY, of which LDS instructions: SQ_WAIT_INST_LDS); issuing (SQ_ACTIVE_INST_ANY, "
             "of which VALU and LDS). The first, second and fourth columns add up to 1. MFMA busy: "
             "SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE (summed over the 8 XCDs) times the 1024 SIMDs.", "",
             "| kernel | dispatches | waiting at s_waitcnt | ready, not issued | (LDS) | issuing | (VALU) | (LDS) | MFMA busy |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(tot):
        c, wc = tot[k], tot[k]["SQ_WAVE_CYCLES"]
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (c["GRBM_GUI_ACTIVE"] / N_XCD * N_SIMD) if c["GRBM_GUI_ACTIVE"] else 0.0
        lines.append(f"| {k} | {len(disp[k])} | {c['SQ_WAIT_ANY'] / wc:.3f} | {c['SQ_WAIT_INST_ANY'] / wc:.3f} | "
                     f"{c['SQ_WAIT_INST_LDS'] / wc:.3f} | {c['SQ_ACTIVE_INST_ANY'] / wc:.3f} | "
                     f"{c['SQ_ACTIVE_INST_VALU'] / wc:.3f} | {c['SQ_ACTIVE_INST_LDS'] / wc:.3f} | {100 * busy:.1f}% |")
    text = "\n".join(lines) + "\n"
    with open(out_md, "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_md")
    t.add_argument("command")
    t.add_argument("title")
    t.add_argument("--bench-json", help="the traced bench.py run's output line, appended as a section")
    t.add_argument("--plain-json", help="the same bench.py command's line without the profiler")
    r = sub.add_parser("traffic")
    for name in ("--copy-fetch", "--copy-write", "--out-json", "--out-md", "--commands"):
        r.add_argument(name, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    r.add_argument("--run", nargs=4, action="append", required=True,
                   metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "KERNEL_STATS_CSV"))
    st = sub.add_parser("stalls", help="wave-cycle breakdown (waiting / ready / issuing) from one counter pass")
    st.add_argument("directory")
    st.add_argument("out_md")
    st.add_argument("title")
    st.add_argument("command")
    c = sub.add_parser("counters", help="MFMA / VALU / LDS counter summary; --run LABEL DIR WORKLOAD per workload")
    c.add_argument("--run", nargs=3, action="append", required=True, metavar=("LABEL", "DIR", "WORKLOAD"))
    c.add_argument("--out-md", required=True)
    c.add_argument("--commands", required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        print(trace(a.stats_csv, a.out_md, a.command, a.title, a.bench_json, a.plain_json))
    elif a.cmd == "stalls":
        print(stall_md(a.directory, a.out_md, a.title, a.command))
    elif a.cmd == "counters":
        from . import inputs
        runs = []
        for label, directory, wname in a.run:
            w = inputs.WORKLOADS[wname]
            f = w.fwd_flops()
            runs.append((label, directory, {"fwd": f, "fwd_fp32": f, "bwd_dq": 0.5 * f, "bwd_dkdv": 2.0 * f}))
        print(counters_md(runs, a.out_md, a.commands))
    else:
        print(json.dumps(traffic(a), indent=1))


if __name__ == "__main__":
    main()
