"""Turn rocprofv3 output into the short text summaries kept under profiles/.

  python -m io_aware_flashattention_flash_amd.profiling trace STATS_CSV OUT_MD "COMMAND" "TITLE"
      kernel-trace summary (calls, average / min / max duration, share) of this library's kernels

  python -m io_aware_flashattention_flash_amd.profiling traffic --fetch DIR --write DIR \
      --copy-fetch DIR --copy-write DIR --copy-bytes N --out-json JSON --out-md MD --commands "..."
      HBM traffic per launch of each attention kernel from FETCH_SIZE / WRITE_SIZE (KiB per
      dispatch), each scaled by what the same counter reports for a plain device copy of N bytes
      (bench.py --copy-calibration), stored with a digest of the kernel's source so that a stale
      figure is never reported for a changed kernel.
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
KERNEL_SOURCES = {"fwd": "fa_fwd_16bit.hip", "bwd_dq": "fa_bwd_16bit.hip", "bwd_dkdv": "fa_bwd_16bit.hip"}
KERNEL_PREFIX = {"fwd": "fa::fwd16_kernel", "bwd_dq": "fa::bwd_dq_kernel", "bwd_dkdv": "fa::bwd_dkdv_kernel"}


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
    for key, prefix in KERNEL_PREFIX.items():
        if short.startswith(prefix + "<"):
            return key
    return None


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


def trace(stats_csv: str, out_md: str, command: str, title: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command (run from the repository root on one MI355X):", "", "```", command, "```", "",
             "| kernel | calls | avg µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in rows:
        short = readable_name(r["Name"])
        if not short.startswith("fa::"):
            continue
        lines.append(f"| `{short}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f}% |")
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
    fetch = counter_per_dispatch(a.fetch, "FETCH_SIZE", kernel_key)
    write = counter_per_dispatch(a.write, "WRITE_SIZE", kernel_key)
    out = {"_calibration": {"copy_bytes": a.copy_bytes, "fetch_kib_per_dispatch": cf, "write_kib_per_dispatch": cw,
                            "fetch_scale": f_scale, "write_scale": w_scale}}
    for k in sorted(set(fetch) & set(write)):
        fb, wb = fetch[k] * 1024.0 / f_scale, write[k] * 1024.0 / w_scale
        out[k] = {"source_digest": source_digest(k), "fetch_bytes_per_launch": round(fb),
                  "write_bytes_per_launch": round(wb), "bytes_per_launch": round(fb + wb)}
    with open(a.out_json, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, copy-calibrated)", "",
             "Commands (run from the repository root on one MI355X; one counter per pass):", "", "```",
             a.commands, "```", "",
             f"Calibration: a device copy of {a.copy_bytes} bytes reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE "
             f"{cw:.0f} KiB per dispatch, i.e. {f_scale:.4f} / {w_scale:.4f} of the bytes moved; kernel figures "
             "below are divided by these factors.", "",
             "| kernel | fetch MB / launch | write MB / launch | total MB / launch |", "|---|---|---|---|"]
    for k, v in out.items():
        if k.startswith("_"):
            continue
        lines.append(f"| {k} | {v['fetch_bytes_per_launch'] / 1e6:.2f} | {v['write_bytes_per_launch'] / 1e6:.2f} | "
                     f"{v['bytes_per_launch'] / 1e6:.2f} |")
    with open(a.out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    return out


# One counter pass per workload (at most 8 SQ and 2 GRBM counters, so they fit a single pass).
COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
            "SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE SQ_WAVE_CYCLES GRBM_GUI_ACTIVE")
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
        mfma_flops = 512.0 * c["SQ_INSTS_VALU_MFMA_MOPS_BF16"]
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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats_csv")
    t.add_argument("out_md")
    t.add_argument("command")
    t.add_argument("title")
    r = sub.add_parser("traffic")
    for name in ("--fetch", "--write", "--copy-fetch", "--copy-write", "--out-json", "--out-md", "--commands"):
        r.add_argument(name, required=True)
    r.add_argument("--copy-bytes", type=int, required=True)
    c = sub.add_parser("counters", help="MFMA / VALU / LDS counter summary; --run LABEL DIR WORKLOAD per workload")
    c.add_argument("--run", nargs=3, action="append", required=True, metavar=("LABEL", "DIR", "WORKLOAD"))
    c.add_argument("--out-md", required=True)
    c.add_argument("--commands", required=True)
    a = ap.parse_args()
    if a.cmd == "trace":
        print(trace(a.stats_csv, a.out_md, a.command, a.title))
    elif a.cmd == "counters":
        from . import inputs
        runs = []
        for label, directory, wname in a.run:
            w = inputs.WORKLOADS[wname]
            f = w.fwd_flops()
            runs.append((label, directory, {"fwd": f, "bwd_dq": 0.5 * f, "bwd_dkdv": 2.0 * f}))
        print(counters_md(runs, a.out_md, a.commands))
    else:
        print(json.dumps(traffic(a), indent=1))


if __name__ == "__main__":
    main()
