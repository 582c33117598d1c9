"""Builds libflashattn.so in-tree with hipcc for gfx950.

Each HIP source compiles to its own object (in parallel), then one link step
produces the shared library next to this file. Usage:
    python -m io_aware_flashattention_flash_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libflashattn.so")
SOURCES = ["flash_attn_abi.hip", "fa_fwd_16bit.hip", "fa_fwd_fp32.hip", "fa_bwd_16bit.hip", "fa_dropout.hip"]
ARCH = "gfx950"

# Packed fp32 VALU forms are disabled for every HIP object: the compiler then emits only
# scalar fp32 VALU instructions, never v_pk_{add,mul,fma}_f32.
HIPCC_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines() if "is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + out)
    return out


# Library variants: (file name, extra compiler flags). The race-guard variant puts a full wait and a
# workgroup barrier after every pipeline stage (FA_DEBUG_SYNC in csrc/fa_device.h); tests require
# its results to equal the main library's bit for bit.
VARIANTS = {
    "main": ("libflashattn.so", ()),
    "debugsync": ("libflashattn_debugsync.so", ("-DFA_DEBUG_SYNC=1",)),
}
DEBUGSYNC_LIB_PATH = os.path.join(PKG, VARIANTS["debugsync"][0])


def build(verbose: bool = False, extra_flags=(), variants=("main", "debugsync")) -> str:
    """Compile every HIP source for each library variant and link them; returns the main library's
    path. All objects of all variants compile in one pool."""
    hipcc = _hipcc()
    cmds, links = [], []
    for name in variants:
        lib_name, vflags = VARIANTS[name]
        bdir = BUILD_DIR if name == "main" else BUILD_DIR + "_" + name
        os.makedirs(bdir, exist_ok=True)
        objs = []
        for src in SOURCES:
            obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
            objs.append(obj)
            cmds.append([hipcc, *HIPCC_FLAGS, *vflags, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
        links.append((os.path.join(PKG, lib_name), objs))
    # the largest sources first, so the pool's tail is short
    cmds.sort(key=lambda c: -os.path.getsize(c[-3]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for path, objs in links:
        tmp = path + ".tmp"
        _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, path)
    build_abi_roundtrip(hipcc)
    return LIB_PATH


ROUNDTRIP_SRC = os.path.join(os.path.dirname(PKG), "tests", "c_abi", "abi_roundtrip.cpp")
ROUNDTRIP_BIN = os.path.join(os.path.dirname(PKG), "tests", "c_abi", "abi_roundtrip")


def build_abi_roundtrip(hipcc: str) -> None:
    """The host program that exercises the C ABI without Python (tests/c_abi), linked against the
    in-tree library with a relative run path."""
    if not os.path.exists(ROUNDTRIP_SRC):
        return
    rpath = "-Wl,-rpath,$ORIGIN/" + os.path.relpath(PKG, os.path.dirname(ROUNDTRIP_BIN))
    _run([hipcc, "-O2", "-std=c++17", ROUNDTRIP_SRC, "-o", ROUNDTRIP_BIN + ".tmp", "-L" + PKG, "-lflashattn",
          rpath])
    os.replace(ROUNDTRIP_BIN + ".tmp", ROUNDTRIP_BIN)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
