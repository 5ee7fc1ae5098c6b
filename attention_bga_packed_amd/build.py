"""Build libbga.so (the HIP kernels and the C-ABI) in-tree for gfx950.

    python -m attention_bga_packed_amd.build

Each csrc/*.hip is compiled with hipcc in parallel into _build/, then linked
into attention_bga_packed_amd/libbga.so. The debug library libbga_debug.so is
linked from the same kernel objects plus the C-ABI layer and the device-side
precondition checks compiled with -DBGA_DEBUG.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libbga.so")
DEBUG_LIB = os.path.join(PKG, "libbga_debug.so")
# sources compiled a second time, with -DBGA_DEBUG, for the debug library
DEBUG_SOURCES = ("bga_abi.hip", "debug_checks.hip")
ARCH = os.environ.get("BGA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# The attention kernels never produce or consume NaN on purpose (masking uses
# -inf); letting the compiler drop IEEE NaN quieting turns max chains into v_max3.
PER_FILE_FLAGS = {"prefill.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
                  "decode.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"],
                  "topk.hip": ["-fno-honor-nans", "-mno-amdgpu-ieee"]}


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile_all(jobs, hipcc, verbose):
    """jobs: [(src, obj, extra flags)], compiled in parallel; raises on any failure."""
    procs = []
    for src, obj, extra in jobs:
        cmd = [hipcc, *HIPCC_FLAGS, *PER_FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        for src, out in failed:
            print(f"--- {src}\n{out}", file=sys.stderr)
        raise RuntimeError("hipcc failed for " + ", ".join(os.path.basename(s) for s, _ in failed))


def _link(hipcc, objs, lib):
    tmp = lib + ".tmp"
    subprocess.run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    debug_dir = os.path.join(BUILD, "debug")
    os.makedirs(debug_dir, exist_ok=True)
    hipcc = os.environ.get("HIPCC", "hipcc")
    jobs, objs, debug_objs = [], [], []
    for src in sources():
        base = os.path.basename(src)[:-4] + ".o"
        obj = os.path.join(BUILD, base)
        jobs.append((src, obj, []))
        objs.append(obj)
        if os.path.basename(src) in DEBUG_SOURCES:
            dobj = os.path.join(debug_dir, base)
            jobs.append((src, dobj, ["-DBGA_DEBUG"]))
            debug_objs.append(dobj)
        else:
            debug_objs.append(obj)
    _compile_all(jobs, hipcc, verbose)
    _link(hipcc, objs, LIB)
    _link(hipcc, debug_objs, DEBUG_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
