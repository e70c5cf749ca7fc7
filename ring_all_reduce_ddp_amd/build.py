"""Builds libddp_ring.so (the C-ABI library) in the package directory.

Device code is compiled by hipcc for gfx950 only. Every HIP source gets
`-Xclang -target-feature -Xclang -packed-fp32-ops`, which keeps the compiler
from emitting packed fp32 instructions. The host-only planner is compiled by
g++. Usage: python -m ring_all_reduce_ddp_amd.build [--asm DIR]
"""

import argparse
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libddp_ring.so")

HIP_SOURCES = ["fused_kernels.hip", "ring_kernels.hip", "pack_kernels.hip", "view_kernels.hip", "scatter_kernels.hip", "reducer.hip", "runtime.hip"]
HOST_SOURCES = ["plan.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", INCLUDE, "-I", CSRC]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if proc.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + proc.stdout)
    return proc.stdout


def build(verbose=False, asm_dir=None):
    """Compiles every source and links libddp_ring.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    hc = hipcc()
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [hc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if asm_dir:
            os.makedirs(asm_dir, exist_ok=True)
            cmd += ["-save-temps=obj"]
        jobs.append((cmd, obj))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append((["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for (cmd, _), out in zip(jobs, outs):
            print(" ".join(cmd))
            if out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *[o for _, o in jobs]])
    os.replace(tmp, LIB)
    if asm_dir:
        for f in os.listdir(BUILD):
            if f.endswith(".s") and ARCH in f:
                shutil.copy(os.path.join(BUILD, f), os.path.join(asm_dir, f))
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="also keep the gfx950 assembly in this directory")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose, asm_dir=args.asm))


if __name__ == "__main__":
    sys.exit(main())
