"""Build libpararnn.so (HIP, gfx950 only) in-tree with hipcc.

    python -m nonlinear_rnn_solve_amd.build            # build the library and its look-back stress variant
    python -m nonlinear_rnn_solve_amd.build --asm      # also keep the gfx950 assembly for inspection

Flags: -O3, --offload-arch=gfx950, the packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops; hipcc's host pass prints
that it does not know that feature, the device pass honours it), and
-ffp-contract=on: a multiply and an add fuse into an fma only within one source
expression (or where the source calls fmaf), never across statements, so a
computation inlined into two kernels rounds the same way in both.

libpararnn_stress.so is the same source with -DPR_LB_STRESS=1: tiles pause for
pseudo-random times before publishing look-back words, so that scans walk far
back.  Only the tests load it; its results must equal libpararnn.so's bit for bit.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "pararnn.hip")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libpararnn.so")
STRESS_LIB = os.path.join(HERE, "libpararnn_stress.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def _command(out: str, stress: bool, asm: bool) -> list:
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=on",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-I", INC, SRC, "-o", out]
    if stress:
        cmd.insert(1, "-DPR_LB_STRESS=1")
    if asm:
        cmd += ["--save-temps"]
    return cmd


def build(asm: bool = False, verbose: bool = True, stress: bool = True) -> str:
    """Compile libpararnn.so (and, with stress, libpararnn_stress.so in parallel); returns the library path."""
    jobs = [(LIB, False)] + ([(STRESS_LIB, True)] if stress else [])
    if asm:
        os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
    procs = []
    for lib, st in jobs:
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = _command(tmp, st, asm and not st)
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        p = subprocess.Popen(cmd, cwd=os.path.join(ROOT, "_build") if (asm and not st) else HERE,
                             stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        procs.append((p, tmp, lib))
    failed = []
    for p, tmp, lib in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if out.strip() and verbose:
            print(out)
        if p.returncode != 0:
            failed.append((lib, p.returncode))
        else:
            os.replace(tmp, lib)
    if failed:
        raise RuntimeError("hipcc failed: %s" % failed)
    return LIB


if __name__ == "__main__":
    if "--asm" in sys.argv:
        os.makedirs(os.path.join(ROOT, "_work"), exist_ok=True)
    build(asm="--asm" in sys.argv)
