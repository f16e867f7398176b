"""Build libpararnn.so (HIP, gfx950 only) in-tree with hipcc.

    python -m nonlinear_rnn_solve_amd.build            # build
    python -m nonlinear_rnn_solve_amd.build --asm      # also keep the gfx950 assembly for inspection

Flags: -O3, --offload-arch=gfx950, the packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops; hipcc's host pass prints
that it does not know that feature, the device pass honours it), and
-ffp-contract=on: a multiply and an add fuse into an fma only within one source
expression (or where the source calls fmaf), never across statements, so a
computation inlined into two kernels rounds the same way in both.
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
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "bin", "hipcc")
    return p if os.path.exists(p) else "hipcc"


def build(asm: bool = False, verbose: bool = True) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=on",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-I", INC, SRC, "-o", tmp]
    if asm:
        cmd += ["--save-temps"]
    env = dict(os.environ)
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    if asm:
        os.makedirs(os.path.join(ROOT, "_build"), exist_ok=True)
    p = subprocess.run(cmd, cwd=os.path.join(ROOT, "_build") if asm else HERE, env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if out.strip() and verbose:
        print(out)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed (%d)" % p.returncode)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    if "--asm" in sys.argv:
        os.makedirs(os.path.join(ROOT, "_work"), exist_ok=True)
    build(asm="--asm" in sys.argv)
