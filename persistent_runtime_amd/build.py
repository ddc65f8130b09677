"""Build libmk.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m persistent_runtime_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["planner.cpp", "capi.cpp", "kernels.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out=LIB, extra=()):
    return [HIPCC, "-std=c++17", "-O3", "-fPIC", "-shared", f"--offload-arch={ARCH}",
            # keep the compiler from emitting packed fp32 VALU instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # multiply-adds fused only where one source expression asks for it,
            # so every executor (differently inlined copies of the same tile
            # code) rounds identically
            "-ffp-contract=on",
            "-Wno-unused-command-line-argument",
            "-I", os.path.join(ROOT, "include"),
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out, *extra]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmk.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
