"""Build libmk.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m persistent_runtime_amd.build
"""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmk.so")
SOURCES = ["kernels_m1.hip", "kernels_m2.hip", "kernels_m0.hip", "kernels_sched.hip",
           "kernels.hip", "planner.cpp", "capi.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def source_hash() -> str:
    """Hash of every source file the library is compiled from (the C-ABI
    header and everything under csrc/).  Built into the library and checked
    by the binding, so a library built from other sources is refused."""
    h = hashlib.sha256()
    files = [os.path.join(ROOT, "include", "mk.h")]
    files += sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                    if f.endswith((".hip", ".cpp", ".h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _flags():
    return ["-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
            # keep the compiler from emitting packed fp32 VALU instructions
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # multiply-adds fused only where one source expression asks for it,
            # so every executor (differently inlined copies of the same tile
            # code) rounds identically
            "-ffp-contract=on",
            "-Wno-unused-command-line-argument",
            f'-DMK_SOURCE_HASH="{source_hash()}"',
            "-I", os.path.join(ROOT, "include")]


def command(out=LIB, extra=()):
    """One hipcc line that compiles and links every source (for reference)."""
    return [HIPCC, *_flags(), "-shared", *[os.path.join(CSRC, s) for s in SOURCES],
            "-o", out, *extra]


def build(verbose: bool = False) -> str:
    """Compile the sources in parallel into objects under _build/, then link
    libmk.so in place (atomically replacing an older library)."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        cmd = [HIPCC, *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                            stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out)
            failed = True
    if failed:
        raise RuntimeError("hipcc failed compiling libmk.so sources")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed linking libmk.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
