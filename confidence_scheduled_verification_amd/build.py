"""Builds libdspark.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdspark.so")
SOURCES = ["chain.hip", "cand.hip", "sched.hip", "step.hip", "accept.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    # packed fp32 vector ops stay off on this target (the host pass ignores the feature)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libdspark.so next to this file; returns its path.

    The sources compile in parallel to objects under _build/ and are then linked."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *FLAGS, "-c", "-I", INCLUDE, "-I", CSRC, os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, obj, subprocess.Popen(cmd)))
    failed = [src for src, _, p in procs if p.wait() != 0]
    if failed:
        raise subprocess.CalledProcessError(1, f"hipcc {' '.join(failed)}")
    tmp = LIB + ".tmp"
    link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for _, o, _ in procs], "-o", tmp]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.check_call(link)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
