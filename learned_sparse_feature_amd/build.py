"""Build libsg.so (the HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libsg.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions are kept out of every code object
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into libsg.so; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
           *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
