"""Builds libmoe.so (all HIP kernels and the C ABI) in-tree for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False) -> str:
    """Compile every source into libmoe.so next to this file; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("libmoe build failed")
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise and verbose:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
