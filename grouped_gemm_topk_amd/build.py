"""Builds libmoe.so (all HIP kernels and the C ABI) in-tree for gfx950, and
libmoe_probe.so, the achievable-peak probes that the benchmark uses for its
roofline denominators (measurement only, not part of the library)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
PROBE_LIB = os.path.join(PKG, "libmoe_probe.so")

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


def _compile(srcs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
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
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source into libmoe.so next to this file (and the probe
    library beside it); returns libmoe.so's path."""
    _compile(sources(), LIB, verbose)
    _compile([os.path.join(CSRC, "probe", "peaks.hip")], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
