"""Builds libflce.so (HIP kernels + C-ABI) for gfx950 with hipcc, in-tree,
and libflce_timeline.so, the same sources with the per-workgroup timeline of
the main kernels compiled in (a profiling aid; bench.py --timeline).

Usage: python -m linear_cross_entropy_flce_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libflce.so")
TIMELINE_LIB = os.path.join(PKG, "libflce_timeline.so")
SOURCES = ["flce_kernels.hip", "flce_api.cpp"]
ARCH = os.environ.get("FLCE_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def flags(extra=()):
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), *extra,
    ]


def build(verbose: bool = False, extra=(), out: str = LIB) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(extra), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that note is harmless
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, out)
    return out


def build_all(verbose: bool = False) -> list:
    """libflce.so, then libflce_timeline.so."""
    return [build(verbose=verbose),
            build(verbose=verbose, extra=["-DFLCE_TIMELINE=1"], out=TIMELINE_LIB)]


if __name__ == "__main__":
    extra = [a for a in sys.argv[1:] if a != "--verbose"]
    if extra:
        print(build(verbose="--verbose" in sys.argv, extra=extra))
    else:
        print("\n".join(build_all(verbose="--verbose" in sys.argv)))
