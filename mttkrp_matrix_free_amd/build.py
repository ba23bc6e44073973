"""Build the HIP library (gfx950) in-tree with hipcc.

    python -m mttkrp_matrix_free_amd.build

produces ``mttkrp_matrix_free_amd/libmttkrp_amd.so``.  Every HIP source is
compiled with packed-fp32 instructions disabled ("Build").
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmttkrp_amd.so")
ARCH = "gfx950"


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm toolchain required)")
    return p


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, extra=None) -> str:
    """Compile every source into one shared library; returns its path."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-Wno-unused-variable", "-Wno-unused-but-set-variable",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp] + list(extra or []) + sources()
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to build libmttkrp_amd.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
