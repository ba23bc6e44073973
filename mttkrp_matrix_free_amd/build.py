"""Build the HIP library (gfx950) in-tree with hipcc.

    python -m mttkrp_matrix_free_amd.build

compiles every source under csrc/ to an object (in parallel; the tile-kernel
instantiations are spread over several units for this) and links
``mttkrp_matrix_free_amd/libmttkrp_amd.so``.  Every HIP source is compiled
with packed-fp32 instructions disabled.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmttkrp_amd.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
         "-Wno-unused-but-set-variable"]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found (ROCm toolchain required)")
    return p


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str, verbose: bool):
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-c"] + FLAGS + [
        "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    return obj, res


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every source (in parallel) and link the shared library; returns its path."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), len(os.sched_getaffinity(0)), 16))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), srcs))
    failed = [(o, r) for o, r in results if r.returncode != 0]
    for _, r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed to compile " + ", ".join(os.path.basename(o) for o, _ in failed))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for o, _ in results]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed to link libmttkrp_amd.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
