"""CPU oracle for dense MTTKRP and CP-ALS -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package.  The HIP library and its Python binding never do:
the product path fails loudly when its own extension is missing and has no
CPU fallback.

The arithmetic lives in ``mttkrp_oracle.c`` (plain C, long-double
accumulation, OpenMP over output rows).  This wrapper only marshals numpy
arrays.  fp32 inputs are promoted to float64 before the call; that promotion
is exact, so the oracle computes the exact-input result for them too.

Definitions followed (see the C file for the element formula):
  * MTTKRP -- "A Performance Portable Matrix Free Dense MTTKRP in GenTen",
    abstract and TL;DR (matricized tensor times Khatri-Rao product, never
    forming the Khatri-Rao matrix), with the mode-n unfolding of
    "An HPC Approach to Accelerate Tensor Decompositions", Sec. 2.
  * CP-ALS -- GenTen page, Fig. 5 (MTTKRP plus inner product and Cholesky
    solve per step).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mttkrp_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ENOTSPD = -7


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math; IEEE semantics kept)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-Wextra", "-Wno-unused-parameter", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_mttkrp_rows.argtypes = [P, P, ctypes.c_int, P, i64, ctypes.c_int, P, i64, P,
                                           ctypes.c_int]
        lib.oracle_mttkrp_rows.restype = ctypes.c_int
        lib.oracle_cp_als.argtypes = [P, P, ctypes.c_int, i64, P, P, ctypes.c_int, P, ctypes.c_int]
        lib.oracle_cp_als.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _as_f64(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a), dtype=np.float64)


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def mttkrp(X: np.ndarray, factors: Sequence[Optional[np.ndarray]], mode: int,
           rows: Optional[Sequence[int]] = None, nthreads: int = 0) -> np.ndarray:
    """M = MTTKRP_mode(X, factors) in float64 (rounded once from long double).

    ``factors[mode]`` is not read and may be None.  When ``rows`` is given,
    only those output rows are computed and returned (len(rows) x R).
    """
    lib = _load()
    X64 = _as_f64(X)
    d = X64.ndim
    if len(factors) != d:
        raise ValueError("need one factor per mode")
    R = None
    keep = []
    ptrs = (ctypes.c_void_p * d)()
    for m, U in enumerate(factors):
        if m == mode or U is None:
            ptrs[m] = None
            continue
        U64 = _as_f64(U)
        if U64.ndim != 2 or U64.shape[0] != X64.shape[m]:
            raise ValueError(f"factor {m} has shape {U64.shape}")
        if R is None:
            R = U64.shape[1]
        elif U64.shape[1] != R:
            raise ValueError("factors disagree on the rank")
        keep.append(U64)
        ptrs[m] = _ptr(U64)
    if R is None:
        raise ValueError("no factor given")
    dims = np.array(X64.shape, dtype=np.int64)
    if rows is None:
        out = np.empty((X64.shape[mode], R), dtype=np.float64)
        rp, nr = None, 0
    else:
        rr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        out = np.empty((rr.size, R), dtype=np.float64)
        rp, nr = _ptr(rr), rr.size
        keep.append(rr)
    st = lib.oracle_mttkrp_rows(_ptr(X64), _ptr(dims), d, ptrs, R, mode, rp, nr, _ptr(out),
                                int(nthreads))
    if st != 0:
        raise RuntimeError(f"oracle_mttkrp_rows failed with status {st}")
    return out


def cp_als(X: np.ndarray, factors: Sequence[np.ndarray], iters: int,
           nthreads: int = 0) -> Tuple[List[np.ndarray], np.ndarray, np.ndarray, int]:
    """CP-ALS from the given initial factors.

    Returns (factors, lambda, fit_hist, status).  status is 0 or ENOTSPD;
    on ENOTSPD the fit history holds NaN from the failing sweep on.
    """
    lib = _load()
    X64 = _as_f64(X)
    d = X64.ndim
    F = [_as_f64(U).copy() for U in factors]
    R = F[0].shape[1]
    ptrs = (ctypes.c_void_p * d)(*[_ptr(f) for f in F])
    lam = np.empty(R, dtype=np.float64)
    fit = np.empty(max(iters, 1), dtype=np.float64)
    dims = np.array(X64.shape, dtype=np.int64)
    st = lib.oracle_cp_als(_ptr(X64), _ptr(dims), d, R, ptrs, _ptr(lam), int(iters), _ptr(fit),
                           int(nthreads))
    if st not in (0, ENOTSPD):
        raise RuntimeError(f"oracle_cp_als failed with status {st}")
    return F, lam, fit[:iters], int(st)
