"""Seeded synthetic inputs shared by the HIP path and the CPU oracle.

This module only draws random numbers and assembles the input tensors; it holds
none of the MTTKRP arithmetic.  Both sides (the kernels and the oracle) receive
exactly the arrays built here, so a parity comparison is always made on the
same data.

The pages measure on two application tensors (tearing mode and island
coalescence; "A Performance Portable Matrix Free Dense MTTKRP in GenTen",
TL;DR and Figs. 3-5) that are not available; the five workloads below are
synthetic stand-ins with fixed shapes, distributions and seeds.  Every draw
uses numpy's PCG64 ``default_rng`` in the fixed order written in each
function, so a given workload is reproducible bit for bit on any host.

Layout: every tensor is a C-order (row-major) array, last mode fastest.
Every factor is an ``I_m x R`` C-order array.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np


@dataclasses.dataclass
class Problem:
    """One MTTKRP workload: tensor, factors and the name it is reported under."""

    name: str
    X: np.ndarray
    factors: List[np.ndarray]
    rank: int
    # Optional: the exact low-rank part the tensor was built from (noise free),
    # for the closed-form check M_n = U_n * Hadamard_{m != n}(U_m^T U_m).
    cp_factors: Optional[List[np.ndarray]] = None
    noise_sigma: float = 0.0
    # CP-ALS workloads: number of sweeps.
    als_iters: int = 0

    @property
    def dims(self) -> tuple:
        return tuple(int(s) for s in self.X.shape)

    @property
    def order(self) -> int:
        return self.X.ndim


def cp_tensor(factors: Sequence[np.ndarray]) -> np.ndarray:
    """Dense tensor of a CP model [[U_0, ..., U_{d-1}]] (sum of R outer products).

    Used only to assemble inputs with a known low-rank structure.
    """
    d = len(factors)
    letters = "abcdefgh"[:d]
    spec = ",".join(f"{c}z" for c in letters) + "->" + letters
    return np.ascontiguousarray(np.einsum(spec, *factors, optimize=True))


# ---------------------------------------------------------------------------
# The five workloads.  Sizes and distributions are the ones the benchmark names;
# the seeds and the draw order are fixed here.
# ---------------------------------------------------------------------------

def small_uniform_3way() -> Problem:
    """64x48x32 fp64, X ~ U[-1,1], R = 16 factors ~ U[0,1]."""
    rng = np.random.default_rng(1)
    X = rng.uniform(-1.0, 1.0, (64, 48, 32))
    U = [rng.uniform(0.0, 1.0, (I, 16)) for I in X.shape]
    return Problem("3way_64x48x32_f64_R16", X, U, 16)


def lowrank_cube_256(with_noise: bool = True) -> Problem:
    """256^3 fp64 built as an exact rank-32 CP tensor (factors ~ N(0,1)) plus
    i.i.d. N(0, 1e-3^2) noise; the MTTKRP factors are the generating ones."""
    rng = np.random.default_rng(2)
    A = rng.standard_normal((256, 32))
    B = rng.standard_normal((256, 32))
    C = rng.standard_normal((256, 32))
    X = cp_tensor([A, B, C])
    sigma = 1e-3
    if with_noise:
        X += sigma * rng.standard_normal((256, 256, 256))
    return Problem("3way_256cube_f64_R32_cp32", X, [A, B, C], 32,
                   cp_factors=[A, B, C], noise_sigma=sigma if with_noise else 0.0)


def highrank_cube_512() -> Problem:
    """512^3 fp64 (1 GiB), X ~ N(0,1); R = 2000 factors ~ U[0,1]."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((512, 512, 512))
    U = [rng.uniform(0.0, 1.0, (512, 2000)) for _ in range(3)]
    return Problem("3way_512cube_f64_R2000", X, U, 2000)


def fourway_f32(rank: int) -> Problem:
    """128x128x128x64 fp32, X ~ U[0,1); R in {8, 64, 512}, factors ~ U[0,1)."""
    rng = np.random.default_rng(4)
    X = rng.random((128, 128, 128, 64), dtype=np.float32)
    rr = np.random.default_rng([4, rank])
    U = [rr.random((I, rank), dtype=np.float32) for I in X.shape]
    return Problem(f"4way_128x128x128x64_f32_R{rank}", X, U, rank)


def fiveway_als() -> Problem:
    """50x50x50x20x10 fp64 from an exact rank-10 CP model (factors ~ N(0,1))
    plus i.i.d. N(0, 1e-2^2) noise; CP-ALS at R = 64 from U[0,1] factors,
    10 sweeps."""
    dims = (50, 50, 50, 20, 10)
    rng = np.random.default_rng(5)
    A = [rng.standard_normal((I, 10)) for I in dims]
    X = cp_tensor(A)
    sigma = 1e-2
    X += sigma * rng.standard_normal(dims)
    ri = np.random.default_rng([5, 1])
    U = [ri.uniform(0.0, 1.0, (I, 64)) for I in dims]
    return Problem("5way_50x50x50x20x10_f64_R64_als", X, U, 64,
                   cp_factors=A, noise_sigma=sigma, als_iters=10)


# The workloads, keyed by the name each Problem carries (what it is, with
# its sizes).
WORKLOADS = {
    "3way_64x48x32_f64_R16": small_uniform_3way,
    "3way_256cube_f64_R32_cp32": lowrank_cube_256,
    "3way_512cube_f64_R2000": highrank_cube_512,
    "4way_128x128x128x64_f32_R8": lambda: fourway_f32(8),
    "4way_128x128x128x64_f32_R64": lambda: fourway_f32(64),
    "4way_128x128x128x64_f32_R512": lambda: fourway_f32(512),
    "5way_50x50x50x20x10_f64_R64_als": fiveway_als,
}


def workload(name: str) -> Problem:
    return WORKLOADS[name]()


# ---------------------------------------------------------------------------
# Small random problems for sweeps and edge cases.
# ---------------------------------------------------------------------------

def random_problem(dims: Sequence[int], rank: int, dtype=np.float64, seed: int = 0,
                   x_dist: str = "normal", u_dist: str = "uniform") -> Problem:
    """Seeded random tensor and factors of the given shape and rank."""
    rng = np.random.default_rng([7, seed, len(dims), rank])
    dims = tuple(int(d) for d in dims)
    if x_dist == "normal":
        X = rng.standard_normal(dims)
    elif x_dist == "uniform":
        X = rng.uniform(-1.0, 1.0, dims)
    else:
        raise ValueError(x_dist)
    if u_dist == "uniform":
        U = [rng.uniform(0.0, 1.0, (I, rank)) for I in dims]
    elif u_dist == "normal":
        U = [rng.standard_normal((I, rank)) for I in dims]
    else:
        raise ValueError(u_dist)
    X = np.ascontiguousarray(X.astype(dtype))
    U = [np.ascontiguousarray(u.astype(dtype)) for u in U]
    return Problem(f"rand_{'x'.join(map(str, dims))}_R{rank}_{np.dtype(dtype).name}_s{seed}",
                   X, U, rank)


def random_cp_problem(dims: Sequence[int], true_rank: int, rank: int, sigma: float,
                      seed: int = 0) -> Problem:
    """Exact rank-``true_rank`` CP tensor plus N(0, sigma^2) noise, with
    U[0,1] initial factors of rank ``rank`` (a small CP-ALS workload)."""
    rng = np.random.default_rng([11, seed, len(dims), true_rank, rank])
    dims = tuple(int(d) for d in dims)
    A = [rng.standard_normal((I, true_rank)) for I in dims]
    X = cp_tensor(A)
    if sigma:
        X = X + sigma * rng.standard_normal(dims)
    U = [rng.uniform(0.0, 1.0, (I, rank)) for I in dims]
    return Problem(f"cp_{'x'.join(map(str, dims))}_T{true_rank}_R{rank}_s{seed}", X, U, rank,
                   cp_factors=A, noise_sigma=sigma)
