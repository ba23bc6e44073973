"""GPU CP-ALS driver against the CPU oracle's CP-ALS ("A Performance Portable
Matrix Free Dense MTTKRP in GenTen", Fig. 5: MTTKRP plus inner product and
Cholesky solve per step).

Bars: the fit of every sweep within 1e-9 of the oracle's; lambda and factors
after the first sweep within 1e-10 (relative); after more sweeps the R x R
solves may amplify rounding differences (an over-factored model), so only
the fit is binding there and factors are checked loosely.
"""
import json
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mttkrp_matrix_free_amd import _lib, api, inputs  # noqa: E402

pytestmark = pytest.mark.gpu

NT = min(16, len(os.sched_getaffinity(0)))
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


@pytest.mark.parametrize("dims,true_rank,R,iters", [
    ((12, 10, 8), 3, 4, 1), ((12, 10, 8), 3, 4, 6), ((9, 8, 7, 6), 2, 5, 5),
    ((6, 5, 7, 4, 3), 2, 3, 4), ((40, 35, 30), 5, 70, 3),
    ((80, 12, 10), 3, 64, 2),  # mode 0: two 64-row passes of the one-workgroup update
    ((200, 12, 10), 3, 64, 2),  # mode 0 too tall for the one-workgroup update, modes 1-2 not
    ((70, 9, 8), 3, 40, 2), ((33, 21, 17), 3, 20, 2),  # frames that start 48 and 32 wide
    # an unsplit last mode (the fit kernel ends the sweep and orders the next
    # sweep's first side kernel) and an unsplit middle mode (an event orders
    # the side kernel after it)
    ((12, 10, 200), 3, 64, 3), ((12, 200, 10), 3, 64, 3),
    # blocked factorization and solves (R > 64): 3 blocks, a 4-way case with a
    # ragged last block, and R = 300 (the model norm summed by workgroups)
    ((30, 28, 26), 3, 150, 2), ((12, 11, 10, 9), 2, 100, 2), ((40, 38, 36), 3, 300, 2),
    ((20, 18, 16), 3, 65, 2), ((24, 22, 20), 3, 128, 2),  # a 1-wide last block; whole blocks
    # blocked update with many row blocks of M (a 700-row mode, first and middle)
    ((700, 20, 18), 3, 100, 2), ((20, 700, 18), 3, 130, 2),
])
def test_als_small_vs_oracle(dims, true_rank, R, iters):
    p = inputs.random_cp_problem(dims, true_rank, R, sigma=0.05, seed=31)
    say(f"  cp_als {dims} R={R} iters={iters}")
    F0, lam0, fit0, st0 = oracle.cp_als(p.X, p.factors, iters, nthreads=NT)
    assert st0 == 0
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, iters)
    assert st == 0 and done == iters
    for it in range(iters):
        assert abs(fit[it] - fit0[it]) <= 1e-9, (it, fit[it], fit0[it])
    if iters == 1:
        assert rel(lam.cpu().numpy(), lam0) <= 1e-10
        for m in range(len(dims)):
            assert rel(U[m].cpu().numpy(), F0[m]) <= 1e-10, m
    else:
        assert rel(lam.cpu().numpy(), lam0) <= 1e-6
        for m in range(len(dims)):
            assert rel(U[m].cpu().numpy(), F0[m]) <= 1e-6, m


def test_fiveway_als_workload_vs_stored_oracle():
    """50x50x50x20x10, rank-10 model + noise, R = 64, 10 sweeps.  The oracle's
    run is stored by tests/golden/make_oracle_golden.py (oracle only)."""
    g = json.load(open(os.path.join(GOLDEN, "fiveway_als_oracle.json")))
    p = inputs.fiveway_als()
    assert list(p.dims) == g["dims"] and p.rank == g["rank"]
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, g["iters"])
    say("  fit gpu   ", fit)
    say("  fit oracle", g["fit"])
    assert st == 0 and done == g["iters"]
    for it in range(g["iters"]):
        assert abs(fit[it] - g["fit"][it]) <= 1e-9, (it, fit[it], g["fit"][it])
    assert np.all(np.diff(fit) >= -1e-12)
    assert rel(lam.cpu().numpy(), g["lambda"]) <= 1e-6
    # the final factors, as far as the golden stores them (each factor's first
    # row and the sum of its entries), at the loose bar for many sweeps
    for m in range(len(p.dims)):
        Um = U[m].cpu().numpy()
        e_row = rel(Um[0], g["factor_row0"][m])
        # (relative to the sum of the entries' magnitudes: the signed sum may
        # cancel, while the 1e-6 bar is relative to the factor's size)
        e_sum = abs(float(Um.sum()) - g["factor_sum"][m]) / float(np.abs(Um).sum())
        say(f"  factor {m}: row 0 {e_row:.2e}, sum {e_sum:.2e}")
        assert e_row <= 1e-6, (m, e_row)
        assert e_sum <= 1e-6, (m, e_sum)


def test_als_not_spd_leaves_factors():
    p = inputs.random_cp_problem((10, 9, 8), 2, 3, sigma=0.0, seed=32)
    Z = [u.copy() for u in p.factors]
    for u in Z:
        u[:, 1] = 0.0
    X = dev(p.X)
    U = [dev(u) for u in Z]
    lam, fit, done, st = api.cp_als(X, U, 3)
    assert st == _lib.ENOTSPD and done == 0
    assert all(np.isnan(f) for f in fit)
    for m in range(3):
        assert np.array_equal(U[m].cpu().numpy(), Z[m])


def test_als_rank2000_normal_equations():
    # the blocked path at the rank of the 512^3 workload (32 diagonal blocks):
    # after a sweep the last mode's factor satisfies its normal equations,
    # (U_n diag(lambda)) V = M_n with V the Hadamard product of the other
    # Grams and M_n the MTTKRP with the other final factors
    p = inputs.random_cp_problem((60, 56, 52), 4, 2000, sigma=0.1, seed=36)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, 1)
    assert st == 0 and done == 1 and np.isfinite(fit[0])
    n = 2
    M = api.mttkrp(X, U, n).double()
    V = (U[0].t() @ U[0]) * (U[1].t() @ U[1])
    res = (M - (U[n] * lam) @ V).norm() / M.norm()
    assert float(res) <= 1e-10, float(res)
    # the factor columns are unit-norm where lambda > 0
    nrm = U[n].norm(dim=0)
    assert torch.allclose(nrm[lam > 0], torch.ones_like(nrm[lam > 0]), atol=1e-12)


def test_als_rank2000_vs_stored_oracle():
    """Rank 2000 (the blocked factorization over 32 diagonal blocks and the
    blocked solves) against the oracle's run on the same inputs, stored by
    tests/golden/make_oracle_golden.py (oracle only): the fit of every sweep,
    lambda, and each final factor's first row and entry sum."""
    g = json.load(open(os.path.join(GOLDEN, "rank2000_als_oracle.json")))
    c = g["recipe"]
    p = inputs.random_cp_problem(tuple(c["dims"]), c["true_rank"], c["rank"], sigma=c["sigma"],
                                 seed=c["seed"])
    assert list(p.dims) == g["dims"] and p.rank == g["rank"] == 2000
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, g["iters"])
    say("  fit gpu   ", fit)
    say("  fit oracle", g["fit"])
    assert st == 0 and done == g["iters"]
    for it in range(g["iters"]):
        assert abs(fit[it] - g["fit"][it]) <= 1e-9, (it, fit[it], g["fit"][it])
    e_lam = rel(lam.cpu().numpy(), g["lambda"])
    say(f"  lambda {e_lam:.2e}")
    assert e_lam <= 1e-6
    for m in range(len(p.dims)):
        Um = U[m].cpu().numpy()
        e_row = rel(Um[0], g["factor_row0"][m])
        e_sum = abs(float(Um.sum()) - g["factor_sum"][m]) / float(np.abs(Um).sum())
        say(f"  factor {m}: row 0 {e_row:.2e}, sum {e_sum:.2e}")
        assert e_row <= 1e-6, (m, e_row)
        assert e_sum <= 1e-6, (m, e_sum)


def test_als_not_spd_blocked_leaves_factors():
    # R > 64 (the blocked factorization): a zero column makes a pivot of the
    # second block exactly zero, if no earlier one fails
    p = inputs.random_cp_problem((10, 9, 8), 2, 80, sigma=0.0, seed=35)
    Z = [u.copy() for u in p.factors]
    for u in Z:
        u[:, 70] = 0.0
    X = dev(p.X)
    U = [dev(u) for u in Z]
    lam, fit, done, st = api.cp_als(X, U, 2)
    assert st == _lib.ENOTSPD and done == 0
    assert all(np.isnan(f) for f in fit)
    for m in range(3):
        assert np.array_equal(U[m].cpu().numpy(), Z[m])


def test_als_tolerance_stops_early():
    p = inputs.random_cp_problem((15, 14, 13), 2, 2, sigma=0.0, seed=33)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, 50, tol=1e-10)
    assert st == 0 and 1 < done < 50
    assert all(np.isnan(f) for f in fit[done:])
    # the sweep queued past the stop changes nothing: the result equals that
    # of a run of exactly `done` sweeps
    U2 = [dev(u) for u in p.factors]
    lam2, fit2, done2, st2 = api.cp_als(X, U2, done)
    assert st2 == 0 and done2 == done
    assert np.array_equal(fit2, fit[:done])
    assert torch.equal(lam2, lam)
    for a, b in zip(U, U2):
        assert torch.equal(a, b)


def test_als_float32_blocked():
    # fp32 factors with R > 64: the blocked R x R path and the tiled Gram of
    # fp32 factors
    p = inputs.random_cp_problem((22, 20, 18), 3, 80, sigma=0.05, seed=37)
    F0, lam0, fit0, st0 = oracle.cp_als(p.X, p.factors, 2, nthreads=NT)
    X = dev(p.X.astype(np.float32))
    U = [dev(u.astype(np.float32)) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, 2)
    assert st == 0 and done == 2
    for it in range(2):
        assert abs(fit[it] - fit0[it]) <= 1e-4, (it, fit[it], fit0[it])


def test_als_float32():
    p = inputs.random_cp_problem((20, 18, 16, 6), 3, 4, sigma=0.05, seed=34)
    F0, lam0, fit0, st0 = oracle.cp_als(p.X, p.factors, 4, nthreads=NT)
    X = dev(p.X.astype(np.float32))
    U = [dev(u.astype(np.float32)) for u in p.factors]
    lam, fit, done, st = api.cp_als(X, U, 4)
    assert st == 0
    # fp32 inputs differ from the fp64 ones by rounding: compare the fit loosely
    for it in range(4):
        assert abs(fit[it] - fit0[it]) <= 1e-4, (it, fit[it], fit0[it])


def test_als_two_host_threads_at_once():
    """Two host threads run split-update CP-ALS calls at the same time, each on
    its own stream.  They share the library's second stream on the device; each
    kernel waits only for work queued before it, so both calls finish, with
    the results (bit for bit) of the same calls run one at a time."""
    import threading
    probs = [inputs.random_cp_problem(d, 3, 32, sigma=0.05, seed=sd)
             for d, sd in (((40, 36, 30), 41), ((30, 28, 26, 6), 42))]
    ref = []
    for p in probs:
        U = [dev(u) for u in p.factors]
        lam, fit, done, st = api.cp_als(dev(p.X), U, 6)
        assert st == 0 and done == 6
        ref.append((lam.cpu().numpy(), np.array(fit), [u.cpu().numpy() for u in U]))
    out = [None, None]
    errs = []

    def run(i):
        try:
            s = torch.cuda.Stream()
            p = probs[i]
            with torch.cuda.stream(s):
                X = dev(p.X)
                U = [dev(u) for u in p.factors]
                lam, fit, done, st = api.cp_als(X, U, 6, stream=s)
                s.synchronize()
                out[i] = (st, done, lam.cpu().numpy(), np.array(fit), [u.cpu().numpy() for u in U])
        except Exception as e:  # reported below
            errs.append(repr(e))

    threads = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errs, errs
    for i in range(2):
        st, done, lam, fit, U = out[i]
        assert st == 0 and done == 6
        assert np.array_equal(lam, ref[i][0])
        assert np.array_equal(fit, ref[i][1])
        for a, b in zip(U, ref[i][2]):
            assert np.array_equal(a, b)
