"""Writes the stored CP-ALS runs of the CPU oracle that the GPU tests compare
against, so that those tests do not re-run the long-double oracle for
minutes:

  fiveway_als_oracle.json   the 50x50x50x20x10 rank-10 + noise workload at
                            R = 64, 10 sweeps;
  rank2000_als_oracle.json  a 60x56x52 exact rank-4 CP tensor plus N(0, 0.1^2)
                            noise at R = 2000 (the rank of the GenTen page's
                            largest decomposition, TL;DR and Fig. 5), 2 sweeps,
                            so that the blocked R x R factorization and solves
                            (32 diagonal blocks) are checked against the oracle.

Calls only the oracle (oracle/) and the shared seeded input generators.

    python tests/golden/make_oracle_golden.py [fiveway|rank2000|all]
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from mttkrp_matrix_free_amd import inputs  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))

# The rank-2000 run: shape, truth rank, noise, seed and sweeps.  The GPU test
# rebuilds the same inputs from these values.
RANK2000 = {"dims": [60, 56, 52], "true_rank": 4, "rank": 2000, "sigma": 0.1, "seed": 36,
            "iters": 2}


def record(p, F, lam, fit, st, dt, iters, extra=None):
    out = {
        "workload": p.name,
        "dims": list(p.dims),
        "rank": p.rank,
        "iters": iters,
        "status": st,
        "fit": [float(v) for v in fit],
        "lambda": [float(v) for v in lam],
        # column norms are 1; store each final factor's first row and the sum
        # of its entries
        "factor_row0": [[float(v) for v in f[0]] for f in F],
        "factor_sum": [float(np.sum(f)) for f in F],
        "oracle_seconds": dt,
        "oracle_threads": oracle.max_threads(),
        "generator": "tests/golden/make_oracle_golden.py (oracle.cp_als, long double)",
    }
    if extra:
        out.update(extra)
    return out


def fiveway():
    p = inputs.fiveway_als()
    t0 = time.time()
    F, lam, fit, st = oracle.cp_als(p.X, p.factors, p.als_iters)
    return "fiveway_als_oracle.json", record(p, F, lam, fit, st, time.time() - t0, p.als_iters)


def rank2000():
    c = RANK2000
    p = inputs.random_cp_problem(tuple(c["dims"]), c["true_rank"], c["rank"], sigma=c["sigma"],
                                 seed=c["seed"])
    t0 = time.time()
    F, lam, fit, st = oracle.cp_als(p.X, p.factors, c["iters"])
    return "rank2000_als_oracle.json", record(p, F, lam, fit, st, time.time() - t0, c["iters"],
                                              {"recipe": c})


def main():
    which = sys.argv[1] if len(sys.argv) > 1 else "all"
    jobs = {"fiveway": fiveway, "rank2000": rank2000}
    for name, fn in jobs.items():
        if which not in (name, "all"):
            continue
        fname, out = fn()
        path = os.path.join(HERE, fname)
        with open(path, "w") as f:
            json.dump(out, f, indent=1)
        print(f"wrote {path} in {out['oracle_seconds']:.1f} s")


if __name__ == "__main__":
    main()
