"""Writes tests/golden/fiveway_als_oracle.json: the CPU oracle's CP-ALS run on
the 50x50x50x20x10 rank-10 + noise workload at R = 64 (10 sweeps), so that
the GPU test can compare its per-sweep fit without re-running the long-double
oracle for minutes.

Calls only the oracle (oracle/) and the shared seeded input generators.

    python tests/golden/make_oracle_golden.py
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


def main():
    p = inputs.fiveway_als()
    t0 = time.time()
    F, lam, fit, st = oracle.cp_als(p.X, p.factors, p.als_iters)
    dt = time.time() - t0
    out = {
        "workload": p.name,
        "dims": list(p.dims),
        "rank": p.rank,
        "iters": p.als_iters,
        "status": st,
        "fit": [float(v) for v in fit],
        "lambda": [float(v) for v in lam],
        # column norms are 1; store each final factor's first row and a checksum
        "factor_row0": [[float(v) for v in f[0]] for f in F],
        "factor_sum": [float(np.sum(f)) for f in F],
        "oracle_seconds": dt,
        "oracle_threads": oracle.max_threads(),
        "generator": "tests/golden/make_oracle_golden.py (oracle.cp_als, long double)",
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fiveway_als_oracle.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {path} in {dt:.1f} s")


if __name__ == "__main__":
    main()
