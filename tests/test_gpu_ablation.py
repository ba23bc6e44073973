"""The untiled matrix-free baselines (MTTKRP-ELEM and MTTKRP-SLICE of "A
Performance Portable Matrix Free Dense MTTKRP in GenTen") against the oracle:
bench.py times them beside the tiled kernels, so they must compute the same
MTTKRP.  ELEM adds with atomics in no fixed order (fp64 within 1e-12); fp32
runs compare within 1e-5 (both baselines sum in fp32)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mttkrp_matrix_free_amd import api, inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind", ["elem", "slice"])
@pytest.mark.parametrize("dims,R", [((9, 8, 7), 5), ((6, 5, 4, 7), 3), ((4, 3, 5, 2, 3), 6),
                                    ((5, 4, 3), 300)])
def test_ablation_vs_oracle(kind, dims, R):
    p = inputs.random_cp_problem(dims, 2, R, sigma=0.1, seed=43)
    for dt, tol in ((torch.float64, 1e-12), (torch.float32, 1e-5)):
        X = torch.from_numpy(p.X).cuda().to(dt)
        U = [torch.from_numpy(u).cuda().to(dt) for u in p.factors]
        for n in range(len(dims)):
            M = api.mttkrp_ablation(X, U, n, kind).double().cpu().numpy()
            ref = oracle.mttkrp(p.X, p.factors, n)
            assert np.linalg.norm(M - ref) <= tol * np.linalg.norm(ref), (kind, dims, n, dt)
