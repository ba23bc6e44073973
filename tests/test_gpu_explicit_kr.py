"""The explicit Khatri-Rao + vendor GEMM baseline that bench.py times beside
the library (the matrix-based MTTKRP of the GenTen page, Fig. 3): its output
against the oracle, so that the comparison times a correct computation."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

torch = pytest.importorskip("torch")
import bench  # noqa: E402
import oracle  # noqa: E402
from mttkrp_matrix_free_amd import inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dims,R", [((9, 8, 7), 5), ((6, 5, 4, 7), 3), ((4, 3, 5, 2, 3), 6)])
def test_explicit_kr_baseline_vs_oracle(dims, R):
    p = inputs.random_cp_problem(dims, 2, R, sigma=0.1, seed=41)
    X = torch.from_numpy(p.X).cuda()
    U = [torch.from_numpy(u).cuda() for u in p.factors]
    for n in range(len(dims)):
        M, kb, cb = bench.explicit_kr_mttkrp(X, U, n)
        ref = oracle.mttkrp(p.X, p.factors, n)
        got = M.cpu().numpy()
        assert got.shape == ref.shape
        assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref), (dims, n)
        assert kb == int(np.prod(dims)) // dims[n] * R * 8
        assert cb == (0 if n in (0, len(dims) - 1) else int(np.prod(dims)) * 8)
