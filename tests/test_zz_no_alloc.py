"""The allocation-free entry point mttkrp_noalloc against the workspace entry
points it varies (mttkrp_f64 / mttkrp_f32) and the CPU oracle, through the C
ABI: two calls in a row on the GPU's shared scratch array, the second with a
smaller input, each equal bit for bit to the workspace entry point (same plan,
same kernels) and within the parity bar of the oracle.  Collected last: it
must pass alone in a fresh process and after the other tests."""
import ctypes
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mttkrp_matrix_free_amd import _lib, api, inputs  # noqa: E402

pytestmark = pytest.mark.gpu

NT = min(16, len(os.sched_getaffinity(0)))


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def noalloc(X, U, n, out):
    L = _lib.lib()
    dims = (ctypes.c_int64 * X.dim())(*X.shape)
    ptrs = (ctypes.c_void_p * X.dim())(*[u.data_ptr() for u in U])
    eb = X.element_size()
    return L.mttkrp_noalloc(X.data_ptr(), dims, X.dim(), ptrs, U[0].shape[1], n, out.data_ptr(),
                            eb, torch.cuda.current_stream().cuda_stream)


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# (dims, rank, mode, dtype): larger input first, then a smaller one, per dtype
SEQUENCES = [
    [((256, 256, 256), 32, 2, np.float64), ((40, 36, 64), 12, 2, np.float64)],
    [((50, 50, 50, 20, 10), 64, 4, np.float64), ((37, 41, 23, 19, 7), 64, 4, np.float64)],
    [((64, 64, 64, 32), 64, 3, np.float32), ((48, 40, 36, 16), 20, 3, np.float32)],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["f64-3way", "f64-5way-trailing", "f32-4way"])
def test_noalloc_equals_workspace_entry_two_calls(seq):
    for k, (dims, R, n, dt) in enumerate(seq):
        tdt = torch.float64 if dt == np.float64 else torch.float32
        assert api.plan(dims, R, n, tdt)["splits"] > 1, "the case must use the scratch array"
        p = inputs.random_problem(dims, R, dtype=dt, seed=90 + k)
        say(f"  call {k}: {dims} R={R} mode {n} {np.dtype(dt).name}")
        X = torch.from_numpy(p.X).cuda()
        U = [torch.from_numpy(u).cuda() for u in p.factors]
        out = torch.full((dims[n], R), float("nan"), dtype=tdt, device="cuda")
        assert noalloc(X, U, n, out) == 0
        ref = api.mttkrp(X, U, n)  # the workspace entry point (own workspace)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (k, dims)
        e = rel_fro(out.cpu().numpy(), oracle.mttkrp(p.X, p.factors, n, nthreads=NT))
        say(f"    equal to the workspace entry point; oracle error {e:.2e}")
        assert e <= (1e-12 if dt == np.float64 else 1e-5)


def test_noalloc_refuses_before_any_work():
    """Too large for the scratch array, or a bad argument: refused on the
    host, the output untouched."""
    L = _lib.lib()
    X = torch.zeros(8, dtype=torch.float64, device="cuda")
    out = torch.full((4,), 7.0, dtype=torch.float64, device="cuda")
    big = (ctypes.c_int64 * 3)(2048, 512, 512)
    ptrs = (ctypes.c_void_p * 3)(X.data_ptr(), X.data_ptr(), X.data_ptr())
    need = api.workspace_bytes((2048, 512, 512), 2000, 0)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert L.mttkrp_noalloc(X.data_ptr(), big, 3, ptrs, 2000, 0, out.data_ptr(), 8, None) \
        == _lib.ESCRATCH
    assert L.mttkrp_noalloc(X.data_ptr(), big, 3, ptrs, 2000, 0, out.data_ptr(), 2, None) \
        == _lib.EINVAL
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 7.0))
