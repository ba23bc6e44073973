"""GPU parity: the HIP MTTKRP against the CPU oracle on the same seeded inputs.

Bar (relative Frobenius error per mode): 1e-12 for fp64, 1e-5 for fp32.
Small and ragged shapes are compared in full; the large workloads on sampled
output rows (which the oracle computes one by one) plus properties that hold
at any size (closed form for exact CP tensors, cross-mode inner product).
Every call goes through the C ABI (include/mttkrp.h) via the ctypes binding.
"""
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
TOL = {np.dtype(np.float64): 1e-12, np.dtype(np.float32): 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rel_fro(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def run_modes(p, modes=None, rows=None):
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    d = p.X.ndim
    errs = {}
    for n in (range(d) if modes is None else modes):
        say(f"  {p.name} mode {n} R={p.rank} dtype={p.X.dtype}")
        M = api.mttkrp(X, U, n)
        torch.cuda.synchronize()
        Mg = M.cpu().numpy()
        if rows is None:
            Mo = oracle.mttkrp(p.X, p.factors, n, nthreads=NT)
            errs[n] = rel_fro(Mg, Mo)
        else:
            rr = rows(p.dims[n])
            Mo = oracle.mttkrp(p.X, p.factors, n, rows=rr, nthreads=NT)
            errs[n] = rel_fro(Mg[rr], Mo)
    del X, U
    return errs


SWEEP = [
    ((33, 17, 19), 17, np.float64), ((33, 17, 19), 17, np.float32),
    ((5, 7, 1), 100, np.float64), ((1, 1, 1), 1, np.float64), ((7, 1, 5, 3), 5, np.float64),
    ((2, 3, 2, 3, 2), 3, np.float64), ((1, 9, 4, 1, 6), 33, np.float32),
    ((40, 30, 20, 10), 64, np.float32), ((13, 11, 9, 7, 5), 24, np.float64),
    ((100, 3, 70), 1, np.float64), ((130, 70, 50), 40, np.float64),
    ((24, 20, 520), 40, np.float64),     # contraction too long for LDS: factor read from L2
    ((36, 520, 20), 40, np.float64),     # same, output is the unit-stride mode
    ((64, 64, 96), 130, np.float32),     # several rank tiles, 8-block tiles in fp32
    ((17, 19, 23, 4), 19, np.float64),   # short last mode merged into the contraction
    ((9, 10, 11, 12, 13), 7, np.float32),
    ((24, 20, 50, 48), 72, np.float32),  # fp32 long merged contraction: 9 chunks, ragged last
    # item reductions against two row factors (merged row modes): fp32 16- and 32-column
    # tiles, and fp64 with an outer mode (every row's factor loads at once)
    ((8, 50, 40, 20, 10), 16, np.float32), ((4, 33, 45, 60), 24, np.float32),
    ((6, 30, 20, 24, 9), 12, np.float64),
]


@pytest.mark.parametrize("dims,R,dt", SWEEP, ids=[f"{'x'.join(map(str, d))}-R{r}-{np.dtype(t).name}"
                                                  for d, r, t in SWEEP])
def test_sweep_full_parity(dims, R, dt):
    p = inputs.random_problem(dims, R, dtype=dt, seed=len(dims) * 1000 + R)
    errs = run_modes(p)
    for n, e in errs.items():
        assert e <= TOL[np.dtype(dt)], (dims, R, n, e)


def test_small_workload_64x48x32():
    p = inputs.small_uniform_3way()
    errs = run_modes(p)
    say("  errors", errs)
    assert all(e <= 1e-12 for e in errs.values()), errs


def tile_rows(dims, R, n, dtype):
    """Output rows that cover every output tile of the plan the library
    launches for mode n: every row when each output row is a unit of its own
    (form 1) or the output is a short trailing mode; otherwise two rows of
    every row tile (at positions that move from tile to tile, so that
    different lanes and accumulator elements are checked), plus the first and
    last rows.  Every rank tile, contraction chunk and split contributes to
    each of these rows, so all of them are checked too."""
    tdt = torch.float64 if np.dtype(dtype) == np.float64 else torch.float32
    pl = api.plan(dims, R, n, tdt)
    I = dims[n]
    if pl["form"] == 1 or pl["rows"] != I or I <= 64:
        return list(range(I)), pl
    rpt = 16 * pl["mb"]
    rows = {0, I - 1}
    for t in range(-(-I // rpt)):
        lo, hi = t * rpt, min(I, (t + 1) * rpt)
        span = hi - lo
        rows.add(lo + (t * 5) % span)
        rows.add(hi - 1 - (t * 3) % span)
    return sorted(rows), pl


def check_every_tile(p, tol):
    """Every mode of a large workload against the oracle on the rows of
    tile_rows(), element by element and by relative Frobenius error."""
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    worst = {}
    for n in range(p.X.ndim):
        rows, pl = tile_rows(p.dims, p.rank, n, p.X.dtype)
        say(f"  {p.name} mode {n}: {len(rows)} rows (form {pl['form']}, layout {pl['layout']}, "
            f"{16 * pl['mb']}-row tiles, {pl['rtiles']} rank tiles, {pl['splits']} splits)")
        M = api.mttkrp(X, U, n)
        torch.cuda.synchronize()
        Mg = M.cpu().numpy()[rows].astype(np.float64)
        del M
        Mo = oracle.mttkrp(p.X, p.factors, n, rows=rows, nthreads=NT)
        e = rel_fro(Mg, Mo)
        # element by element: each entry within the bar relative to its row's size
        scale = np.linalg.norm(Mo, axis=1, keepdims=True) / np.sqrt(Mo.shape[1])
        elem = float(np.max(np.abs(Mg - Mo) / np.maximum(scale, 1e-300)))
        say(f"    rel Frobenius {e:.3e}, worst entry / row rms {elem:.3e}")
        assert e <= tol, (n, e)
        assert elem <= 10 * tol, (n, elem)
        worst[n] = e
    del X, U
    return worst


def test_lowrank_cube_256_full_and_closed_form():
    """The 256^3 rank-32 CP tensor with noise, as specified, compared in full
    with the oracle (every output of every mode); then the noise-free tensor
    in full against the closed form U_n * Hadamard_{m != n}(U_m^T U_m)."""
    p = inputs.lowrank_cube_256(with_noise=True)
    errs = run_modes(p)
    say("  full errors", errs)
    assert all(e <= 1e-12 for e in errs.values()), errs
    q = inputs.lowrank_cube_256(with_noise=False)
    X = dev(q.X)
    U = [dev(u) for u in q.factors]
    for n in range(3):
        V = np.ones((32, 32))
        for m in range(3):
            if m != n:
                V *= q.factors[m].T @ q.factors[m]
        M = api.mttkrp(X, U, n).cpu().numpy()
        e = rel_fro(M, q.factors[n] @ V)
        say(f"  closed form mode {n}: {e:.3e}")
        assert e <= 1e-12


def test_highrank_cube_512_every_tile_and_inner_products():
    """512^3 fp64, R = 2000: two rows of every output tile of every mode
    against the oracle, then <X, [[U]]> through every mode."""
    p = inputs.highrank_cube_512()
    check_every_tile(p, 1e-12)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    inner = []
    for n in range(3):
        M = api.mttkrp(X, U, n)
        inner.append(float(torch.sum(M * U[n]).item()))
        del M
    ref = inner[0]
    for v in inner[1:]:
        assert abs(v - ref) <= 1e-12 * abs(ref) * 10, inner


@pytest.mark.parametrize("R", [8, 64, 512])
def test_fourway_f32_every_tile(R):
    """128x128x128x64 fp32: every form-1 unit (output row), else two rows of
    every output tile, of every mode against the oracle."""
    p = inputs.fourway_f32(R)
    check_every_tile(p, 1e-5)


TRAILING = [
    ((37, 41, 23, 19, 7), 64, np.float64),   # 133 rows: ragged 32-row tiles, scalar loads
    ((37, 41, 23, 20, 6), 80, np.float32),   # 120 rows, vector loads, ragged rank tile
    ((31, 29, 17, 24, 40), 64, np.float64),  # 960 rows
]


@pytest.mark.parametrize("dims,R,dt", TRAILING, ids=[f"{'x'.join(map(str, d))}-R{r}-{np.dtype(t).name}"
                                                     for d, r, t in TRAILING])
def test_trailing_rows_32row_tiles(dims, R, dt):
    """Outputs that are one of the two short trailing modes: the tile rows are
    the contiguous block of the last two modes, in 32-row tiles, and the
    contraction is cut into many chunks."""
    p = inputs.random_problem(dims, R, dtype=dt, seed=sum(dims) + R)
    d = len(dims)
    tdt = torch.float64 if dt == np.float64 else torch.float32
    modes = [n for n in (d - 2, d - 1) if api.plan(dims, R, n, tdt)["rows"] == dims[-2] * dims[-1]]
    assert modes, "no trailing-rows plan for this shape"
    for n in modes:
        pl = api.plan(dims, R, n, tdt)
        assert pl["layout"] == 1 and pl["mb"] == 2 and pl["nb"] == 4 and pl["kchunks"] > 1, pl
    errs = run_modes(p, modes=modes)
    say("  errors", errs)
    for n, e in errs.items():
        assert e <= TOL[np.dtype(dt)], (dims, R, n, e)


def test_fiveway_workload_full():
    p = inputs.fiveway_als()
    errs = run_modes(p)
    say("  errors", errs)
    assert all(e <= 1e-12 for e in errs.values()), errs


def test_all_modes_entry_and_determinism():
    p = inputs.random_problem((45, 38, 29, 6), 21, seed=5)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    outs = api.mttkrp_all(X, U)
    outs2 = api.mttkrp_all(X, U)
    for n in range(4):
        single = api.mttkrp(X, U, n)
        assert torch.equal(outs[n], single), n
        assert torch.equal(outs[n], outs2[n]), n
        assert rel_fro(outs[n].cpu().numpy(), oracle.mttkrp(p.X, p.factors, n, nthreads=NT)) <= 1e-12


@pytest.mark.parametrize("dims,rank,dtype", [
    ((256, 256, 256), 32, np.float64),   # 64 splits: 16 thread groups per output
    ((128, 96, 256), 40, np.float64),    # 19 splits: 4 groups; two rank tiles
    ((256, 384, 192), 24, np.float32),   # fp32, ragged rank; two split modes, one partner
    ((64, 64, 64, 32), 64, np.float32),  # every mode splits: a chain of three hand-offs
    ((50, 50, 50, 20, 10), 64, np.float64),  # three split modes, then two trailing-rows modes
    ((96, 64, 80, 24), 40, np.float32),  # 143 splits handed to a mode without partials
])
def test_all_modes_hand_split_sums_to_another_launch(dims, rank, dtype):
    """In the all-mode call a mode whose plan splits hands its partial sums to
    the next launch's tile kernel, which may write partials of its own to the
    other half of the workspace; the result must equal the per-mode call (its
    own reduction kernel) bit for bit, and the oracle."""
    plans = [api.plan(dims, rank, n, torch.float64 if dtype == np.float64 else torch.float32)
             for n in range(len(dims))]
    assert any(pl["splits"] > 1 for pl in plans)
    p = inputs.random_problem(dims, rank, seed=31, dtype=dtype)
    say(f"  all-mode {dims} R={rank} {np.dtype(dtype).name}: splits {[pl['splits'] for pl in plans]}")
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    outs = api.mttkrp_all(X, U)
    for n in range(len(dims)):
        single = api.mttkrp(X, U, n)
        assert torch.equal(outs[n], single), n
    n = int(np.argmax([pl["splits"] for pl in plans]))
    rr = np.linspace(0, dims[n] - 1, 24).astype(np.int64)
    Mo = oracle.mttkrp(p.X, p.factors, n, rows=rr, nthreads=NT)
    assert rel_fro(outs[n].cpu().numpy()[rr], Mo) <= TOL[np.dtype(dtype)]


def test_target_factor_not_read():
    p = inputs.random_problem((20, 30, 40), 9, seed=6)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    for n in range(3):
        ref = api.mttkrp(X, U, n)
        V = list(U)
        V[n] = None
        assert torch.equal(api.mttkrp(X, V, n), ref)
        V[n] = torch.full_like(U[n], float("nan"))
        assert torch.equal(api.mttkrp(X, V, n), ref)


def test_nan_propagates_to_its_rows():
    p = inputs.random_problem((12, 10, 8, 6), 5, seed=7)
    Xn = p.X.copy()
    Xn[3, 4, 5, 2] = np.nan
    X = dev(Xn)
    U = [dev(u) for u in p.factors]
    star = (3, 4, 5, 2)
    for n in range(4):
        M = api.mttkrp(X, U, n).cpu().numpy()
        bad = np.isnan(M).any(axis=1)
        assert bad[star[n]] and bad.sum() == 1, (n, np.nonzero(bad))


def test_workspace_and_alignment_errors_on_device():
    p = inputs.random_problem((256, 64, 128), 32, seed=8)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    need = api.workspace_bytes(X.shape, 32, 2)
    assert need > 0
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.MttkrpError) as ei:
        api.mttkrp(X, U, 2, ws=small)
    assert ei.value.status == _lib.EWORKSPACE
    L = _lib.lib()
    dims = (ctypes.c_int64 * 3)(256, 64, 128)
    ptrs = (ctypes.c_void_p * 3)(*[u.data_ptr() for u in U])
    out = torch.empty(256, 32, dtype=torch.float64, device="cuda")
    st = L.mttkrp_f64(X.data_ptr() + 8, dims, 3, ptrs, 32, 0, out.data_ptr(), None, 0, None)
    assert st == _lib.EALIGN


def test_workspace_reuse_across_calls():
    """One workspace buffer serves several calls in a row (partials are fully
    rewritten each time)."""
    p = inputs.random_problem((64, 96, 40), 24, seed=9)
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    ws = torch.full((api.all_workspace_bytes(X.shape, 24),), 255, dtype=torch.uint8, device="cuda")
    for n in (2, 0, 1, 2):
        M = api.mttkrp(X, U, n, ws=ws).cpu().numpy()
        assert rel_fro(M, oracle.mttkrp(p.X, p.factors, n, nthreads=NT)) <= 1e-12


def test_two_stream_sweep_orders_with_caller_stream():
    """A long all-mode sweep runs on the caller's stream and a second stream;
    work queued on the caller's stream after the call must see every output
    complete, and work queued before it must finish before the sweep reads its
    inputs."""
    p = inputs.fiveway_als()
    X = dev(p.X)
    U = [dev(u) for u in p.factors]
    ref = [api.mttkrp(X, U, n) for n in range(5)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    outs = [torch.zeros_like(r) for r in ref]
    ws = torch.empty(api.all_workspace_bytes(X.shape, p.rank, X.dtype), dtype=torch.uint8,
                     device="cuda")
    U2 = [torch.zeros_like(u) for u in U]
    with torch.cuda.stream(s):
        for _ in range(3):
            # factors written on the caller's stream right before the call
            for a, b in zip(U2, U):
                a.copy_(b)
            api.mttkrp_all(X, U2, outs=outs, ws=ws, stream=s)
            # read back on the caller's stream right after the call
            copies = [o.clone() for o in outs]
            for o in outs:
                o.zero_()
            for a in U2:
                a.zero_()
    s.synchronize()
    for n in range(5):
        assert torch.equal(copies[n], ref[n]), n
