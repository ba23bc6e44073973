"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments with the documented codes before any
HIP call, and plans within the hardware limits and the matrix-free memory
contract (workspace independent of the Khatri-Rao size; "A Performance
Portable Matrix Free Dense MTTKRP in GenTen", TL;DR).

Calls made here all fail validation or are pure queries; none launches work.
"""
import ctypes
import os
import re

import pytest

from mttkrp_matrix_free_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mttkrp.h")

P = ctypes.c_void_p
FAKE = 0x7F0000001000          # aligned, never dereferenced (validation fails first)
FAKE_MIS = 0x7F0000001008      # 8-byte aligned only


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for", "sizeof")))


def dims_arr(d):
    return (ctypes.c_int64 * len(d))(*d)


def ptrs(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert set(_lib.EXPORTS) == set(names), (sorted(set(names) ^ set(_lib.EXPORTS)))
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_version(L):
    for code in range(0, -9, -1):
        s = _lib.strerror(code)
        assert s and s != "unknown status"
    assert _lib.strerror(-99) == "unknown status"
    assert L.mttkrp_version() >= 100


def test_fast_division_constants(L):
    """The planner's multiply-high division constants (Granlund and Montgomery,
    "Division by Invariant Integers using Multiplication", Sec. 4) agree with
    plain division over the library's fixed set of divisors and dividends."""
    assert L.mttkrp_selftest() == 0


def call_f64(L, X=FAKE, dims=(4, 5, 6), order=None, factors=None, rank=3, mode=0, out=FAKE,
             ws=None, ws_bytes=0):
    order = len(dims) if order is None else order
    if factors is None:
        factors = [FAKE] * max(len(dims) if dims is not None else order, 1)
    return L.mttkrp_f64(X, dims_arr(dims) if dims is not None else None, order,
                        ptrs(factors) if factors != "null" else None, rank, mode, out, ws,
                        ws_bytes, None)


def test_validation_codes(L):
    # null pointers
    assert call_f64(L, X=None) == _lib.EINVAL
    assert call_f64(L, out=None) == _lib.EINVAL
    assert call_f64(L, dims=None, order=3) == _lib.EINVAL
    assert call_f64(L, factors="null") == _lib.EINVAL
    assert call_f64(L, factors=[FAKE, None, FAKE]) == _lib.EINVAL
    # order
    assert call_f64(L, dims=(4, 5), order=2) == _lib.EORDER
    assert call_f64(L, dims=(2, 2, 2, 2, 2, 2), order=6) == _lib.EORDER
    # sizes, rank, mode
    assert call_f64(L, dims=(4, 0, 6)) == _lib.EINVAL
    assert call_f64(L, dims=(4, -1, 6)) == _lib.EINVAL
    assert call_f64(L, rank=0) == _lib.EINVAL
    assert call_f64(L, mode=3) == _lib.EINVAL
    assert call_f64(L, mode=-1) == _lib.EINVAL
    # alignment
    assert call_f64(L, X=FAKE_MIS) == _lib.EALIGN
    assert call_f64(L, out=FAKE_MIS) == _lib.EALIGN
    assert call_f64(L, factors=[FAKE, FAKE_MIS, FAKE]) == _lib.EALIGN
    # overflow of the element count / index range
    assert call_f64(L, dims=(1 << 40, 1 << 40, 4)) == _lib.ERANGE
    assert call_f64(L, dims=(1 << 20, 1 << 20, 1 << 12)) == _lib.ERANGE
    # workspace too small (this plan needs partial sums)
    need = ctypes.c_size_t()
    assert L.mttkrp_workspace_bytes(dims_arr((256, 256, 256)), 3, 32, 2, 8, ctypes.byref(need)) == 0
    assert need.value > 0
    assert call_f64(L, dims=(256, 256, 256), rank=32, mode=2, ws=FAKE, ws_bytes=need.value - 256) \
        == _lib.EWORKSPACE
    assert call_f64(L, dims=(256, 256, 256), rank=32, mode=2, ws=None, ws_bytes=0) == _lib.EWORKSPACE


def test_target_factor_may_be_null(L):
    # factors[mode] == NULL is allowed; with the workspace missing the call stops
    # at the workspace check, before any launch.
    st = L.mttkrp_f64(FAKE, dims_arr((256, 256, 256)), 3, ptrs([FAKE, FAKE, None]), 32, 2, FAKE,
                      None, 0, None)
    assert st == _lib.EWORKSPACE


def test_all_and_als_validation(L):
    d = dims_arr((4, 5, 6))
    outs = ptrs([FAKE, FAKE, FAKE])
    assert L.mttkrp_all_f64(FAKE, d, 3, ptrs([FAKE, None, FAKE]), 3, outs, None, 0, None) == _lib.EINVAL
    assert L.mttkrp_all_f64(FAKE, d, 3, ptrs([FAKE] * 3), 3, ptrs([FAKE, FAKE_MIS, FAKE]), None, 0,
                            None) == _lib.EALIGN
    assert L.mttkrp_all_f32(FAKE, d, 7, ptrs([FAKE] * 3), 3, outs, None, 0, None) == _lib.EORDER
    fit = (ctypes.c_double * 4)()
    done = ctypes.c_int()
    args = dict(X=FAKE, dims=d, order=3, R=3, F=ptrs([FAKE] * 3), lam=FAKE, iters=4, tol=0.0,
                fit=fit, done=ctypes.byref(done), ws=FAKE, wsb=1 << 20)

    def als(**kw):
        a = dict(args)
        a.update(kw)
        return L.cp_als_f64(a["X"], a["dims"], a["order"], a["R"], a["F"], a["lam"], a["iters"],
                            a["tol"], a["fit"], a["done"], a["ws"], a["wsb"], None)
    assert als(X=None) == _lib.EINVAL
    assert als(lam=None) == _lib.EINVAL
    assert als(fit=None) == _lib.EINVAL
    assert als(iters=-1) == _lib.EINVAL
    assert als(order=2) == _lib.EORDER
    assert als(F=ptrs([FAKE, FAKE, None])) == _lib.EINVAL
    assert als(lam=FAKE_MIS) == _lib.EALIGN
    assert als(wsb=16) == _lib.EWORKSPACE
    assert als(R=5000) == _lib.ERANGE


WORKLOADS = [
    ((64, 48, 32), 16, 8), ((256, 256, 256), 32, 8), ((512, 512, 512), 2000, 8),
    ((128, 128, 128, 64), 8, 4), ((128, 128, 128, 64), 64, 4), ((128, 128, 128, 64), 512, 4),
    ((50, 50, 50, 20, 10), 64, 8),
    # ragged and degenerate shapes
    ((1, 1, 1), 1, 8), ((33, 17, 19), 17, 8), ((7, 1, 5, 3), 5, 4), ((2, 3, 2, 3, 2), 3, 8),
    ((5, 7, 1), 100, 8), ((1, 9, 4, 1, 6), 33, 4),
]


@pytest.mark.parametrize("dims,R,eb", WORKLOADS)
def test_plans_within_limits_and_matrix_free_memory(L, dims, R, eb):
    d = len(dims)
    kr_bytes_max = 0
    max_ws = 0
    for n in range(d):
        info = _lib.PlanInfo()
        assert L.mttkrp_plan(dims_arr(dims), d, R, n, eb, ctypes.byref(info)) == 0
        assert info.grid % 8 == 0 and info.grid >= 8
        assert info.waves in (4, 8)
        assert info.lds_bytes <= (144 if info.waves == 8 else 80) * 1024
        assert info.mb in (2, 4) and info.nb in (1, 2, 4, 8)
        assert info.splits >= 1 and info.rtiles == -(-R // (16 * info.nb))
        # the contraction modes and the tile-row modes are disjoint and exclude n
        used = [m for m in list(info.k_modes) + list(info.row_modes) + list(info.outer_modes) if m >= 0]
        if info.form == 0:
            assert n in list(info.row_modes)
        else:
            assert n not in used
        assert len(used) == len(set(used))
        assert sorted(set(used) | {n}) == list(range(d))
        # workspace: bounded by the output size times a hardware constant,
        # never by the Khatri-Rao size prod_{m != n} I_m * R
        ws = ctypes.c_size_t()
        assert L.mttkrp_workspace_bytes(dims_arr(dims), d, R, n, eb, ctypes.byref(ws)) == 0
        assert ws.value == info.ws_bytes
        max_ws = max(max_ws, ws.value)
        # partials: at most max(1024, contraction chunks) copies of the kernel's
        # output rows (I_n, or the trailing block I_{d-2} I_{d-1} with
        # I_{d-1} < 64 for a layout-1 plan) times R, in fp64
        rows_k = info.rows if info.layout == 1 else dims[n]
        if info.layout == 1:
            assert rows_k in (dims[n], dims[d - 2] * dims[d - 1])
            assert rows_k <= 64 * max(dims)
        assert ws.value <= 8 * max(1024, info.kchunks) * rows_k * R + 256
        kr = 1
        for m in range(d):
            if m != n:
                kr *= dims[m]
        kr_bytes_max = max(kr_bytes_max, kr * R * eb)
    allws = ctypes.c_size_t()
    assert L.mttkrp_all_workspace_bytes(dims_arr(dims), d, R, eb, ctypes.byref(allws)) == 0
    # two halves: one mode's pending partials and the next mode's own
    assert allws.value == 2 * max_ws
    als = ctypes.c_size_t()
    if R <= 4096:
        assert L.cp_als_workspace_bytes(dims_arr(dims), d, R, eb, ctypes.byref(als)) == 0
        assert als.value >= max_ws


def test_workspace_far_below_khatri_rao_at_rank_2000(L):
    """The 512^3, R = 2000 case: the explicit Khatri-Rao matrix of one mode is
    512*512*2000*8 B = 4.19 GB.  The matrix-free path's workspace (partial
    sums of the I_n x R output, a few copies) stays below 2% of it -- the
    memory ratio the GenTen page reports at rank 2000 (TL;DR) -- and below
    16 copies of the output."""
    for n in range(3):
        ws = ctypes.c_size_t()
        assert L.mttkrp_workspace_bytes(dims_arr((512, 512, 512)), 3, 2000, n, 8, ctypes.byref(ws)) == 0
        assert ws.value <= 0.02 * 512 * 512 * 2000 * 8
        assert ws.value <= 16 * 512 * 2000 * 8


def test_three_wave_plans_leave_room_for_three_workgroups(L):
    """Four-wave form-0 workgroups of the 32 x 64 row-major and 64 x 32
    row-contiguous tiles run three waves per SIMD (fp64 with one outer slot,
    fp32 with one or two): their LDS must let three share a compute unit
    (160 KB).  The matrix-core-bound workloads take such plans."""
    seen = 0
    for dims, R, eb in WORKLOADS:
        d = len(dims)
        for n in range(d):
            info = _lib.PlanInfo()
            assert L.mttkrp_plan(dims_arr(dims), d, R, n, eb, ctypes.byref(info)) == 0
            slots = max(1, sum(1 for m in info.outer_modes if m >= 0))
            tile = (info.mb, info.nb, info.layout)
            three = (info.form == 0 and info.waves == 4 and tile in ((2, 4, 0), (4, 2, 1)) and
                     (slots == 1 if eb == 8 else slots in (1, 2)))
            if three:
                seen += 1
                assert 3 * info.lds_bytes <= 160 * 1024, (dims, R, n, info.lds_bytes)
    assert seen >= 10  # the 512^3 rank-2000 modes and the fp32 rank-64 and rank-512 modes


MODEL_CASES = [((256, 256, 256), 32, 8), ((512, 512, 512), 2000, 8), ((128, 128, 128, 64), 8, 4),
               ((128, 128, 128, 64), 512, 4), ((50, 50, 50, 20, 10), 64, 8), ((33, 17, 19), 17, 8)]


@pytest.mark.parametrize("dims,R,eb", MODEL_CASES)
def test_plan_cache_model(L, dims, R, eb):
    """The plan's cache model: T(p) is the largest of its four resource times,
    never below the plan-free bound T_inf (every byte once, unpadded flops)
    and never above T_0 for these sizes; the matrix-core term covers at least
    the algorithmic flops."""
    d = len(dims)
    N = 1
    for v in dims:
        N *= v
    P = 78.6e12 if eb == 8 else 157.3e12
    for n in range(d):
        info = _lib.PlanInfo()
        assert L.mttkrp_plan(dims_arr(dims), d, R, n, eb, ctypes.byref(info)) == 0
        assert info.launchable == 1
        terms = [info.model_flop_s, info.model_hbm_s, info.model_l2_s, info.model_lds_s]
        assert all(t > 0 for t in terms)
        assert info.model_s == max(terms)
        assert info.model_flop_s >= 2.0 * R * N / P * (1 - 1e-12)
        assert info.model_s >= info.t_inf_s * (1 - 1e-12)
        assert info.t_0_s >= info.t_inf_s


def test_force_tile_override(L, monkeypatch):
    """MTTKRP_FORCE_TILE (experiments only) replaces the wave tile; a bad value
    makes planning fail with EINVAL; a forced tile without a kernel is
    reported (launchable = 0) and the entry point refuses it before any HIP
    call."""
    dims = dims_arr((512, 512, 512))
    info = _lib.PlanInfo()
    assert L.mttkrp_plan(dims, 3, 2000, 0, 8, ctypes.byref(info)) == 0
    base = (info.mb, info.nb, info.waves, info.splits)
    monkeypatch.setenv("MTTKRP_FORCE_TILE", "4,2")
    assert L.mttkrp_plan(dims, 3, 2000, 0, 8, ctypes.byref(info)) == 0
    assert (info.mb, info.nb) == (4, 2) and info.launchable == 1
    monkeypatch.setenv("MTTKRP_FORCE_TILE", "2,8,8")
    assert L.mttkrp_plan(dims, 3, 2000, 0, 8, ctypes.byref(info)) == 0
    assert (info.mb, info.nb, info.waves) == (2, 8, 8) and info.launchable == 0
    st = L.mttkrp_f64(FAKE, dims, 3, ptrs([FAKE] * 3), 2000, 0, FAKE, FAKE, 1 << 30, None)
    assert st == _lib.EINVAL
    for bad in ("3,1", "2", "2,3", "2,4,6", "x", "2,4,8,1"):
        monkeypatch.setenv("MTTKRP_FORCE_TILE", bad)
        assert L.mttkrp_plan(dims, 3, 2000, 0, 8, ctypes.byref(info)) == _lib.EINVAL, bad
    monkeypatch.delenv("MTTKRP_FORCE_TILE")
    assert L.mttkrp_plan(dims, 3, 2000, 0, 8, ctypes.byref(info)) == 0
    assert (info.mb, info.nb, info.waves, info.splits) == base


def test_probe_validation(L):
    assert L.mttkrp_probe_read_grid() > 0 and L.mttkrp_probe_mfma_grid() > 0
    assert L.mttkrp_probe_read(None, 16, FAKE, None) == _lib.EINVAL
    assert L.mttkrp_probe_read(FAKE, 16, None, None) == _lib.EINVAL
    assert L.mttkrp_probe_read(FAKE_MIS, 16, FAKE, None) == _lib.EALIGN
    assert L.mttkrp_probe_read(FAKE, 17, FAKE, None) == _lib.EINVAL
    assert L.mttkrp_probe_mfma(8, 0, FAKE, None) == _lib.EINVAL
    assert L.mttkrp_probe_mfma(8, 10, None, None) == _lib.EINVAL
    assert L.mttkrp_probe_mfma(8, 10, FAKE_MIS, None) == _lib.EALIGN


def test_noalloc_host_checks(L):
    """mttkrp_noalloc refuses bad arguments and plans larger than its fixed
    scratch array on the host, before any HIP call (fake pointers here)."""
    d = dims_arr((2048, 512, 512))
    f = ptrs([FAKE] * 3)
    need = ctypes.c_size_t()
    assert L.mttkrp_workspace_bytes(d, 3, 2000, 0, 8, ctypes.byref(need)) == 0
    assert need.value > _lib.NOALLOC_SCRATCH_BYTES
    assert L.mttkrp_noalloc(FAKE, d, 3, f, 2000, 0, FAKE, 8, None) == _lib.ESCRATCH
    assert L.mttkrp_noalloc(FAKE, d, 3, f, 2000, 0, FAKE, 2, None) == _lib.EINVAL
    assert L.mttkrp_noalloc(None, d, 3, f, 2000, 0, FAKE, 8, None) == _lib.EINVAL
    assert L.mttkrp_noalloc(FAKE, d, 3, f, 2000, 3, FAKE, 8, None) == _lib.EINVAL
    assert L.mttkrp_noalloc(FAKE, d, 3, f, 2000, 0, FAKE_MIS, 8, None) == _lib.EALIGN
    assert L.mttkrp_noalloc(FAKE, dims_arr((4, 5)), 2, f, 3, 0, FAKE, 8, None) == _lib.EORDER
    # every benchmark workload's single-mode call fits the array
    for dims, R, eb in WORKLOADS[:7]:
        for n in range(len(dims)):
            assert L.mttkrp_workspace_bytes(dims_arr(dims), len(dims), R, n, eb,
                                            ctypes.byref(need)) == 0
            assert need.value <= _lib.NOALLOC_SCRATCH_BYTES, (dims, R, n)
