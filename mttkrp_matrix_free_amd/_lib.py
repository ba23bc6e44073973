"""ctypes binding of libmttkrp_amd.so (the C ABI in include/mttkrp.h).

Argument marshalling only.  There is no CPU fallback: when the library is
missing the import of any entry point raises, naming the build command.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmttkrp_amd.so")

OK = 0
EINVAL = -1
EORDER = -2
ERANGE = -3
EALIGN = -4
EWORKSPACE = -5
EHIP = -6
ENOTSPD = -7
ESCRATCH = -8
NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol the header declares (checked by the CPU test suite).
EXPORTS = (
    "mttkrp_strerror", "mttkrp_version", "mttkrp_selftest",
    "mttkrp_workspace_bytes", "mttkrp_all_workspace_bytes", "cp_als_workspace_bytes",
    "mttkrp_f64", "mttkrp_f32", "mttkrp_all_f64", "mttkrp_all_f32",
    "cp_als_f64", "cp_als_f32", "mttkrp_plan",
    "mttkrp_elem_f64", "mttkrp_elem_f32", "mttkrp_slice_f64", "mttkrp_slice_f32",
    "mttkrp_probe_read_grid", "mttkrp_probe_read", "mttkrp_probe_mfma_grid", "mttkrp_probe_mfma",
    "mttkrp_noalloc",
)


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("form", ctypes.c_int),
        ("layout", ctypes.c_int),
        ("k_modes", ctypes.c_int * 2),
        ("row_modes", ctypes.c_int * 2),
        ("outer_modes", ctypes.c_int * 3),
        ("mb", ctypes.c_int),
        ("nb", ctypes.c_int),
        ("b_in_lds", ctypes.c_int),
        ("vec", ctypes.c_int),
        ("k_len", ctypes.c_int64),
        ("rows", ctypes.c_int64),
        ("batches", ctypes.c_int64),
        ("splits", ctypes.c_int64),
        ("rtiles", ctypes.c_int64),
        ("grid", ctypes.c_int64),
        ("lds_bytes", ctypes.c_size_t),
        ("ws_bytes", ctypes.c_size_t),
        ("kchunks", ctypes.c_int64),
        ("waves", ctypes.c_int),
        ("launchable", ctypes.c_int),
        ("model_flop_s", ctypes.c_double),
        ("model_hbm_s", ctypes.c_double),
        ("model_l2_s", ctypes.c_double),
        ("model_lds_s", ctypes.c_double),
        ("model_s", ctypes.c_double),
        ("t_inf_s", ctypes.c_double),
        ("t_0_s", ctypes.c_double),
    ]

    def as_dict(self):
        d = {}
        for name, _ in self._fields_:
            v = getattr(self, name)
            d[name] = list(v) if isinstance(v, ctypes.Array) else (
                float(v) if isinstance(v, float) else int(v))
        return d


class MttkrpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {strerror(status)} (status {status})")


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} not found: build it with `python -m mttkrp_matrix_free_amd.build` "
                "(there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        I = ctypes.c_int
        sz = ctypes.c_size_t
        L.mttkrp_strerror.argtypes = [I]
        L.mttkrp_strerror.restype = ctypes.c_char_p
        L.mttkrp_version.restype = I
        L.mttkrp_selftest.restype = I
        L.mttkrp_selftest.argtypes = []
        for f in ("mttkrp_workspace_bytes",):
            getattr(L, f).argtypes = [P, I, i64, I, I, ctypes.POINTER(sz)]
            getattr(L, f).restype = I
        for f in ("mttkrp_all_workspace_bytes", "cp_als_workspace_bytes"):
            getattr(L, f).argtypes = [P, I, i64, I, ctypes.POINTER(sz)]
            getattr(L, f).restype = I
        for f in ("mttkrp_f64", "mttkrp_f32"):
            getattr(L, f).argtypes = [P, P, I, P, i64, I, P, P, sz, P]
            getattr(L, f).restype = I
        for f in ("mttkrp_all_f64", "mttkrp_all_f32"):
            getattr(L, f).argtypes = [P, P, I, P, i64, P, P, sz, P]
            getattr(L, f).restype = I
        for f in ("cp_als_f64", "cp_als_f32"):
            getattr(L, f).argtypes = [P, P, I, i64, P, P, I, ctypes.c_double, P, P, P, sz, P]
            getattr(L, f).restype = I
        for f in ("mttkrp_elem_f64", "mttkrp_elem_f32", "mttkrp_slice_f64", "mttkrp_slice_f32"):
            getattr(L, f).argtypes = [P, P, I, P, i64, I, P, P]
            getattr(L, f).restype = I
        L.mttkrp_probe_read_grid.restype = I
        L.mttkrp_probe_read_grid.argtypes = []
        L.mttkrp_probe_mfma_grid.restype = I
        L.mttkrp_probe_mfma_grid.argtypes = []
        L.mttkrp_probe_read.argtypes = [P, sz, P, P]
        L.mttkrp_probe_read.restype = I
        L.mttkrp_probe_mfma.argtypes = [I, i64, P, P]
        L.mttkrp_probe_mfma.restype = I
        L.mttkrp_noalloc.argtypes = [P, P, I, P, i64, I, P, I, P]
        L.mttkrp_noalloc.restype = I
        L.mttkrp_plan.argtypes = [P, I, i64, I, I, ctypes.POINTER(PlanInfo)]
        L.mttkrp_plan.restype = I
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().mttkrp_strerror(int(status)).decode()
