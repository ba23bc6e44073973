"""Python entry points over the C ABI (include/mttkrp.h).

Argument marshalling only: torch provides device memory and the current HIP
stream, every step of the computation runs in the library's kernels.

    mttkrp(X, factors, mode)        -> I_mode x R tensor
    mttkrp_all(X, factors)          -> list of I_m x R tensors
    cp_als(X, factors, iters)       -> (lambda, fit_hist, iters_done); factors updated in place
"""
from __future__ import annotations

import contextlib
import ctypes
import math
from typing import List, Optional, Sequence

import torch

from . import _lib
from ._lib import MttkrpError, PlanInfo

_DT = {torch.float64: ("f64", 8), torch.float32: ("f32", 4)}


def _dims(shape) -> ctypes.Array:
    return (ctypes.c_int64 * len(shape))(*[int(s) for s in shape])


def _ptrs(tensors) -> ctypes.Array:
    return (ctypes.c_void_p * len(tensors))(*[None if t is None else t.data_ptr() for t in tensors])


def _stream_handle(stream) -> Optional[int]:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check_tensor(X: torch.Tensor):
    if not isinstance(X, torch.Tensor) or not X.is_cuda:
        raise ValueError("X must be a CUDA (HIP) tensor")
    if X.dtype not in _DT:
        raise ValueError(f"unsupported dtype {X.dtype}; float64 or float32")
    if not X.is_contiguous():
        raise ValueError("X must be contiguous (row-major)")


def _check_factors(X: torch.Tensor, factors: Sequence[Optional[torch.Tensor]], skip: int = -1) -> int:
    if len(factors) != X.dim():
        raise ValueError(f"need {X.dim()} factors, got {len(factors)}")
    R = None
    for m, U in enumerate(factors):
        if U is None:
            if m == skip:
                continue
            raise ValueError(f"factor {m} is missing")
        if U.dtype != X.dtype or U.device != X.device:
            raise ValueError(f"factor {m} must match X in dtype and device")
        if U.dim() != 2 or U.shape[0] != X.shape[m] or not U.is_contiguous():
            raise ValueError(f"factor {m} must be a contiguous {X.shape[m]} x R matrix")
        if R is None:
            R = U.shape[1]
        elif U.shape[1] != R:
            raise ValueError("factors disagree on the rank")
    if R is None:
        raise ValueError("no factor given")
    return int(R)


def workspace_bytes(dims: Sequence[int], rank: int, mode: int, dtype=torch.float64) -> int:
    n = ctypes.c_size_t(0)
    st = _lib.lib().mttkrp_workspace_bytes(_dims(dims), len(dims), int(rank), int(mode),
                                           _DT[dtype][1], ctypes.byref(n))
    if st:
        raise MttkrpError(st, "mttkrp_workspace_bytes")
    return int(n.value)


def all_workspace_bytes(dims: Sequence[int], rank: int, dtype=torch.float64) -> int:
    n = ctypes.c_size_t(0)
    st = _lib.lib().mttkrp_all_workspace_bytes(_dims(dims), len(dims), int(rank), _DT[dtype][1],
                                               ctypes.byref(n))
    if st:
        raise MttkrpError(st, "mttkrp_all_workspace_bytes")
    return int(n.value)


def cp_als_workspace_bytes(dims: Sequence[int], rank: int, dtype=torch.float64) -> int:
    n = ctypes.c_size_t(0)
    st = _lib.lib().cp_als_workspace_bytes(_dims(dims), len(dims), int(rank), _DT[dtype][1],
                                           ctypes.byref(n))
    if st:
        raise MttkrpError(st, "cp_als_workspace_bytes")
    return int(n.value)


def plan(dims: Sequence[int], rank: int, mode: int, dtype=torch.float64) -> dict:
    info = PlanInfo()
    st = _lib.lib().mttkrp_plan(_dims(dims), len(dims), int(rank), int(mode), _DT[dtype][1],
                                ctypes.byref(info))
    if st:
        raise MttkrpError(st, "mttkrp_plan")
    return info.as_dict()


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _allocating_on(stream):
    """Context for the tensors a call allocates itself (workspace, outputs):
    torch's caching allocator ties a block to the stream that was current
    when it was allocated and may hand it out again as soon as it is freed,
    ordered only on that stream.  The kernels run on `stream`, so the block
    is allocated there: a workspace freed when the call returns is not
    reused by other work before the queued kernels are done with it."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def mttkrp(X: torch.Tensor, factors: Sequence[Optional[torch.Tensor]], mode: int,
           out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
           stream=None) -> torch.Tensor:
    """M = X_(mode) times the Khatri-Rao product of the other factors."""
    _check_tensor(X)
    R = _check_factors(X, factors, skip=mode)
    if not 0 <= mode < X.dim():
        raise ValueError("mode out of range")
    sfx, eb = _DT[X.dtype]
    need = workspace_bytes(X.shape, R, mode, X.dtype)
    with _allocating_on(stream):
        if out is None:
            out = torch.empty((X.shape[mode], R), dtype=X.dtype, device=X.device)
        if ws is None:
            ws = _workspace(need, X.device)
    fn = getattr(_lib.lib(), f"mttkrp_{sfx}")
    st = fn(X.data_ptr(), _dims(X.shape), X.dim(), _ptrs(factors), R, int(mode), out.data_ptr(),
            None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
            _stream_handle(stream))
    if st:
        raise MttkrpError(st, f"mttkrp_{sfx}")
    return out


def mttkrp_ablation(X: torch.Tensor, factors: Sequence[Optional[torch.Tensor]], mode: int,
                    kind: str, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The untiled matrix-free baselines (kind "elem" or "slice"): the same
    result as mttkrp(), for comparison only."""
    if kind not in ("elem", "slice"):
        raise ValueError("kind must be 'elem' or 'slice'")
    _check_tensor(X)
    R = _check_factors(X, factors, skip=mode)
    if not 0 <= mode < X.dim():
        raise ValueError("mode out of range")
    sfx, eb = _DT[X.dtype]
    if out is None:
        with _allocating_on(stream):
            out = torch.empty((X.shape[mode], R), dtype=X.dtype, device=X.device)
    fn = getattr(_lib.lib(), f"mttkrp_{kind}_{sfx}")
    st = fn(X.data_ptr(), _dims(X.shape), X.dim(), _ptrs(factors), R, int(mode), out.data_ptr(),
            _stream_handle(stream))
    if st:
        raise MttkrpError(st, f"mttkrp_{kind}_{sfx}")
    return out


def mttkrp_all(X: torch.Tensor, factors: Sequence[torch.Tensor],
               outs: Optional[List[torch.Tensor]] = None, ws: Optional[torch.Tensor] = None,
               stream=None) -> List[torch.Tensor]:
    """MTTKRP of every mode, ordered on the caller's stream (a long sweep also
    runs part of its modes on a second stream, forked from and joined back to
    the caller's)."""
    _check_tensor(X)
    R = _check_factors(X, factors)
    sfx, eb = _DT[X.dtype]
    with _allocating_on(stream):
        if outs is None:
            outs = [torch.empty((X.shape[m], R), dtype=X.dtype, device=X.device)
                    for m in range(X.dim())]
        if ws is None:
            ws = _workspace(all_workspace_bytes(X.shape, R, X.dtype), X.device)
    fn = getattr(_lib.lib(), f"mttkrp_all_{sfx}")
    st = fn(X.data_ptr(), _dims(X.shape), X.dim(), _ptrs(factors), R, _ptrs(outs),
            None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(),
            _stream_handle(stream))
    if st:
        raise MttkrpError(st, f"mttkrp_all_{sfx}")
    return outs


def prepare_all(X: torch.Tensor, factors: Sequence[torch.Tensor], outs: List[torch.Tensor],
                ws: Optional[torch.Tensor] = None, stream=None):
    """Check and marshal the arguments of mttkrp_all once; return a callable
    that enqueues the all-mode sweep with them (no per-call Python checks, for
    timing loops).  The tensors must stay alive and unchanged in shape."""
    _check_tensor(X)
    R = _check_factors(X, factors)
    sfx, eb = _DT[X.dtype]
    for m, o in enumerate(outs):
        if o.shape != (X.shape[m], R) or o.dtype != X.dtype or not o.is_contiguous():
            raise ValueError(f"output {m} must be a contiguous {X.shape[m]} x {R} tensor")
    need = all_workspace_bytes(X.shape, R, X.dtype)
    if ws is None:
        with _allocating_on(stream):
            ws = _workspace(need, X.device)
    fn = getattr(_lib.lib(), f"mttkrp_all_{sfx}")
    args = (ctypes.c_void_p(X.data_ptr()), _dims(X.shape), ctypes.c_int(X.dim()), _ptrs(factors),
            ctypes.c_int64(R), _ptrs(outs), ctypes.c_void_p(None if ws is None else ws.data_ptr()),
            ctypes.c_size_t(0 if ws is None else ws.numel()),
            ctypes.c_void_p(_stream_handle(stream)))
    keep = (X, list(factors), list(outs), ws)

    def run():
        st = fn(*args)
        if st:
            raise MttkrpError(st, f"mttkrp_all_{sfx}")
        return keep[2]

    return run


def cp_als(X: torch.Tensor, factors: List[torch.Tensor], iters: int, tol: float = 0.0,
           ws: Optional[torch.Tensor] = None, stream=None):
    """CP-ALS from the given factors (updated in place).

    Returns (lambda, fit_hist, iters_done, status); status is 0 or ENOTSPD.
    """
    _check_tensor(X)
    R = _check_factors(X, factors)
    sfx, eb = _DT[X.dtype]
    with _allocating_on(stream):
        lam = torch.empty(R, dtype=X.dtype, device=X.device)
        if ws is None:
            ws = _workspace(cp_als_workspace_bytes(X.shape, R, X.dtype), X.device)
    fit = (ctypes.c_double * max(1, iters))()
    done = ctypes.c_int(0)
    fn = getattr(_lib.lib(), f"cp_als_{sfx}")
    st = fn(X.data_ptr(), _dims(X.shape), X.dim(), R, _ptrs(factors), lam.data_ptr(), int(iters),
            float(tol), fit, ctypes.byref(done), ws.data_ptr(), ws.numel(), _stream_handle(stream))
    if st not in (0, _lib.ENOTSPD):
        raise MttkrpError(st, f"cp_als_{sfx}")
    hist = [fit[i] for i in range(iters)]
    return lam, hist, int(done.value), int(st)
