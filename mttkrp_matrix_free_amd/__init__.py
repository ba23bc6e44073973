"""Matrix-free dense MTTKRP for MI355X (gfx950).

Entry points (torch tensors on the GPU; the work runs in HIP kernels behind
the C ABI of include/mttkrp.h):

    mttkrp(X, factors, mode), mttkrp_all(X, factors), cp_als(X, factors, iters),
    plan(dims, rank, mode), workspace_bytes(...)

The binding is loaded on first use; a missing library raises (no CPU fallback).
"""
__all__ = ["mttkrp", "mttkrp_all", "cp_als", "plan", "workspace_bytes", "all_workspace_bytes",
           "cp_als_workspace_bytes", "MttkrpError"]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
