"""Benchmark of the all-mode matrix-free MTTKRP on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-configs]

One step is one all-mode sweep (MTTKRP of every mode, through the library's
all-mode entry point) over a tensor and factors already resident in HBM.  The
headline workload is the 512x512x512 fp64 tensor (entries N(0,1)) with rank
R = 2000 factors (U[0,1]): the high-rank, matrix-core-bound case, whose 1 GiB
tensor is four times the 256 MB last-level cache.

Printed: one JSON line with
  * the whole-job throughput (GFLOP/s, flops per mode 2 * R * prod(I));
  * `roofline` for the MTTKRP launches: algorithmic flops (or bytes) per mode
    launch over its average duration, from HIP events on the library's stream
    (the timed region's sweeps; for a tensor that fits in the last-level cache
    the cold-cache medians, where a 1 GiB buffer is read before every mode);
    the published peak; the fraction; the copy-calibrated HBM traffic from the
    committed counter summary; the plain cache model's bounds per mode;
  * `peaks`: the achievable HBM read rate and matrix-core rates measured by
    the library's probes, and the fractions against them;
  * `configs`: every benchmark workload (the five tensors, three ranks of the
    4-way one) with warm and cold per-mode times and fractions;
  * `cpu_baseline`: the CPU oracle timed on a bounded sample of the headline
    workload on this host's CPU share;
  * comparison legs: the explicit Khatri-Rao + vendor GEMM MTTKRP and the
    untiled ELEM / SLICE kernels where they finish in seconds.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PEAK_TFLOPS = {"f64": 78.6, "f32": 157.3}
MALL_BYTES = 256 * 1024 * 1024  # last-level (Infinity) cache of the device
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = "3way_512cube_f64_R2000"
METRIC = "MTTKRP GFLOP/s (all-mode avg) and % of HBM/FP64 roofline, 1 MI355X"
# wave tiles (mb, nb) and workgroup sizes the tile sweep tries
SWEEP_TILES = [(2, 1), (2, 2), (2, 4), (2, 8), (4, 1), (4, 2), (4, 4)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sources_digest() -> str:
    """sha256 of the MTTKRP kernel sources, their planner and launchers, with
    comments and blank space removed: traffic counters taken on other code no
    longer describe the kernels that run, while an edit of a comment leaves
    them valid.  The CP-ALS kernels and their header, the ablation baselines,
    the measurement probes and the C ABI file do not take part in the MTTKRP
    launches the counters describe."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mttkrp_matrix_free_amd", "csrc", "*")))
    skip = ("als_kernels.hip", "als_kernels.hpp", "ablation_kernels.hip", "peak_probe.hip",
            "capi.cpp", "noalloc.hip")
    for f in files:
        if os.path.isfile(f) and os.path.basename(f) not in skip:
            with open(f, "r", encoding="utf-8") as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(os.path.basename(f).encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per mode launch from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE runs scaled by the copy calibration),
    or None when there is none or the kernel sources changed since."""
    import glob
    digest = kernel_sources_digest()
    for path in sorted(glob.glob(os.path.join(PROFILES, "*counters*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec.get("workload") == workload and rec.get("sources_sha256") == digest:
                        return rec
    return None


def khatri_rao(U, modes):
    """The explicit Khatri-Rao matrix of the factors of `modes` (in mode
    order): row (i_a, i_b, ...) with the last index fastest, column r holds
    prod_m U_m(i_m, r)."""
    R = U[modes[0]].shape[1]
    K = U[modes[0]]
    for m in modes[1:]:
        K = (K[:, None, :] * U[m][None, :, :]).reshape(-1, R)
    return K


def unfold(X, n):
    """Mode-n unfolding of a row-major tensor (columns: the other indices in
    mode order, the last fastest).  A view for the first and last modes (the
    last as a transposed view), a permuted copy otherwise."""
    d = X.dim()
    if n == 0:
        return X.reshape(X.shape[0], -1)
    if n == d - 1:
        return X.reshape(-1, X.shape[-1]).t()
    others = [m for m in range(d) if m != n]
    return X.permute(n, *others).contiguous().reshape(X.shape[n], -1)


def explicit_kr_mttkrp(X, U, n):
    """The matrix-based MTTKRP the GenTen page compares against (its Fig. 3):
    form the Khatri-Rao product of the other factors explicitly, unfold X
    along mode n, and multiply with the vendor GEMM (torch.matmul, i.e.
    hipBLASLt / rocBLAS).  A comparison baseline only: the product path never
    forms the Khatri-Rao matrix.  Returns (M_n, khatri_rao_bytes,
    unfold_copy_bytes)."""
    import torch
    d = X.dim()
    K = khatri_rao(U, [m for m in range(d) if m != n])
    Xn = unfold(X, n)
    copy_bytes = 0 if n in (0, d - 1) else Xn.numel() * Xn.element_size()
    return torch.matmul(Xn, K), K.numel() * K.element_size(), copy_bytes


def cpu_share():
    """Threads the CPU baseline may use: the host's CPU share as the job
    environment states it (OMP_NUM_THREADS), within this process's affinity
    set; and that set's size and the CPU model for the report."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    share = int(env) if env.isdigit() and int(env) > 0 else aff
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return min(share, aff), aff, model


def stats(v):
    import numpy as np
    return {"median": round(float(np.median(v)), 5), "min": round(float(np.min(v)), 5),
            "max": round(float(np.max(v)), 5)}


class Workload:
    """A workload resident on the device with its sweep prepared."""

    def __init__(self, name, dev):
        import numpy as np
        import torch

        from mttkrp_matrix_free_amd import api, inputs
        t0 = time.time()
        self.p = inputs.workload(name)
        self.name = name
        self.gen_s = time.time() - t0
        p = self.p
        self.dims = p.dims
        self.d = len(p.dims)
        self.R = p.rank
        self.N = int(np.prod(p.dims))
        self.s = p.X.dtype.itemsize
        self.dt = "f64" if self.s == 8 else "f32"
        self.X = torch.from_numpy(p.X).to(dev)
        self.U = [torch.from_numpy(u).to(dev) for u in p.factors]
        self.outs = [torch.empty((p.dims[m], self.R), dtype=self.X.dtype, device=dev)
                     for m in range(self.d)]
        self.ws_bytes = api.all_workspace_bytes(p.dims, self.R, self.X.dtype)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.stream = torch.cuda.current_stream()
        self.sweep = api.prepare_all(self.X, self.U, self.outs, ws=self.ws, stream=self.stream)
        self.flops_mode = 2.0 * self.R * self.N
        self.bytes_mode = [self.s * (self.N + self.R * sum(p.dims[m] for m in range(self.d) if m != n)
                                     + self.R * p.dims[n]) for n in range(self.d)]
        self.plans = [api.plan(p.dims, self.R, n, self.X.dtype) for n in range(self.d)]
        torch.cuda.synchronize()

    def free(self):
        import torch
        del self.X, self.U, self.outs, self.ws, self.sweep
        torch.cuda.empty_cache()

    def mode_call(self, n):
        from mttkrp_matrix_free_amd import api
        api.mttkrp(self.X, self.U, n, out=self.outs[n], ws=self.ws, stream=self.stream)

    def preheat(self, seconds):
        """The chip raises its clocks only after some tens of milliseconds of
        sustained load (measured on the 256^3 sweep: 0.563 of the roofline
        after 3 warm-up sweeps, 0.615 after 300): sweeps run for `seconds`
        (untimed) so that the timed region sees the steady state of a long
        CP-ALS run."""
        import torch
        t = time.perf_counter()
        n = 0
        while time.perf_counter() - t < seconds:
            for _ in range(4):
                self.sweep()
            n += 4
            torch.cuda.synchronize()
        return n

    def timed_sweeps(self, steps, warmup):
        """Exactly `steps` all-mode sweeps back to back between two HIP events
        on the library's stream (an event between sweeps would drain the
        queue there), bracketed by device synchronisations."""
        import torch
        for _ in range(warmup):
            self.sweep()
        ev_a = torch.cuda.Event(enable_timing=True)
        ev_b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        ev_a.record(self.stream)
        for _ in range(steps):
            self.sweep()
        t_issued = time.perf_counter()
        ev_b.record(self.stream)
        torch.cuda.synchronize()
        t_end = time.perf_counter()
        return {"wall_s": t_end - t_start, "event_ms": ev_a.elapsed_time(ev_b),
                "issue_us_per_sweep": (t_issued - t_start) * 1e6 / steps}

    def per_mode(self, reps, cold, flush=None):
        """Per-mode time of the single-mode entry point on one stream (HIP
        events around each call): back to back, or after reading `flush` (a
        1 GiB buffer, four times the last-level cache) outside the events."""
        import torch
        if reps <= 0:
            return None
        ms = [[] for _ in range(self.d)]
        for _ in range(reps):
            for n in range(self.d):
                if cold:
                    flush.sum()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(self.stream)
                self.mode_call(n)
                b.record(self.stream)
                torch.cuda.synchronize()
                ms[n].append(a.elapsed_time(b))
        return ms

    def model(self):
        return [{"t_p_ms": round(pl["model_s"] * 1e3, 5),
                 "flop_ms": round(pl["model_flop_s"] * 1e3, 5),
                 "hbm_ms": round(pl["model_hbm_s"] * 1e3, 5),
                 "l2_ms": round(pl["model_l2_s"] * 1e3, 5),
                 "lds_ms": round(pl["model_lds_s"] * 1e3, 5),
                 "t_inf_ms": round(pl["t_inf_s"] * 1e3, 5),
                 "t_0_ms": round(pl["t_0_s"] * 1e3, 5),
                 "tile": [pl["mb"], pl["nb"], pl["waves"]]} for pl in self.plans]

    def bound(self):
        import numpy as np
        ai = float(np.mean([self.flops_mode / b for b in self.bytes_mode]))
        ridge = PEAK_TFLOPS[self.dt] * 1e12 / (HBM_PEAK_GBS * 1e9)
        return ("hbm" if ai < ridge else "mfma"), ai

    def fraction(self, mode_ms_sum):
        """(achieved, peak, unit, frac) for modes taking mode_ms_sum in all."""
        bound, _ = self.bound()
        t = mode_ms_sum / 1e3
        if bound == "hbm":
            a = sum(self.bytes_mode) / t / 1e9
            return round(a, 1), HBM_PEAK_GBS, "GB/s", round(a / HBM_PEAK_GBS, 4)
        a = self.d * self.flops_mode / t / 1e12
        return round(a, 2), PEAK_TFLOPS[self.dt], "TFLOP/s", round(a / PEAK_TFLOPS[self.dt], 4)

    def fits_cache(self):
        return self.N * self.s <= MALL_BYTES


def measure_peaks(dev):
    """Achievable rates from the library's probes: a 4 GiB streaming read
    (sixteen times the last-level cache, so it comes from HBM) and
    dependency-free fp64 / fp32 MFMA loops.  Best of five each."""
    import ctypes

    import torch

    from mttkrp_matrix_free_amd import _lib
    L = _lib.lib()
    s = torch.cuda.current_stream()
    h = s.cuda_stream
    out = {}
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 8, dtype=torch.float64, device=dev)
    sink = torch.empty(L.mttkrp_probe_read_grid(), dtype=torch.int32, device=dev)
    best = None
    for _ in range(6):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        st = L.mttkrp_probe_read(ctypes.c_void_p(buf.data_ptr()), ctypes.c_size_t(nbytes),
                                 ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(h))
        b.record(s)
        torch.cuda.synchronize()
        if st:
            raise _lib.MttkrpError(st, "mttkrp_probe_read")
        t = a.elapsed_time(b)
        best = t if best is None else min(best, t)
    out["hbm_read_gbs"] = round(nbytes / (best / 1e3) / 1e9, 1)
    del buf, sink
    msink = torch.empty(4 * L.mttkrp_probe_mfma_grid(), dtype=torch.float64, device=dev)
    for eb, key in ((8, "f64"), (4, "f32")):
        iters = 16384 if eb == 8 else 32768  # about 7 ms at the published rates
        flops = L.mttkrp_probe_mfma_grid() * 4 * 8 * 2048.0 * iters
        best = None
        for _ in range(6):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(s)
            st = L.mttkrp_probe_mfma(eb, ctypes.c_int64(iters), ctypes.c_void_p(msink.data_ptr()),
                                     ctypes.c_void_p(h))
            b.record(s)
            torch.cuda.synchronize()
            if st:
                raise _lib.MttkrpError(st, "mttkrp_probe_mfma")
            t = a.elapsed_time(b)
            best = t if best is None else min(best, t)
        out[f"mfma_{key}_tflops"] = round(flops / (best / 1e3) / 1e12, 2)
    del msink
    torch.cuda.empty_cache()
    return out


def config_entry(w, sweep_ms, warm, cold, peaks):
    """Per-mode and all-mode figures of one workload."""
    import numpy as np
    bound, ai = w.bound()
    warm_med = [float(np.median(v)) for v in warm] if warm else None
    cold_med = [float(np.median(v)) for v in cold] if cold else None
    e = {
        "workload": w.name, "dims": list(w.dims), "rank": w.R, "dtype": w.dt,
        "bound": bound, "ai_flop_per_byte": round(ai, 2),
        "tensor_fits_last_level_cache": w.fits_cache(),
        "sweep_ms": round(sweep_ms, 5),
        "gflops_all_mode_sweep": round(w.d * w.flops_mode / (sweep_ms / 1e3) / 1e9, 1),
        "frac_sweep": w.fraction(sweep_ms)[3],
    }
    if warm_med:
        e["warm_ms_per_mode"] = [stats(v) for v in warm]
        e["frac_warm"] = w.fraction(sum(warm_med))[3]
    if cold_med:
        e["cold_ms_per_mode"] = [stats(v) for v in cold]
        e["gflops_all_mode_cold"] = round(w.d * w.flops_mode / (sum(cold_med) / 1e3) / 1e9, 1)
        e["tensor_gbs_cold"] = [round(w.N * w.s / (v / 1e3) / 1e9, 1) for v in cold_med]
        e["frac_cold"] = w.fraction(sum(cold_med))[3]
    # the fraction the roofline uses: cold when the tensor fits in the
    # last-level cache (warm repeats would read it from there), else the sweep
    e["frac"] = e["frac_cold"] if (w.fits_cache() and cold_med) else e["frac_sweep"]
    if peaks:
        ach = (peaks["hbm_read_gbs"] / HBM_PEAK_GBS if bound == "hbm"
               else peaks[f"mfma_{w.dt}_tflops"] / PEAK_TFLOPS[w.dt])
        e["frac_of_achievable"] = round(e["frac"] / ach, 4)
    e["model_per_mode"] = w.model()
    return e


def als_leg(w, iters):
    """CP-ALS: time per sweep of the whole driver (per mode: MTTKRP, Hadamard
    of Grams, Cholesky, row solves, normalization, Gram refresh; then the fit,
    one read-back), and the share of it the MTTKRP launches take.  A call also
    has a fixed set-up (||X||^2, the starting Grams, the host's set-up), so the
    steady per-sweep time is reported as well: the difference between an
    `iters`-sweep call and a one-sweep call, over iters - 1."""
    import torch

    from mttkrp_matrix_free_amd import api
    ws_als = torch.empty(api.cp_als_workspace_bytes(w.dims, w.R, w.X.dtype), dtype=torch.uint8,
                         device=w.X.device)
    U0 = [u.clone() for u in w.U]
    Ua = [u.clone() for u in U0]
    api.cp_als(w.X, Ua, iters=min(2, iters), ws=ws_als, stream=w.stream)  # warm-up

    def timed_call(n):
        Ub = [u.clone() for u in U0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        out = api.cp_als(w.X, Ub, iters=n, ws=ws_als, stream=w.stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, out, Ub

    t_one = timed_call(1)[0] if iters > 1 else None
    t_call, (_, hist, done, st), Ua = timed_call(iters)
    t_als = t_call / max(1, done)
    t_steady = (t_call - t_one) / (done - 1) if (t_one is not None and done > 1) else None
    # the same iterations' MTTKRP launches alone, mode after mode on one
    # stream as the driver issues them
    ev_c = torch.cuda.Event(enable_timing=True)
    ev_d = torch.cuda.Event(enable_timing=True)
    ev_c.record(w.stream)
    for _ in range(iters):
        for n in range(w.d):
            api.mttkrp(w.X, Ua, n, out=w.outs[n], ws=w.ws, stream=w.stream)
    ev_d.record(w.stream)
    torch.cuda.synchronize()
    t_mt = ev_c.elapsed_time(ev_d) / 1e3 / iters
    del ws_als
    out = {"ms_per_iter": round(t_als * 1e3, 4), "iters": int(done), "status": int(st),
           "final_fit": round(float(hist[done - 1]), 6) if done else None,
           "mttkrp_ms_per_iter": round(t_mt * 1e3, 4),
           "mttkrp_share": round(t_mt / t_als, 3)}
    if t_steady is not None and t_steady > 0:
        out["ms_per_sweep_steady"] = round(t_steady * 1e3, 4)
        out["mttkrp_share_steady"] = round(t_mt / t_steady, 3)
        out["call_setup_ms"] = round((t_one - t_steady) * 1e3, 4)
    return out


def cpu_baseline(w, budget_s):
    """The CPU oracle on output rows of the workload, row chunks of every
    mode in turn, until the time budget is spent."""
    import oracle
    nthreads, aff, model = cpu_share()
    done_flops = 0.0
    t_cpu = 0.0
    rows_done = [0] * w.d
    while t_cpu < budget_s:
        progressed = False
        for n in range(w.d):
            if rows_done[n] >= w.dims[n] or t_cpu >= budget_s:
                continue
            rr = list(range(rows_done[n], min(w.dims[n], rows_done[n] + nthreads)))
            a = time.perf_counter()
            oracle.mttkrp(w.p.X, w.p.factors, n, rows=rr, nthreads=nthreads)
            t_cpu += time.perf_counter() - a
            done_flops += w.flops_mode * len(rr) / w.dims[n]
            rows_done[n] += len(rr)
            progressed = True
        if not progressed:
            break
    return {"value": round(done_flops / t_cpu / 1e9, 4), "unit": "GFLOP/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"output rows {rows_done} of modes 0..{w.d - 1} of {w.name} "
                      f"({t_cpu:.1f} s; long-double oracle, OpenMP over rows)",
            "threads_used": nthreads, "affinity_cpus": aff, "cpu_model": model,
            "threads_note": "the job's CPU share (OMP_NUM_THREADS) within the affinity set"}


def gemm_leg(w):
    """The matrix-based comparison (explicit Khatri-Rao matrix, unfolded X,
    vendor GEMM): time per mode with its extra memory, and its largest
    difference from this library's outputs."""
    import torch

    from mttkrp_matrix_free_amd import api
    ms, kr_b, cp_b, diff = [], [], [], 0.0
    parts = {"khatri_rao_ms": [], "unfold_ms": [], "gemm_ms": []}
    for n in range(w.d):
        explicit_kr_mttkrp(w.X, w.U, n)  # warm-up (library handles, allocations)
        torch.cuda.synchronize()
        reps = 3
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        t_parts = [0.0, 0.0, 0.0]
        for _ in range(reps):
            ev[0].record(w.stream)
            K = khatri_rao(w.U, [m for m in range(w.d) if m != n])
            ev[1].record(w.stream)
            Xn = unfold(w.X, n)
            ev[2].record(w.stream)
            Mn = torch.matmul(Xn, K)
            ev[3].record(w.stream)
            torch.cuda.synchronize()
            for i in range(3):
                t_parts[i] += ev[i].elapsed_time(ev[i + 1]) / reps
        for key, v in zip(parts, t_parts):
            parts[key].append(round(v, 4))
        ms.append(sum(t_parts))
        kr_b.append(K.numel() * K.element_size())
        cp_b.append(0 if n in (0, w.d - 1) else Xn.numel() * Xn.element_size())
        del K, Xn
        api.mttkrp(w.X, w.U, n, out=w.outs[n], ws=w.ws, stream=w.stream)
        torch.cuda.synchronize()
        ref = w.outs[n].double()
        diff = max(diff, float((Mn.double() - ref).norm() / ref.norm().clamp_min(1e-300)))
        del Mn
    torch.cuda.empty_cache()
    return {"kind": "explicit Khatri-Rao + torch.matmul (vendor GEMM)",
            "ms_per_mode": [round(v, 4) for v in ms], **parts,
            "gflops_all_mode": round(w.d * w.flops_mode / (sum(ms) / 1e3) / 1e9, 2),
            "khatri_rao_bytes_per_mode": kr_b, "unfold_copy_bytes_per_mode": cp_b,
            "library_workspace_bytes": w.ws_bytes,
            "rel_diff_vs_library": diff}


def ablation_leg(w):
    """The untiled matrix-free baselines (one thread per element with
    atomics; one workgroup per slice), where they finish in seconds."""
    import torch

    from mttkrp_matrix_free_amd import api
    if w.N * w.R > (1 << 31):
        return {"skipped": f"N * R = {w.N * w.R} products per mode is past the 2^31 bound"}
    res = {}
    for kind in ("elem", "slice"):
        ms_k, diff = [], 0.0
        for n in range(w.d):
            Mk = api.mttkrp_ablation(w.X, w.U, n, kind, stream=w.stream)  # warm-up
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(w.stream)
            api.mttkrp_ablation(w.X, w.U, n, kind, out=Mk, stream=w.stream)
            b.record(w.stream)
            torch.cuda.synchronize()
            ms_k.append(a.elapsed_time(b))
            w.mode_call(n)
            torch.cuda.synchronize()
            ref = w.outs[n].double()
            diff = max(diff, float((Mk.double() - ref).norm() / ref.norm().clamp_min(1e-300)))
        res[kind] = {"ms_per_mode": [round(v, 4) for v in ms_k],
                     "gflops_all_mode": round(w.d * w.flops_mode / (sum(ms_k) / 1e3) / 1e9, 2),
                     "rel_diff_vs_library": diff}
    return res


def tile_sweep(w, reps):
    """The tile heuristic against an exhaustive sweep: every wave tile
    (mb, nb) and workgroup size that has a kernel for the mode's plan is
    forced through MTTKRP_FORCE_TILE, timed (median of `reps` warm calls)
    and its output checked against the planner's own; the plain cache
    model's T(p) is reported beside each."""
    import numpy as np
    import torch

    from mttkrp_matrix_free_amd import api
    tol = 1e-12 if w.s == 8 else 1e-5
    res = []
    for n in range(w.d):
        os.environ.pop("MTTKRP_FORCE_TILE", None)
        base_pl = api.plan(w.dims, w.R, n, w.X.dtype)
        ref = api.mttkrp(w.X, w.U, n).double()
        rows = []
        for mb, nb in SWEEP_TILES:
            for wv in (4, 8):
                os.environ["MTTKRP_FORCE_TILE"] = f"{mb},{nb},{wv}"
                pl = api.plan(w.dims, w.R, n, w.X.dtype)
                if not pl["launchable"]:
                    continue
                need = api.workspace_bytes(w.dims, w.R, n, w.X.dtype)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device=w.X.device)
                out = torch.empty_like(w.outs[n])
                api.mttkrp(w.X, w.U, n, out=out, ws=ws, stream=w.stream)  # warm-up
                ts = []
                for _ in range(reps):
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(w.stream)
                    api.mttkrp(w.X, w.U, n, out=out, ws=ws, stream=w.stream)
                    b.record(w.stream)
                    torch.cuda.synchronize()
                    ts.append(a.elapsed_time(b))
                err = float((out.double() - ref).norm() / ref.norm().clamp_min(1e-300))
                rows.append({"tile": [mb, nb, wv], "ms": round(float(np.median(ts)), 5),
                             "model_ms": round(pl["model_s"] * 1e3, 5),
                             "splits": pl["splits"], "kchunks": pl["kchunks"],
                             "rel_diff": err, "ok": err <= tol})
                del ws, out
        os.environ.pop("MTTKRP_FORCE_TILE", None)
        mine = [mb_ for mb_ in rows if mb_["tile"] == [base_pl["mb"], base_pl["nb"], base_pl["waves"]]]
        best = min(rows, key=lambda r: r["ms"])
        by_model = min(rows, key=lambda r: r["model_ms"])
        res.append({"mode": n, "heuristic": [base_pl["mb"], base_pl["nb"], base_pl["waves"]],
                    "heuristic_ms": mine[0]["ms"] if mine else None,
                    "best": best["tile"], "best_ms": best["ms"],
                    "model_pick": by_model["tile"], "model_pick_ms": by_model["ms"],
                    "heuristic_over_best": round(mine[0]["ms"] / best["ms"], 4) if mine else None,
                    "all_ok": all(r["ok"] for r in rows), "tiles": rows})
        torch.cuda.empty_cache()
    return res


def main():
    from mttkrp_matrix_free_amd import inputs  # workload generators (numpy only)

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--cold-reps", type=int, default=5)
    ap.add_argument("--warm-reps", type=int, default=5)
    ap.add_argument("--preheat", type=float, default=0.3, help="seconds of untimed sweeps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-als", action="store_true", help="skip the CP-ALS legs")
    ap.add_argument("--als-iters", type=int, default=0,
                    help="time this many CP-ALS sweeps on the headline workload (CP-ALS "
                         "workloads get their own sweep count in the per-config block)")
    ap.add_argument("--no-gemm-baseline", action="store_true",
                    help="skip the explicit Khatri-Rao + vendor GEMM comparison")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the untiled ELEM / SLICE baselines")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config block (every other benchmark workload)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak probes")
    ap.add_argument("--tile-sweep", action="store_true",
                    help="also time every wave tile of the headline workload's modes")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: there is no multi-GPU path "
              "(the MTTKRP would shard by slabs of the first mode, one slab per GPU).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        # A copy of known size: its FETCH_SIZE / WRITE_SIZE counters read what
        # 1 GiB of HBM traffic looks like on this device.
        a = torch.ones(1 << 27, dtype=torch.float64, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": a.numel() * 8, "launches": 3}), flush=True)
        return

    from mttkrp_matrix_free_amd import api

    peaks = None if args.no_peaks else measure_peaks(dev)
    if peaks:
        log(f"[bench] achievable peaks {peaks}")

    # ---- headline workload ----
    w = Workload(args.workload, dev)
    log(f"[bench] workload {w.name} generated in {w.gen_s:.1f} s")
    n_pre = w.preheat(args.preheat)
    t = w.timed_sweeps(args.steps, args.warmup)
    ms_per_step = t["wall_s"] * 1e3 / args.steps
    sweep_ms = t["event_ms"] / args.steps
    value = w.d * w.flops_mode / (t["wall_s"] / args.steps) / 1e9
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    warm = w.per_mode(args.warm_reps, cold=False)
    cold = w.per_mode(args.cold_reps, cold=True, flush=flush) if args.cold_reps > 0 else None
    head = config_entry(w, sweep_ms, warm, cold, peaks)
    log(f"[bench] headline {head}")

    # ---- roofline of the MTTKRP launches: algorithmic flops (or bytes) per
    # mode launch over the average launch time -- the timed region's sweeps
    # (HIP events on the library's stream), or the cold-cache medians for a
    # tensor the last-level cache would hold between warm repeats ----
    bound, ai = w.bound()
    use_cold = w.fits_cache() and cold is not None
    basis_ms = sum(float(np.median(v)) for v in cold) if use_cold else sweep_ms
    achieved, peak, unit, frac = w.fraction(basis_ms)
    roof = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": frac,
            "basis": ("cold-cache per-mode medians (a 1 GiB read before each mode)" if use_cold
                      else "timed-region sweeps (HIP events on the library's stream)"),
            "frac_sweep": head["frac_sweep"], "frac_warm_per_mode": head.get("frac_warm"),
            "frac_cold": head.get("frac_cold")}
    if peaks:
        roof["frac_of_achievable"] = head.get("frac_of_achievable")
        roof["achievable_peak"] = (peaks["hbm_read_gbs"] if bound == "hbm"
                                   else peaks[f"mfma_{w.dt}_tflops"])
    tr = measured_traffic(w.name)
    roof["traffic"] = round(float(np.mean(tr["bytes_per_mode"])), 0) if tr else None
    roof["traffic_unit"] = "bytes/launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
    roof["per_launch_ms"] = round(basis_ms / w.d, 5)
    roof["sweep_ms"] = round(sweep_ms, 5)
    roof["algorithmic_bytes_per_launch"] = w.bytes_mode
    roof["flops_per_launch"] = w.flops_mode
    roof["model_per_mode"] = head["model_per_mode"]

    # ---- host time: the all-mode call's validation, planning and launches
    # (wall clock of the issuing loop), and one plan query through ctypes ----
    t_plan = time.perf_counter()
    for _ in range(50):
        for n in range(w.d):
            api.plan(w.dims, w.R, n, w.X.dtype)
    host = {"issue_us_per_sweep": round(t["issue_us_per_sweep"], 2),
            "plan_query_us_per_mode": round((time.perf_counter() - t_plan) * 1e6 / (50 * w.d), 2)}

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_seconds)
        log(f"[bench] cpu oracle {cpu}")

    als = None
    if args.als_iters and not args.no_als:
        als = als_leg(w, args.als_iters)
        log(f"[bench] cp-als {als}")

    gemm = None
    if not args.no_gemm_baseline:
        gemm = gemm_leg(w)
        log(f"[bench] explicit-KR GEMM baseline {gemm}")
    ablation = None
    if not args.no_ablation:
        ablation = ablation_leg(w)
        log(f"[bench] ablation baselines {ablation}")
    sweep_res = None
    if args.tile_sweep:
        sweep_res = tile_sweep(w, reps=3 if w.flops_mode > 1e11 else 7)
        log(f"[bench] tile sweep {json.dumps(sweep_res)}")
    w.free()

    # ---- every other benchmark workload: warm sweeps, warm and cold
    # per-mode times, the same fractions (CP-ALS workloads: their sweeps) ----
    configs = [head]
    if not args.no_configs:
        for name in inputs.WORKLOADS:
            if name == w.name:
                continue
            c = Workload(name, dev)
            c.preheat(min(args.preheat, 0.15))
            tc = c.timed_sweeps(10, 2)
            wc = c.per_mode(args.warm_reps, cold=False)
            cc = c.per_mode(3, cold=True, flush=flush)
            e = config_entry(c, tc["event_ms"] / 10, wc, cc, peaks)
            if c.p.als_iters and not args.no_als:
                e["cp_als"] = als_leg(c, c.p.als_iters)
            log(f"[bench] config {e}")
            configs.append(e)
            c.free()
    del flush

    cfg = {"workload": w.name, "dims": list(w.dims), "rank": w.R, "modes": list(range(w.d)),
           "step": "all-mode MTTKRP sweep", "cache": "warm (back-to-back sweeps)"}
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preheat": {"seconds": args.preheat, "sweeps": n_pre},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dt,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "peaks": peaks,
        "host": host,
        "cpu_baseline": cpu,
        "cp_als": als,
        "gemm_baseline": gemm,
        "ablation": ablation,
        "tile_sweep": sweep_res,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
