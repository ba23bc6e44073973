"""Benchmark of the all-mode matrix-free MTTKRP on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload c2] [--no-cpu]

One step is one all-mode sweep (MTTKRP of every mode, in mode order, on one
stream) over a tensor and factors already resident in HBM.  The default
workload is the 256x256x256 fp64 tensor built from an exact rank-32 CP model
plus Gaussian noise of standard deviation 1e-3, R = 32.  Other workloads (--workload) are for
exploration; the JSON line names the one measured.

Printed: one JSON line with the whole-job throughput (GFLOP/s, flops per mode
2 * R * prod(I)), a roofline object for the MTTKRP launches (algorithmic
bytes or flops per launch over their average duration, from HIP events on the
library's stream inside the timed region), a cold-cache measurement (a 1 GiB
buffer is read before each mode so the tensor cannot be served from the
256 MB last-level cache), and the CPU oracle timed on a bounded sample of the
same workload on this host's cores.
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
PREHEAT_S = 0.3
PEAK_TFLOPS = {"f64": 78.6, "f32": 157.3}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_sources_digest() -> str:
    """sha256 of the MTTKRP kernel sources, their planner and launchers, with
    comments and blank space removed: traffic counters taken on other code no
    longer describe the kernels that run, while an edit of a comment leaves
    them valid.  The CP-ALS kernels (als_kernels.hip) and the ablation
    baselines (ablation_kernels.hip) do not take part in the MTTKRP launches
    the counters describe."""
    import glob
    import hashlib
    import re
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(ROOT, "mttkrp_matrix_free_amd", "csrc", "*")))
    skip = ("als_kernels.hip", "ablation_kernels.hip")
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    from mttkrp_matrix_free_amd import inputs  # workload generators (numpy only)

    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="3way_256cube_f64_R32_cp32",
                    choices=sorted(inputs.WORKLOADS))
    ap.add_argument("--cold-reps", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-als", action="store_true", help="skip the CP-ALS timing (5-way workload)")
    ap.add_argument("--als-iters", type=int, default=0,
                    help="time this many CP-ALS sweeps on any workload (default: ten on the "
                         "5-way workload only)")
    ap.add_argument("--no-gemm-baseline", action="store_true",
                    help="skip the explicit Khatri-Rao + vendor GEMM comparison")
    ap.add_argument("--no-ablation", action="store_true",
                    help="skip the untiled ELEM / SLICE baselines")
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

    from mttkrp_matrix_free_amd import api

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

    t0 = time.time()
    p = inputs.workload(args.workload)
    log(f"[bench] workload {p.name} generated in {time.time() - t0:.1f} s")
    dims = p.dims
    d = len(dims)
    R = p.rank
    N = int(np.prod(dims))
    s = p.X.dtype.itemsize
    dt_name = "f64" if s == 8 else "f32"
    X = torch.from_numpy(p.X).to(dev)
    U = [torch.from_numpy(u).to(dev) for u in p.factors]
    outs = [torch.empty((dims[m], R), dtype=X.dtype, device=dev) for m in range(d)]
    ws_bytes = api.all_workspace_bytes(dims, R, X.dtype)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    flops_mode = 2.0 * R * N
    bytes_mode = [s * (N + R * sum(dims[m] for m in range(d) if m != n) + R * dims[n])
                  for n in range(d)]

    # One step: the all-mode sweep through the C ABI (mttkrp_all), with its
    # arguments marshalled once so the host keeps ahead of the GPU.
    sweep = api.prepare_all(X, U, outs, ws=ws, stream=stream)

    # Pre-heat (untimed): the chip raises its clocks only after some tens of
    # milliseconds of sustained load (measured on the 256^3 sweep: 0.563 of
    # the roofline after 3 warm-up sweeps, 0.615 after 300), so sweeps run for
    # PREHEAT_S seconds before the W warm-up steps; the timed region then
    # measures the steady state that a long CP-ALS run sees.
    t_pre = time.perf_counter()
    n_pre = 0
    while time.perf_counter() - t_pre < PREHEAT_S:
        for _ in range(8):
            sweep()
        n_pre += 8
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        sweep()
    torch.cuda.synchronize()

    # ---- timed region: exactly `steps` all-mode sweeps, back to back, between
    # two HIP events on the library's stream (an event between sweeps would
    # drain the GPU's queue there) ----
    ev_a = torch.cuda.Event(enable_timing=True)
    ev_b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev_a.record(stream)
    for _ in range(args.steps):
        sweep()
    ev_b.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    wall = t_end - t_start
    ms_per_step = wall * 1e3 / args.steps
    sweep_avg = ev_a.elapsed_time(ev_b) / args.steps
    value = d * flops_mode / (wall / args.steps) / 1e9

    # ---- cold cache: a 1 GiB read of another buffer before each mode, outside
    # the event pair, evicts the tensor from the last-level cache ----
    cold = None
    if args.cold_reps > 0:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        cms = [[] for _ in range(d)]
        for _ in range(args.cold_reps):
            for n in range(d):
                sink = flush.sum()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                api.mttkrp(X, U, n, out=outs[n], ws=ws, stream=stream)
                b.record(stream)
                torch.cuda.synchronize()
                cms[n].append(a.elapsed_time(b))
        del flush
        cold_med = [float(np.median(v)) for v in cms]
        cold = {
            "ms_per_mode_median": [round(v, 5) for v in cold_med],
            "gflops_all_mode": round(d * flops_mode / (sum(cold_med) / 1e3) / 1e9, 2),
            "tensor_gbs_per_mode": [round(N * s / (v / 1e3) / 1e9, 1) for v in cold_med],
            "reps": args.cold_reps,
        }

    # ---- roofline of the MTTKRP launches: the sweeps' mode launches over the
    # event time of the timed region, i.e. the algorithmic bytes (or flops)
    # per launch over the average launch time ----
    ai = [flops_mode / b for b in bytes_mode]
    peak_f = PEAK_TFLOPS[dt_name] * 1e12
    ridge = peak_f / (HBM_PEAK_GBS * 1e9)
    hbm_bound = float(np.mean(ai)) < ridge
    tot_t = sweep_avg / 1e3
    if hbm_bound:
        achieved = sum(bytes_mode) / tot_t / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = d * flops_mode / tot_t / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS[dt_name],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS[dt_name], 4)}
    # The same fraction from the cold-cache medians (the tensor read from HBM
    # rather than from the last-level cache it fits in between modes).
    if cold is not None:
        t_cold = sum(cold_med) / 1e3
        if hbm_bound:
            roof["frac_cold"] = round(sum(bytes_mode) / t_cold / 1e9 / HBM_PEAK_GBS, 4)
        else:
            roof["frac_cold"] = round(d * flops_mode / t_cold / 1e12 / PEAK_TFLOPS[dt_name], 4)
    tr = measured_traffic(p.name)
    roof["traffic"] = (round(float(np.mean(tr["bytes_per_mode"])), 0) if tr else None)
    roof["traffic_unit"] = "bytes/launch (FETCH_SIZE+WRITE_SIZE, copy-calibrated)"
    # the plain cache model's bounds per mode: T_inf moves every byte once,
    # T_0 re-reads the d - 1 factor rows for every tensor element (no reuse)
    t_inf = [max(flops_mode / peak_f, bytes_mode[n] / (HBM_PEAK_GBS * 1e9)) * 1e3 for n in range(d)]
    t_0 = [max(flops_mode / peak_f, s * (N + (d - 1) * N * R) / (HBM_PEAK_GBS * 1e9)) * 1e3
           for n in range(d)]
    roof["model_ms_per_mode"] = {"t_inf": [round(v, 5) for v in t_inf],
                                 "t_0": [round(v, 5) for v in t_0]}
    roof["per_launch_ms"] = round(sweep_avg / d, 5)
    roof["sweep_ms"] = round(sweep_avg, 5)
    roof["algorithmic_bytes_per_launch"] = bytes_mode
    roof["flops_per_launch"] = flops_mode

    # ---- CPU oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu:
        import oracle
        cores = len(os.sched_getaffinity(0))
        nthreads = min(cores, 16)
        done_flops = 0.0
        t_cpu = 0.0
        rows_done = [0] * d
        budget = args.cpu_seconds
        chunk = max(1, nthreads)
        while t_cpu < budget:
            progressed = False
            for n in range(d):
                if rows_done[n] >= dims[n] or t_cpu >= budget:
                    continue
                rr = list(range(rows_done[n], min(dims[n], rows_done[n] + chunk)))
                a = time.perf_counter()
                oracle.mttkrp(p.X, p.factors, n, rows=rr, nthreads=nthreads)
                t_cpu += time.perf_counter() - a
                done_flops += flops_mode * len(rr) / dims[n]
                rows_done[n] += len(rr)
                progressed = True
            if not progressed:
                break
        cpu = {"value": round(done_flops / t_cpu / 1e9, 4), "unit": "GFLOP/s", "cores": nthreads,
               "kind": "oracle",
               "sample": f"output rows {rows_done} of modes 0..{d - 1} "
                         f"({t_cpu:.1f} s; long-double oracle, OpenMP over rows)"}
        log(f"[bench] cpu oracle {cpu}")

    # ---- CP-ALS (the workload that is a CP-ALS run): time per iteration of the
    # whole driver (per mode: MTTKRP, Hadamard of Grams, Cholesky, row
    # solves, normalization, Gram refresh; then the fit, one read-back), and
    # the share of it that the per-mode MTTKRP launches take ----
    als = None
    if (p.als_iters or args.als_iters) and not args.no_als:
        iters = args.als_iters or 10
        ws_als = torch.empty(api.cp_als_workspace_bytes(dims, R, X.dtype), dtype=torch.uint8,
                             device=dev)
        U0 = [u.clone() for u in U]
        Ua = [u.clone() for u in U0]
        api.cp_als(X, Ua, iters=min(2, iters), ws=ws_als, stream=stream)  # warm-up
        torch.cuda.synchronize()
        Ua = [u.clone() for u in U0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        _, hist, done, st = api.cp_als(X, Ua, iters=iters, ws=ws_als, stream=stream)
        torch.cuda.synchronize()
        t_als = (time.perf_counter() - t0) / max(1, done)
        # the same iterations' MTTKRP launches alone, mode after mode on one
        # stream as the driver issues them
        ev_c = torch.cuda.Event(enable_timing=True)
        ev_d = torch.cuda.Event(enable_timing=True)
        ev_c.record(stream)
        for _ in range(iters):
            for n in range(d):
                api.mttkrp(X, Ua, n, out=outs[n], ws=ws, stream=stream)
        ev_d.record(stream)
        torch.cuda.synchronize()
        t_mt = ev_c.elapsed_time(ev_d) / 1e3 / iters
        als = {"ms_per_iter": round(t_als * 1e3, 4), "iters": int(done), "status": int(st),
               "final_fit": round(float(hist[done - 1]), 6) if done else None,
               "mttkrp_ms_per_iter": round(t_mt * 1e3, 4),
               "mttkrp_share": round(t_mt / t_als, 3)}

    # ---- the matrix-based comparison (explicit Khatri-Rao matrix, unfolded
    # X, vendor GEMM): time per mode with its extra memory, and its largest
    # difference from this library's outputs ----
    gemm = None
    if not args.no_gemm_baseline:
        ms, kr_b, cp_b, diff = [], [], [], 0.0
        parts = {"khatri_rao_ms": [], "unfold_ms": [], "gemm_ms": []}
        for n in range(d):
            explicit_kr_mttkrp(X, U, n)  # warm-up (library handles, allocations)
            torch.cuda.synchronize()
            reps = 3
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            t_parts = [0.0, 0.0, 0.0]
            for _ in range(reps):
                ev[0].record(stream)
                K = khatri_rao(U, [m for m in range(d) if m != n])
                ev[1].record(stream)
                Xn = unfold(X, n)
                ev[2].record(stream)
                Mn = torch.matmul(Xn, K)
                ev[3].record(stream)
                torch.cuda.synchronize()
                for i in range(3):
                    t_parts[i] += ev[i].elapsed_time(ev[i + 1]) / reps
            for key, v in zip(parts, t_parts):
                parts[key].append(round(v, 4))
            ms.append(sum(t_parts))
            kr_b.append(K.numel() * K.element_size())
            cp_b.append(0 if n in (0, d - 1) else Xn.numel() * Xn.element_size())
            del K, Xn
            api.mttkrp(X, U, n, out=outs[n], ws=ws, stream=stream)
            torch.cuda.synchronize()
            ref = outs[n].double()
            diff = max(diff, float((Mn.double() - ref).norm() / ref.norm().clamp_min(1e-300)))
            del Mn
        torch.cuda.empty_cache()
        gemm = {"kind": "explicit Khatri-Rao + torch.matmul (vendor GEMM)",
                "ms_per_mode": [round(v, 4) for v in ms], **parts,
                "gflops_all_mode": round(d * flops_mode / (sum(ms) / 1e3) / 1e9, 2),
                "khatri_rao_bytes_per_mode": kr_b, "unfold_copy_bytes_per_mode": cp_b,
                "library_workspace_bytes": ws_bytes,
                "rel_diff_vs_library": diff}
        log(f"[bench] explicit-KR GEMM baseline {gemm}")

    # ---- the untiled matrix-free baselines (one thread per element with
    # atomics; one workgroup per slice), where they finish in seconds ----
    ablation = None
    if not args.no_ablation:
        if N * R > (1 << 31):
            ablation = {"skipped": f"N * R = {N * R} products per mode is past the 2^31 bound"}
        else:
            ablation = {}
            for kind in ("elem", "slice"):
                ms_k, diff = [], 0.0
                for n in range(d):
                    Mk = api.mttkrp_ablation(X, U, n, kind, stream=stream)  # warm-up
                    a = torch.cuda.Event(enable_timing=True)
                    b = torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    api.mttkrp_ablation(X, U, n, kind, out=Mk, stream=stream)
                    b.record(stream)
                    torch.cuda.synchronize()
                    ms_k.append(a.elapsed_time(b))
                    api.mttkrp(X, U, n, out=outs[n], ws=ws, stream=stream)
                    torch.cuda.synchronize()
                    ref = outs[n].double()
                    diff = max(diff, float((Mk.double() - ref).norm() / ref.norm().clamp_min(1e-300)))
                ablation[kind] = {"ms_per_mode": [round(v, 4) for v in ms_k],
                                  "gflops_all_mode": round(d * flops_mode / (sum(ms_k) / 1e3) / 1e9, 2),
                                  "rel_diff_vs_library": diff}
        log(f"[bench] ablation baselines {ablation}")

    cfg = {"workload": p.name, "dims": list(dims), "rank": R, "modes": list(range(d)),
           "step": "all-mode MTTKRP sweep", "cache": "warm (back-to-back sweeps)"}
    line = {
        "metric": "MTTKRP GFLOP/s (all-mode avg) and % of HBM/FP64 roofline, 1 MI355X",
        "value": round(value, 2),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "preheat": {"seconds": PREHEAT_S, "sweeps": n_pre},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_name,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "cold_cache": cold,
        "cpu_baseline": cpu,
        "cp_als": als,
        "gemm_baseline": gemm,
        "ablation": ablation,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
