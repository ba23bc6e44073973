// Launch of one MTTKRP mode: the tile kernel selected for the plan, then the
// fixed-order reduction of the split partials when the plan has more than one.
#include <hip/hip_runtime.h>

#include <mutex>

#include "plan.hpp"
#include "tile_select.hpp"

namespace mttkrp {

// Fixed-order sum of the split partials: out[i] = sum_{s=0}^{S-1} partial[s][i].
// A workgroup covers EW consecutive outputs with 256/EW thread groups; group g
// sums the partials s = g, g + 256/EW, ... and the group sums are added in
// the order g = 0, 1, ..., so the result does not depend on scheduling.
template <typename T, int EW>
__global__ __launch_bounds__(256) void split_reduce_kernel(const double *__restrict__ partial,
                                                           int64_t nsplit, int64_t count,
                                                           void *out, int out64)
{
    constexpr int NG = 256 / EW;
    __shared__ double sh[NG][EW];
    const int c = threadIdx.x % EW;
    const int g = threadIdx.x / EW;
    const int64_t i = (int64_t)blockIdx.x * EW + c;
    // Eight partials are loaded before any is added (one memory round trip per
    // eight, not per partial); out-of-range ones read as zero.
    double v = 0.0;
    if (i < count) {
        for (int64_t s0 = g; s0 < nsplit; s0 += 8 * NG) {
            double t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int64_t s = s0 + (int64_t)u * NG;
                t[u] = s < nsplit ? partial[s * count + i] : 0.0;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) v += t[u];
        }
    }
    sh[g][c] = v;
    __syncthreads();
    if (g == 0 && i < count) {
        double t = sh[0][c];
        for (int j = 1; j < NG; ++j) t += sh[j][c];
        if (out64)
            reinterpret_cast<double *>(out)[i] = t;
        else
            reinterpret_cast<T *>(out)[i] = (T)t;
    }
}

// Trailing-rows reduction: out(i, r) = sum_s sum_j U_red(j, r) partial[s][row(i, j)][r]
// with row(i, j) = i * inner + j (output = the outer row mode) or j * inner + i
// (output = the inner one).  A workgroup covers EW consecutive outputs with
// 256/EW thread groups striding over s (j ascending inside); the group sums
// are added in order, so the result is independent of scheduling.
template <typename T, int EW>
__global__ __launch_bounds__(256) void trailing_reduce_kernel(const double *__restrict__ partial,
                                                              KParams p)
{
    constexpr int NG = 256 / EW;
    __shared__ double sh[NG][EW];
    const int c = threadIdx.x % EW;
    const int g = threadIdx.x / EW;
    const int64_t R = p.R;
    const int64_t o = (int64_t)blockIdx.x * EW + c;
    const int64_t count = p.In_out * R;
    const T *U = reinterpret_cast<const T *>(p.Ured);
    double v = 0.0;
    if (o < count) {
        const int64_t i = o / R;
        const int64_t r = o - i * R;
        // Eight (factor, partial) pairs are loaded before any is used.
        for (int64_t s = g; s < p.nsplit; s += NG) {
            const double *P = partial + s * p.In * R;
            for (int64_t j0 = 0; j0 < p.tr_J; j0 += 8) {
                double u[8], w[8];
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int64_t j = j0 + t;
                    const bool ok = j < p.tr_J;
                    const int64_t jj = ok ? j : 0;
                    const int64_t row = p.tr_div ? i * p.tr_inner + jj : jj * p.tr_inner + i;
                    u[t] = ok ? (double)U[jj * R + r] : 0.0;
                    w[t] = ok ? P[row * R + r] : 0.0;
                }
#pragma unroll
                for (int t = 0; t < 8; ++t) v += u[t] * w[t];
            }
        }
    }
    sh[g][c] = v;
    __syncthreads();
    if (g == 0 && o < count) {
        double t = sh[0][c];
        for (int j = 1; j < NG; ++j) t += sh[j][c];
        if (p.out64)
            reinterpret_cast<double *>(p.out)[o] = t;
        else
            reinterpret_cast<T *>(p.out)[o] = (T)t;
    }
}

// gfx950 has 160 KB of LDS per compute unit; a kernel opts into dynamic sizes
// above 64 KB once per device (the limit is raised to the whole 160 KB, and
// each launch still asks only for what its plan needs).  Launches are often
// issued back to back from the host, so the opt-in is not repeated.
hipError_t allow_large_lds(const void *k)
{
    constexpr int kMaxDev = 64;
    constexpr int kMaxKernels = 256;
    static std::mutex mu;
    static const void *done[kMaxDev][kMaxKernels];
    static int ndone[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    const bool cache = dev >= 0 && dev < kMaxDev;
    if (cache)
        for (int j = 0; j < ndone[dev]; ++j)
            if (done[dev][j] == k) return hipSuccess;
    // the limit covers static and dynamic LDS together
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, k);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024 - (int)fa.sharedSizeBytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();  // leave no sticky error for the caller's next call
        return e;
    }
    if (cache && ndone[dev] < kMaxKernels) done[dev][ndone[dev]++] = k;
    return e;
}

template <typename T>
TileKernel select_kernel(const Plan &pl);
template <>
TileKernel select_kernel<double>(const Plan &pl)
{
    if (pl.layout == 1) return select_tile_f64_rows(pl);
    return pl.form ? select_tile_f64_form1(pl) : select_tile_f64_form0(pl);
}
template <>
TileKernel select_kernel<float>(const Plan &pl)
{
    if (pl.layout == 1) return select_tile_f32_rows(pl);
    return pl.form ? select_tile_f32_form1(pl) : select_tile_f32_form0(pl);
}

bool plan_launchable(const Plan &pl)
{
    return pl.elem_bytes == 8 ? select_kernel<double>(pl) != nullptr
                              : select_kernel<float>(pl) != nullptr;
}

// with_reduce = false leaves a split plan's partials for a later launch to
// sum (the all-mode sweep hands them to the next mode's tile kernel).
template <typename T>
hipError_t launch_mttkrp(const Plan &pl, hipStream_t stream, bool with_reduce)
{
    TileKernel k = select_kernel<T>(pl);
    if (!k) return hipErrorInvalidConfiguration;
    if (pl.lds_bytes > 64 * 1024) {
        hipError_t a = allow_large_lds(reinterpret_cast<const void *>(k));
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)pl.grid), dim3(64 * pl.waves), pl.lds_bytes, stream, pl.kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pl.kp.tr) {
        const int64_t count = pl.kp.In_out * pl.kp.R;
        // Few outputs (a short output mode): four per workgroup, so that the
        // grid still spans the chip.
        if (count < 16 * 1024) {
            hipLaunchKernelGGL((trailing_reduce_kernel<T, 4>), dim3((unsigned)((count + 3) / 4)),
                               dim3(256), 0, stream, (const double *)pl.kp.partial, pl.kp);
        } else if (pl.kp.nsplit >= 16) {
            hipLaunchKernelGGL((trailing_reduce_kernel<T, 16>), dim3((unsigned)((count + 15) / 16)),
                               dim3(256), 0, stream, (const double *)pl.kp.partial, pl.kp);
        } else {
            hipLaunchKernelGGL((trailing_reduce_kernel<T, 64>), dim3((unsigned)((count + 63) / 64)),
                               dim3(256), 0, stream, (const double *)pl.kp.partial, pl.kp);
        }
        e = hipGetLastError();
    } else if (pl.kp.nsplit > 1 && with_reduce) {
        const int64_t count = pl.kp.In * pl.kp.R;
        if (pl.kp.nsplit >= 32) {
            hipLaunchKernelGGL((split_reduce_kernel<T, 16>), dim3((unsigned)((count + 15) / 16)),
                               dim3(256), 0, stream, (const double *)pl.kp.partial, pl.kp.nsplit,
                               count, pl.kp.out, pl.kp.out64);
        } else {
            hipLaunchKernelGGL((split_reduce_kernel<T, 64>), dim3((unsigned)((count + 63) / 64)),
                               dim3(256), 0, stream, (const double *)pl.kp.partial, pl.kp.nsplit,
                               count, pl.kp.out, pl.kp.out64);
        }
        e = hipGetLastError();
    }
    return e;
}

// Two form-1 modes in one launch, one pass each (plans checked by fusable():
// same B tile and decomposition, no partials).  The reduction
// space follows the B tile in LDS.
template <typename T>
hipError_t launch_mttkrp_multi(const Plan *const *pls, int np, hipStream_t stream)
{
    if (np != kMaxPasses) return hipErrorInvalidValue;
    const Plan &pl = *pls[0];
    MultiKernel k = sizeof(T) == 8 ? select_multi_f64(pl) : select_multi_f32(pl);
    if (!k) return hipErrorInvalidConfiguration;
    KPack pk{};
    for (int i = 0; i < np; ++i) pk.p[i] = pls[i]->kp;
    const size_t b_tile = (size_t)pl.kp.Kc * pl.kp.bpitch * sizeof(T);
    pk.red_off = (int64_t)((b_tile + 15) / 16 * 16);
    const size_t lds = (size_t)pk.red_off + (size_t)pl.waves * 16 * pl.nb * sizeof(double);
    if (lds > 160 * 1024) return hipErrorInvalidConfiguration;
    if (lds > 64 * 1024) {
        hipError_t a = allow_large_lds(reinterpret_cast<const void *>(k));
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)pl.grid), dim3(64 * pl.waves), lds, stream, pk);
    return hipGetLastError();
}

template hipError_t launch_mttkrp<double>(const Plan &, hipStream_t, bool);
template hipError_t launch_mttkrp<float>(const Plan &, hipStream_t, bool);
template hipError_t launch_mttkrp_multi<double>(const Plan *const *, int, hipStream_t);
template hipError_t launch_mttkrp_multi<float>(const Plan *const *, int, hipStream_t);

}  // namespace mttkrp
