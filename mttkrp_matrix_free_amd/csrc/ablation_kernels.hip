// Ablation baselines ("A Performance Portable Matrix Free Dense MTTKRP in
// GenTen": the MTTKRP-ELEM and MTTKRP-SLICE strategies that precede its
// cache-aware tiled one).  Both are matrix-free but untiled: no staged
// Khatri-Rao tile, no matrix cores.  They are comparison baselines, not the
// product path.
//   ELEM:  one thread per tensor element; its product with the other factors'
//          rows is added to the output row with one atomic per column (the
//          order of the additions is not fixed).
//   SLICE: one workgroup per output row (a slice of X); a thread takes one
//          column and every G-th element of the slice; the G partial sums of
//          a column are added in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/mttkrp.h"

namespace mttkrp {
namespace {

struct AblDesc {
    const void *U[5];
    int64_t dims[5];
    int64_t stride[5];  // element strides of X
    int order, mode;
    int64_t R, N;
};

template <typename T>
__global__ __launch_bounds__(256) void abl_fill_kernel(T *p, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = T(0);
}

template <typename T>
__global__ __launch_bounds__(256) void elem_kernel(const T *__restrict__ X, AblDesc d,
                                                   T *__restrict__ out)
{
    for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < d.N;
         e += (int64_t)gridDim.x * 256) {
        int64_t idx[5];
        int64_t rem = e;
        for (int m = d.order - 1; m >= 0; --m) {
            idx[m] = rem % d.dims[m];
            rem /= d.dims[m];
        }
        const T x = X[e];
        T *o = out + idx[d.mode] * d.R;
        for (int64_t r = 0; r < d.R; ++r) {
            T p = x;
            for (int m = 0; m < d.order; ++m)
                if (m != d.mode) p *= reinterpret_cast<const T *>(d.U[m])[idx[m] * d.R + r];
            atomicAdd(o + r, p);
        }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void slice_kernel(const T *__restrict__ X, AblDesc d,
                                                    T *__restrict__ out)
{
    __shared__ T red[256];
    const int64_t in = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t slice = d.N / d.dims[d.mode];
    const int RC = d.R < 256 ? (int)d.R : 256;
    const int G = 256 / RC;
    for (int64_t r0 = 0; r0 < d.R; r0 += RC) {
        const int64_t r = r0 + t % RC;
        const int g = t / RC;
        const bool active = g < G && r < d.R;
        T acc = T(0);
        if (active) {
            for (int64_t j = g; j < slice; j += G) {
                // the other modes' indices of the slice's j-th element (last fastest)
                int64_t rem = j, off = in * d.stride[d.mode];
                T p = T(1);
                for (int m = d.order - 1; m >= 0; --m) {
                    if (m == d.mode) continue;
                    const int64_t im = rem % d.dims[m];
                    rem /= d.dims[m];
                    off += im * d.stride[m];
                    p *= reinterpret_cast<const T *>(d.U[m])[im * d.R + r];
                }
                acc += X[off] * p;
            }
        }
        red[t] = acc;
        __syncthreads();
        if (g == 0 && active) {
            T s = red[t];
            for (int h = 1; h < G; ++h) s += red[h * RC + t];
            out[in * d.R + r] = s;
        }
        __syncthreads();
    }
}

template <typename T>
int run_ablation(bool elem, const T *X, const int64_t *dims, int order, const T *const *factors,
                 int64_t rank, int mode, T *out, void *stream_)
{
    if (!X || !dims || !factors || !out) return MTTKRP_EINVAL;
    if (order < 3 || order > 5) return MTTKRP_EORDER;
    if (rank < 1 || mode < 0 || mode >= order) return MTTKRP_EINVAL;
    AblDesc d{};
    d.order = order;
    d.mode = mode;
    d.R = rank;
    d.N = 1;
    for (int m = 0; m < order; ++m) {
        if (dims[m] < 1) return MTTKRP_EINVAL;
        if (m != mode && !factors[m]) return MTTKRP_EINVAL;
        d.dims[m] = dims[m];
        d.U[m] = m != mode ? factors[m] : nullptr;
        if (d.N > INT64_MAX / dims[m]) return MTTKRP_ERANGE;
        d.N *= dims[m];
    }
    if (d.N > INT64_MAX / rank) return MTTKRP_ERANGE;
    int64_t st = 1;
    for (int m = order - 1; m >= 0; --m) {
        d.stride[m] = st;
        st *= dims[m];
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream_);
    if (elem) {
        const int64_t n = dims[mode] * rank;
        hipLaunchKernelGGL(abl_fill_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           out, n);
        const int64_t blocks = std::min<int64_t>((d.N + 255) / 256, 256 * 64);
        hipLaunchKernelGGL(elem_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, X, d, out);
    } else {
        if (dims[mode] > INT32_MAX) return MTTKRP_ERANGE;
        hipLaunchKernelGGL(slice_kernel<T>, dim3((unsigned)dims[mode]), dim3(256), 0, s, X, d, out);
    }
    return hipGetLastError() == hipSuccess ? MTTKRP_OK : MTTKRP_EHIP;
}

}  // namespace
}  // namespace mttkrp

using namespace mttkrp;

extern "C" {

int mttkrp_elem_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
                    int64_t rank, int mode, double *out, void *stream)
{
    return run_ablation<double>(true, X, dims, order, factors, rank, mode, out, stream);
}
int mttkrp_elem_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                    int64_t rank, int mode, float *out, void *stream)
{
    return run_ablation<float>(true, X, dims, order, factors, rank, mode, out, stream);
}
int mttkrp_slice_f64(const double *X, const int64_t *dims, int order,
                     const double *const *factors, int64_t rank, int mode, double *out,
                     void *stream)
{
    return run_ablation<double>(false, X, dims, order, factors, rank, mode, out, stream);
}
int mttkrp_slice_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                     int64_t rank, int mode, float *out, void *stream)
{
    return run_ablation<float>(false, X, dims, order, factors, rank, mode, out, stream);
}

}  // extern "C"
