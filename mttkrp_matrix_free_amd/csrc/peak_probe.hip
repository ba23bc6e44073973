// Measurement probes: the achievable HBM read rate and matrix-core rate of
// the device, the denominators reported beside the published peaks.
//
//   peak_read_kernel   streams a buffer once with 16-byte loads, four loads in
//                      flight per thread, and folds every word into a 32-bit
//                      checksum (so no load can be dropped and the result can
//                      be checked on the host);
//   peak_mfma_kernel   runs chains of independent 16x16x4 MFMAs (eight
//                      accumulators per wave, two waves per SIMD) on register
//                      operands: no memory traffic, no dependency stalls.
//
// Neither is part of the MTTKRP; they only time the hardware.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/mttkrp.h"

namespace mttkrp {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef double dx4 __attribute__((ext_vector_type(4)));
typedef float fx4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 4;

// Word sum of x ^ y ^ z ^ w over every 16-byte group, modulo 2^32, per
// workgroup.
__global__ __launch_bounds__(kReadThreads) void peak_read_kernel(const u32x4 *__restrict__ p,
                                                                  int64_t n16, uint32_t *sink)
{
    __shared__ uint32_t sh[kReadThreads];
    const int64_t stride = (int64_t)gridDim.x * kReadThreads;
    int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc += v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const u32x4 v = p[i];
        acc += v.x ^ v.y ^ v.z ^ v.w;
    }
    sh[threadIdx.x] = acc;
    __syncthreads();
    for (int h = kReadThreads / 2; h > 0; h /= 2) {
        if ((int)threadIdx.x < h) sh[threadIdx.x] += sh[threadIdx.x + h];
        __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = sh[0];
}

// ITERS rounds of eight independent MFMAs per wave; the accumulators' sum of
// lane 0 goes to sink[workgroup * 4 + wave].
template <typename T>
struct ProbeMfma;
template <>
struct ProbeMfma<double> {
    typedef dx4 acc_t;
    static __device__ __forceinline__ acc_t mma(double a, double b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
};
template <>
struct ProbeMfma<float> {
    typedef fx4 acc_t;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename T>
__global__ __launch_bounds__(256, 2) void peak_mfma_kernel(int64_t iters, double *sink)
{
    typedef typename ProbeMfma<T>::acc_t acc_t;
    constexpr int NA = 8;
    const int lane = threadIdx.x & 63;
    // operands of order 1e-3 keep eight million accumulations far from overflow
    const T a = (T)(1e-3 * (1 + (lane & 7)));
    const T b = (T)(1e-3 * (1 + (lane >> 3)));
    acc_t acc[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) acc[j] = acc_t{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] = ProbeMfma<T>::mma(a, b, acc[j]);
    }
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < NA; ++j) s += (double)acc[j][0] + (double)acc[j][1] + (double)acc[j][2] + (double)acc[j][3];
    if (lane == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace mttkrp

using namespace mttkrp;

extern "C" {

int mttkrp_probe_read_grid(void) { return 8 * 256; }

int mttkrp_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream)
{
    if (!buf || !sink) return MTTKRP_EINVAL;
    if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 15u))
        return MTTKRP_EALIGN;
    if (bytes % 16 != 0) return MTTKRP_EINVAL;
    hipLaunchKernelGGL(peak_read_kernel, dim3(mttkrp_probe_read_grid()), dim3(kReadThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4 *>(buf),
                       (int64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? MTTKRP_OK : MTTKRP_EHIP;
}

int mttkrp_probe_mfma_grid(void) { return 2 * 256; }

int mttkrp_probe_mfma(int elem_bytes, int64_t iters, double *sink, void *stream)
{
    if (!sink || iters < 1) return MTTKRP_EINVAL;
    if (reinterpret_cast<uintptr_t>(sink) & 15u) return MTTKRP_EALIGN;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (elem_bytes == 8)
        hipLaunchKernelGGL(peak_mfma_kernel<double>, dim3(mttkrp_probe_mfma_grid()), dim3(256), 0, s,
                           iters, sink);
    else if (elem_bytes == 4)
        hipLaunchKernelGGL(peak_mfma_kernel<float>, dim3(mttkrp_probe_mfma_grid()), dim3(256), 0, s,
                           iters, sink);
    else
        return MTTKRP_EINVAL;
    return hipGetLastError() == hipSuccess ? MTTKRP_OK : MTTKRP_EHIP;
}

}  // extern "C"
