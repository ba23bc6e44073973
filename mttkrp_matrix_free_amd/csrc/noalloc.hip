// The single-mode MTTKRP without any allocation (mttkrp_noalloc): the split
// partial sums go to a fixed scratch array in device memory instead of a
// caller's workspace.  The array is a file-scope device variable, so each GPU
// the library runs on holds its own copy from module load until the process
// ends; its device address is looked up once per device, on the entry
// point's first call there, and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mttkrp.h"

namespace mttkrp {

int check_mode_call(const void *X, const int64_t *dims, int order, const void *const *factors,
                    int64_t rank, int mode, const void *out);

namespace {

constexpr size_t kScratchBytes = MTTKRP_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDev = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's scratch array (looked up once per device,
// with that device current).
hipError_t scratch_address(void **out)
{
    static std::mutex mu;
    static void *addr[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

}  // namespace
}  // namespace mttkrp

extern "C" int mttkrp_noalloc(const void *X, const int64_t *dims, int order,
                              const void *const *factors, int64_t rank, int mode, void *out,
                              int elem_bytes, void *stream)
{
    using namespace mttkrp;
    if (elem_bytes != 8 && elem_bytes != 4) return MTTKRP_EINVAL;
    int st = check_mode_call(X, dims, order, factors, rank, mode, out);
    if (st) return st;
    size_t need = 0;
    st = mttkrp_workspace_bytes(dims, order, rank, mode, elem_bytes, &need);
    if (st) return st;
    if (need > kScratchBytes) return MTTKRP_ESCRATCH;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return MTTKRP_EHIP;
    if (elem_bytes == 8)
        return mttkrp_f64(static_cast<const double *>(X), dims, order,
                          reinterpret_cast<const double *const *>(factors), rank, mode,
                          static_cast<double *>(out), ws, kScratchBytes, stream);
    return mttkrp_f32(static_cast<const float *>(X), dims, order,
                      reinterpret_cast<const float *const *>(factors), rank, mode,
                      static_cast<float *>(out), ws, kScratchBytes, stream);
}
