// CP-ALS kernels around the MTTKRP ("A Performance Portable Matrix Free Dense
// MTTKRP in GenTen", Fig. 5: besides MTTKRP, each step needs inner products
// and a Cholesky solve).  All R x R work is done in fp64 whatever the tensor
// element type; every reduction runs in a fixed order (deterministic).
//
// Per mode n of a sweep:
//   als_chol:      V = Hadamard_{m != n} G_m, then V = L L^T (no pivoting);
//                  a non-positive pivot raises the failure flag.
//   (MTTKRP of mode n into the fp64 buffer M)
//   als_solve:     U_new(i, :) = M(i, :) V^{-1} by a forward and a back
//                  substitution per row.
//   als_normalize: lambda_r = ||U_new(:, r)||_2, U_n = U_new / lambda (columns
//                  with lambda_r = 0 kept as they are).
//   gram:          G_n = U_n^T U_n.
// After the last mode, als_fit forms
//   fit = 1 - sqrt(max(0, ||X||^2 + ||model||^2 - 2 <X, model>)) / ||X||
// with <X, model> = sum_r lambda_r sum_i M(i, r) U_{d-1}(i, r) and
// ||model||^2 = sum_{a,b} lambda_a lambda_b prod_m G_m(a, b).
// Every kernel after a failed Cholesky (flag 1) returns without writing, so
// the factors keep the values of the failing step's start; the same holds
// after a converged sweep (flag 2, set by als_fit), so sweeps queued ahead of
// the host's check change nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>
#include <utility>

#include "als_kernels.hpp"

namespace mttkrp {

constexpr int kRedThreads = 256;

__device__ __forceinline__ double block_sum(double v, double *sh)
{
    // Fixed-order tree: wave butterfly, then wave results in index order.
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) sh[wave] = v;
    __syncthreads();
    double t = 0.0;
    const int nw = (blockDim.x + 63) >> 6;
    for (int w = 0; w < nw; ++w) t += sh[w];
    return t;
}

// The failure word as one value for the whole workgroup: thread 0 loads it
// and the others take its value from LDS, so a write by a kernel running
// beside this one cannot send the waves down different paths.
__device__ __forceinline__ int flag_once(const int *flag, int *sh)
{
    if (threadIdx.x == 0)
        *sh = __hip_atomic_load(const_cast<int *>(flag), __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    return *sh;
}

// Ordering of the split mode update's two streams without events.  A kernel
// waits (one thread, bounded) until a sequence word written by the kernel it
// depends on reaches a value, and when done stores its own value to another
// word.  The host only ever makes a kernel wait for one queued before it, so
// however the two streams map onto hardware queues the awaited kernel runs
// first or beside the waiting one.  Past about 10 s of the 100 MHz constant
// clock the wait gives up: the failure word becomes 3 and the kernel does no
// work but still stores its word, so no waiter is left behind.
struct SeqArgs {
    const unsigned *wait_on;  // word to wait for (null: no wait)
    unsigned wait_for;        // value it must reach (compared with wrap-around)
    unsigned *done;           // word to store when finished (null: none)
    unsigned done_val;
};
constexpr long long kSeqWaitTicks = 1000000000LL;

__device__ __noinline__ bool seq_wait_thread(const unsigned *p, unsigned target)
{
    if (!p) return true;
    const long long t0 = wall_clock64();
    for (;;) {
        const unsigned v = __hip_atomic_load(const_cast<unsigned *>(p), __ATOMIC_ACQUIRE,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if ((int)(v - target) >= 0) return true;
        if (wall_clock64() - t0 > kSeqWaitTicks) return false;
        __builtin_amdgcn_s_sleep(2);
    }
}

// Whole workgroup: wait, then every thread acquires, so what the awaited
// kernel wrote before its word is visible to each of them.  Returns the
// failure word read after the wait (one value for the workgroup).
__device__ __forceinline__ int seq_enter(const SeqArgs &q, int *flag, int *sh)
{
    if (threadIdx.x == 0) {
        int f;
        if (seq_wait_thread(q.wait_on, q.wait_for)) {
            f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            atomicCAS(flag, 0, 3);
            f = 3;
        }
        *sh = f;
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    return *sh;
}

// Whole workgroup: every thread releases its writes, then thread 0 stores the
// word.
__device__ __forceinline__ void seq_leave(const SeqArgs &q)
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0 && q.done)
        __hip_atomic_store(q.done, q.done_val, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// The end of a sweep: the fit, the stop decision and the host-visible slot.
// A sweep whose fit changed by less than tol (tol > 0, a previous sweep's fit
// in scal[2]) sets the failure word to 2, so every later kernel of the run
// returns without writing, just as after a failed Cholesky (1).  The slot
// receives the fit and the word, then the sweep's number (a release at
// system scope): the host polls that number while the next sweep is
// already queued, so the device never waits for the host.
struct FitArgs {
    const double *V;     // (split update) the Hadamard product of the other Grams
    const double *Gall;  // the Grams of every mode, this sweep's last included
    int order;
    double *scal;        // [0] ||X||^2 in, [1] fit out, [2] the previous fit
    double tol;
    int have_prev;
    double *out_fit;     // host-visible slot
    int *out_flag;
    unsigned *out_seq;
    unsigned seq_val;
};

// Thread 0, given <X, model> and ||model||^2.
__device__ __forceinline__ void fit_finish(double inner, double nrm2, int *flag, const FitArgs &fa)
{
    const double nx2 = fa.scal[0];
    double resid = nx2 + nrm2 - 2.0 * inner;
    if (resid < 0.0) resid = 0.0;
    const double fit = nx2 > 0.0 ? 1.0 - sqrt(resid) / sqrt(nx2) : __builtin_nan("");
    const int stop = fa.tol > 0.0 && fa.have_prev && fabs(fit - fa.scal[2]) < fa.tol;
    fa.scal[1] = fit;
    fa.scal[2] = fit;
    if (stop) atomicCAS(flag, 0, 2);
    *fa.out_fit = fit;
    *fa.out_flag = stop ? 2 : 0;
    __hip_atomic_store(fa.out_seq, fa.seq_val, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Thread 0 of a sweep whose kernels found the failure word set: the word and
// the sweep's number go to the slot (the fit is not written).
__device__ __forceinline__ void fit_skip(int f, const FitArgs &fa)
{
    *fa.out_flag = f;
    __hip_atomic_store(fa.out_seq, fa.seq_val, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ||model||^2 = sum_{a,b} lambda_a lambda_b prod_m G_m(a, b): eight entries
// per thread and round, every load of a round in flight at once; each thread
// adds its entries in index order (the workgroup sum follows).
__device__ __forceinline__ double model_norm_part(const double *__restrict__ lam,
                                                  const double *__restrict__ Gall, int order,
                                                  int64_t R)
{
    const int64_t RR = R * R;
    double nrm2 = 0.0;
    constexpr int Q = 8;
    for (int64_t e0 = threadIdx.x; e0 < RR; e0 += (int64_t)blockDim.x * Q) {
        double v[Q];
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            int64_t e = e0 + (int64_t)blockDim.x * q;
            e = e < RR ? e : RR - 1;
            const int64_t a = e / R, b = e - (e / R) * R;
            v[q] = lam[a] * lam[b];
        }
        // modes past the order multiply by 1 (exact), so no load waits on a branch
#pragma unroll
        for (int m = 0; m < 5; ++m) {
            const bool use = m < order;
            const double *Gm = Gall + (use ? (int64_t)m * RR : 0);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int64_t e = e0 + (int64_t)blockDim.x * q;
                const double g = Gm[e < RR ? e : RR - 1];
                v[q] *= use ? g : 1.0;
            }
        }
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (e0 + (int64_t)blockDim.x * q < RR) nrm2 += v[q];
    }
    return nrm2;
}

// ||X||^2, first pass: one fp64 partial per workgroup (grid-stride, fixed order).
template <typename T>
__global__ __launch_bounds__(kRedThreads) void sumsq_partial_kernel(const T *__restrict__ X,
                                                                    int64_t N,
                                                                    double *__restrict__ partial)
{
    __shared__ double sh[kRedThreads / 64];
    double s = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; i < N;
         i += (int64_t)gridDim.x * kRedThreads) {
        const double x = (double)X[i];
        s += x * x;
    }
    s = block_sum(s, sh);
    if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

__global__ __launch_bounds__(kRedThreads) void sum_final_kernel(const double *__restrict__ partial,
                                                                int n, double *__restrict__ out)
{
    __shared__ double sh[kRedThreads / 64];
    double s = 0.0;
    for (int i = threadIdx.x; i < n; i += kRedThreads) s += partial[i];
    s = block_sum(s, sh);
    if (threadIdx.x == 0) *out = s;
}

// G = U^T U (R x R, fp64) of an I x R factor; one thread per entry.
template <typename T>
__global__ __launch_bounds__(256) void gram_kernel(const T *__restrict__ U, int64_t I, int64_t R,
                                                   double *__restrict__ G,
                                                   const int *__restrict__ flag)
{
    if (flag && *flag) return;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= R * R) return;
    const int64_t a = e / R, b = e - (e / R) * R;
    double s = 0.0;
    for (int64_t i = 0; i < I; ++i) s += (double)U[i * R + a] * (double)U[i * R + b];
    G[e] = s;
}

// The Grams of every mode at the start of a run (R <= 64), in one launch:
// blockIdx.y is the mode, a thread one entry summed over i in increasing
// order (as gram_kernel), with eight rows' loads in flight at once.
struct GramAllArgs {
    const void *U[5];
    int64_t I[5];
};

template <typename T>
__global__ __launch_bounds__(256) void gram_all_kernel(GramAllArgs g, int64_t R,
                                                       double *__restrict__ G,
                                                       const int *__restrict__ flag)
{
    if (*flag) return;  // (no barrier follows)
    const int m = blockIdx.y;
    const T *__restrict__ U = static_cast<const T *>(g.U[m]);
    const int64_t I = g.I[m];
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= R * R) return;
    const int64_t a = e / R, b = e - (e / R) * R;
    double s = 0.0;
    for (int64_t i0 = 0; i0 < I; i0 += 8) {
        double ua[8], ub[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int64_t i = i0 + t < I ? i0 + t : I - 1;
            ua[t] = (double)U[i * R + a];
            ub[t] = (double)U[i * R + b];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
            if (i0 + t < I) s += ua[t] * ub[t];
    }
    G[(int64_t)m * R * R + e] = s;
}

// Lane read of a double (the lane index is wave-uniform).
__device__ __forceinline__ double lane_read(double v, int l)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(u >> 32), l);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One step of the one-wave factorization below with a frame of W registers
// (columns j .. j + W - 1; every column past the frame is past R - 1).
// Publishes this lane's entry l of column j (to the column buffer c and to
// its places L1 and L2 in the outputs), applies the column to the frame,
// shifting it by one, and returns the next column's entry in l.
template <int W, int RM>
__device__ __forceinline__ void chol_wave_step(double (&a)[RM], double &l, bool &bad, int i, int j,
                                               int R, double *__restrict__ c,
                                               double *__restrict__ L1, double *__restrict__ L2)
{
    c[i] = l;
    const double lo = i >= j ? l : 0.0;
    *L1 = lo;
    *L2 = lo;
    // the wave's LDS operations are performed in issue order, so the reads
    // below see every lane's entry
    __builtin_amdgcn_wave_barrier();
    double cv[W];
#pragma unroll
    for (int k = 1; k < W - 1; ++k) cv[k] = c[j + 1 + k];
    // the next pivot's path: the one entry it needs comes by lane read
    const int jn = j + 1;
    const double t0 = __builtin_fma(-l, lane_read(l, jn & 63), a[1]);
    const double piv = lane_read(t0, jn & 63);
    bad = bad || (jn < R && !(piv > 0.0));
    const double d = sqrt(piv);
    const double ln = i == jn ? d : t0 / d;
    a[0] = t0;
#pragma unroll
    for (int k = 1; k < W - 1; ++k) a[k] = __builtin_fma(-l, cv[k], a[k + 1]);
    a[W - 1] = 0.0;
    l = ln;
}

// V = Hadamard_{m != n} G_m into A (R x R, pitch P; all threads of the
// workgroup take part, every load of a thread in flight at once).  Factors
// are multiplied in mode order; a skipped mode multiplies by 1 (exact).
template <int RM, int NT>
__device__ __forceinline__ void hadamard_to_lds(const double *__restrict__ Gall, int order, int n,
                                                int R, double *__restrict__ A, int P)
{
    constexpr int EPT = (RM * RM + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int RR = R * R;
    double v[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) v[q] = 1.0;
#pragma unroll
    for (int m = 0; m < 5; ++m) {
        const bool use = m < order && m != n;
        const double *Gm = Gall + (use ? (int64_t)m * RR : 0);
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int e = tid + NT * q;
            const double g = Gm[e < RR ? e : 0];
            v[q] *= use ? g : 1.0;
        }
    }
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = tid + NT * q;
        if (e < RR) {
            const int r = e / R;
            A[r * P + (e - r * R)] = v[q];
        }
    }
}

// The factorization of V (in A, pitch RM + 1, R <= RM <= 64) by one wave
// (called by the whole first wave).  Lane i keeps row i of the trailing
// matrix in registers, in a frame that moves one column per step (at step j
// register k holds column j + k), so the trailing update is a fixed,
// unrolled set of fused multiply-adds whose destinations carry the shift;
// the frame narrows in steps of 16 as the trailing matrix shrinks.  The
// finished column goes through LDS (col, 256 entries, zero on entry), where
// every lane reads its entries with broadcast reads, all issued before the
// first is used.  The next column's pivot, square root and divisions come
// from the first updated register before the rest of the update, so their
// latency overlaps it.  Every entry of L receives the operations of the
// textbook column-by-column factorization,
//   L_jj = sqrt(V_jj - sum_{k<j} L_jk^2),  L_ij = (V_ij - sum_{k<j} L_ik L_jk) / L_jj,
// with the subtractions applied one at a time in the order k = 0, 1, ...;
// entries above the diagonal take throwaway updates and are written as zeros.  L_ij goes
// to out1[i * s1r + j * s1c] and out2[i * s2r + j * s2c]; rows past R - 1
// write to spare.  Returns (in every lane) whether a pivot was not positive.
template <int RM>
__device__ __forceinline__ bool chol_wave_factor(const double *__restrict__ A, int R,
                                                 double *__restrict__ col,
                                                 double *__restrict__ out1, int s1r, int s1c,
                                                 double *__restrict__ out2, int s2r, int s2c,
                                                 double *__restrict__ spare)
{
    constexpr int P = RM + 1;
    const int i = threadIdx.x & 63;
    const bool row = i < R;
    double a[RM];
#pragma unroll
    for (int k = 0; k < RM; ++k) a[k] = row && k < R ? A[(row ? i : 0) * P + k] : 0.0;
    const double piv = lane_read(a[0], 0);
    bool bad = !(piv > 0.0);
    const double d = sqrt(piv);
    double l = i == 0 ? d : a[0] / d;  // this lane's entry of column j
    double *const b1 = row ? out1 + i * s1r : spare;
    double *const b2 = row ? out2 + i * s2r : spare;
    const int c1 = row ? s1c : 0, c2 = row ? s2c : 0;
    int j = 0;
    if constexpr (RM >= 64)
        for (; j < R - 48; ++j)
            chol_wave_step<64>(a, l, bad, i, j, R, col + (j & 1) * 128, b1 + j * c1, b2 + j * c2);
    if constexpr (RM >= 48)
        for (; j < R - 32; ++j)
            chol_wave_step<48>(a, l, bad, i, j, R, col + (j & 1) * 128, b1 + j * c1, b2 + j * c2);
    if constexpr (RM >= 32)
        for (; j < R - 16; ++j)
            chol_wave_step<32>(a, l, bad, i, j, R, col + (j & 1) * 128, b1 + j * c1, b2 + j * c2);
    for (; j < R; ++j)
        chol_wave_step<16>(a, l, bad, i, j, R, col + (j & 1) * 128, b1 + j * c1, b2 + j * c2);
    return bad;
}

// The Cholesky factor alone (for modes the one-workgroup update below does
// not take), R <= RM <= 64: all four waves assemble V and copy L out, the
// first factors it.  One wave per SIMD: the factoring wave may use the whole
// register file.
template <int RM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
als_chol_wave_kernel(const double *__restrict__ Gall, int order, int n, int R,
                     double *__restrict__ Lout, int *__restrict__ flag)
{
    constexpr int P = RM + 1;
    struct Smem {
        double col[256];       // two column buffers
        double A[RM * P + 1];  // V, then L; the last entry takes writes of rows past R - 1
        int fail;
    };
    __shared__ Smem sm;
    if (*flag) return;
    const int tid = threadIdx.x;
    const int RR = R * R;
    hadamard_to_lds<RM, 256>(Gall, order, n, R, sm.A, P);
    sm.col[tid] = 0.0;
    __syncthreads();
    if (tid < 64) {
        // L overwrites V in place: a row's entries are read into registers
        // before any is written
        const bool bad = chol_wave_factor<RM>(sm.A, R, sm.col, sm.A, P, 1, sm.A, P, 1,
                                              sm.A + RM * P);
        if (tid == 0) sm.fail = bad;
    }
    __syncthreads();
    if (sm.fail) {
        if (tid == 0) *flag = 1;
        return;
    }
    for (int e = tid; e < RR; e += 256) {
        const int r = e / R;
        Lout[e] = sm.A[r * P + (e - r * R)];
    }
}

// Row solves (L L^T) x = m for every row of M; one wave per row, R <= 64:
// lane l holds component l.
__global__ __launch_bounds__(256) void als_solve_wave_kernel(const double *__restrict__ M,
                                                             const double *__restrict__ L,
                                                             int64_t I, int64_t R,
                                                             double *__restrict__ Unew,
                                                             const int *__restrict__ flag)
{
    if (*flag) return;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= I) return;
    double b = lane < R ? M[row * R + lane] : 0.0;
    // forward: L y = b
    for (int j = 0; j < (int)R; ++j) {
        const double xj = __shfl(b, j) / L[(int64_t)j * R + j];
        if (lane == j) b = xj;
        if (lane > j && lane < R) b -= L[(int64_t)lane * R + j] * xj;
    }
    // back: L^T x = y
    for (int j = (int)R - 1; j >= 0; --j) {
        const double xj = __shfl(b, j) / L[(int64_t)j * R + j];
        if (lane == j) b = xj;
        if (lane < j) b -= L[(int64_t)j * R + lane] * xj;
    }
    if (lane < R) Unew[row * R + lane] = b;
}

// lambda_r = ||U_new(:, r)||_2 and U_n = U_new / lambda_r.  A workgroup
// takes 16 columns; thread (c, g) sums the squares of rows g, g + 16, ... of
// column c in order, and the 16 group sums of a column are added in group
// order (a fixed order, so results do not depend on scheduling); then every
// thread scales its rows.
template <typename T>
__global__ __launch_bounds__(256) void als_normalize_kernel(const double *__restrict__ Unew,
                                                            int64_t I, int64_t R,
                                                            T *__restrict__ Uout,
                                                            double *__restrict__ lam64,
                                                            T *__restrict__ lamT,
                                                            const int *__restrict__ flag)
{
    __shared__ double part[16][17];
    __shared__ double lam_s[16];
    if (*flag) return;
    const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int64_t r = (int64_t)blockIdx.x * 16 + c;
    const bool ok = r < R;
    double s = 0.0;
    if (ok) {
#pragma unroll 4
        for (int64_t i = g; i < I; i += 16) s += Unew[i * R + r] * Unew[i * R + r];
    }
    part[g][c] = s;
    __syncthreads();
    if (g == 0) {
        double t = part[0][c];
        for (int h = 1; h < 16; ++h) t += part[h][c];
        const double lam = sqrt(t);
        lam_s[c] = lam;
        if (ok) {
            lam64[r] = lam;
            if (lamT) lamT[r] = (T)lam;
        }
    }
    __syncthreads();
    if (!ok) return;
    const double lam = lam_s[c];
#pragma unroll 4
    for (int64_t i = g; i < I; i += 16) {
        const double v = Unew[i * R + r];
        Uout[i * R + r] = (T)(lam > 0.0 ? v / lam : v);
    }
}

// Quad-local lane moves (DPP quad permutations): the value of lane 0 of this
// lane's group of four, and the value of the next lane of the group (lane 3
// gets its own).
__device__ __forceinline__ double quad_first(double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, 0x00, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(u >> 32), 0x00, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double quad_next(double v)
{
    constexpr int kNext = 1 | (2 << 2) | (3 << 4) | (3 << 6);
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, kNext, 0xf, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(u >> 32), kNext, 0xf, 0xf, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Substitution frames split over groups of four lanes: lane 4 r + q holds
// quarter q of row r's frame (16 rows per wave).  With quarter width w,
// register t of quarter q holds component j + S (q w + t) (S = +1 forward,
// -1 back).

// One step: x = (component j) / L_jj from quarter 0, handed to the group;
// every quarter takes x times its L entries cv[t] (entries for offsets
// q w + 1 + t) off its components, shifting by one, the top register taking
// the next quarter's first component.  Quarter 0 of a valid row stores x.
// The next step's reciprocal and entries (rdn, en) are read before this
// step's arithmetic.
template <int w, int S, int RQ>
__device__ __forceinline__ void subst_step4(double (&a)[RQ], double (&cv)[RQ], double &rdj,
                                            const double *__restrict__ rdn,
                                            const double *__restrict__ en,
                                            double *__restrict__ xj, int q)
{
    double cn[w];
#pragma unroll
    for (int t = 0; t < w; ++t) cn[t] = en[S * t];
    const double rn = *rdn;
    const double x = quad_first(a[0] * rdj);
    *xj = x;
    const double up = quad_next(a[0]);
    const double nxt = q == 3 ? 0.0 : up;
#pragma unroll
    for (int t = 0; t < w - 1; ++t) a[t] = __builtin_fma(-cv[t], x, a[t + 1]);
    a[w - 1] = __builtin_fma(-cv[w - 1], x, nxt);
#pragma unroll
    for (int t = 0; t < w; ++t) cv[t] = cn[t];
    rdj = rn;
}

// Moves a frame from quarter width wf to wt (the frame narrows by 16
// components) through the row's own LDS storage: every in-range component is
// written at its place, then read back in the new layout.
template <int wf, int wt, int S, int RQ>
__device__ __forceinline__ void restage4(double (&a)[RQ], double *__restrict__ xrow, int j, int R,
                                         bool ok, int q)
{
    if (wf > 0) {
#pragma unroll
        for (int t = 0; t < wf; ++t) {
            const int c = j + S * (q * wf + t);
            if (ok && c >= 0 && c < R) xrow[c] = a[t];
        }
    }
    // the wave's LDS operations are performed in issue order
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int t = 0; t < wt; ++t) {
        const int c = j + S * (q * wt + t);
        a[t] = ok && c >= 0 && c < R ? xrow[c] : 0.0;
    }
#pragma unroll
    for (int t = wt; t < RQ; ++t) a[t] = 0.0;
}

// One substitution pass (S = +1: L y = m from the row in xrow; S = -1:
// L^T u = y) over rows of 4 lanes, the frame narrowing from 64 to 16
// components as the unsolved part shrinks.  E: L^T rows forward, L rows back
// (with 64 zero entries past the end the pass reads).
template <int S, int RQ>
__device__ __forceinline__ void subst_pass4(double *__restrict__ xrow, double *__restrict__ xout,
                                            int xs, const double *__restrict__ E,
                                            const double *__restrict__ rd, int R, bool ok, int q)
{
    double a[RQ], cv[RQ];
    int j = S > 0 ? 0 : R - 1;
    int w = 0;  // current quarter width (0: nothing loaded yet)
    double rdj = 0.0;
    // this step's operands (on entry to a segment) and the next step's
    // (inside it; the index is clamped at the ends)
    auto ent = [&](int jj, int ww) { return E + jj * R + jj + S * (q * ww + 1); };
    auto nj = [&]() { const int t = j + S; return t < 0 ? 0 : (t >= R ? R - 1 : t); };
    auto enter = [&](auto wc) {
        constexpr int ww = decltype(wc)::value;
        const double *e = ent(j, ww);
#pragma unroll
        for (int t = 0; t < ww; ++t) cv[t] = e[S * t];
        rdj = rd[j];
    };
    if constexpr (RQ >= 16)
        if (R > 48) {
            restage4<0, 16, S>(a, xrow, j, R, ok, q);
            enter(std::integral_constant<int, 16>());
            w = 16;
#pragma unroll 2
            for (; S > 0 ? j < R - 48 : j >= 48; j += S)
                subst_step4<16, S>(a, cv, rdj, rd + nj(), ent(nj(), 16), xout + j * xs, q);
            restage4<16, 12, S>(a, xrow, j, R, ok, q);
            w = 12;
        }
    if constexpr (RQ >= 16)
        if (R > 32) {
            if (w == 0) restage4<0, 12, S>(a, xrow, j, R, ok, q);
            enter(std::integral_constant<int, 12>());
#pragma unroll 2
            for (; S > 0 ? j < R - 32 : j >= 32; j += S)
                subst_step4<12, S>(a, cv, rdj, rd + nj(), ent(nj(), 12), xout + j * xs, q);
            restage4<12, 8, S>(a, xrow, j, R, ok, q);
            w = 8;
        }
    if constexpr (RQ >= 8)
        if (R > 16) {
            if (w == 0) restage4<0, 8, S>(a, xrow, j, R, ok, q);
            enter(std::integral_constant<int, 8>());
#pragma unroll 2
            for (; S > 0 ? j < R - 16 : j >= 16; j += S)
                subst_step4<8, S>(a, cv, rdj, rd + nj(), ent(nj(), 8), xout + j * xs, q);
            restage4<8, 4, S>(a, xrow, j, R, ok, q);
            w = 4;
        }
    if (w == 0) restage4<0, 4, S>(a, xrow, j, R, ok, q);
    enter(std::integral_constant<int, 4>());
#pragma unroll 2
    for (; S > 0 ? j < R : j >= 0; j += S)
        subst_step4<4, S>(a, cv, rdj, rd + nj(), ent(nj(), 4), xout + j * xs, q);
}

// A whole mode step after its MTTKRP in one workgroup (four waves, one per
// SIMD), for R <= RM <= 64 and a mode whose solution, L and L^T fit in LDS
// together: V and its Cholesky factor (as in als_chol_wave_kernel), then the
// solve, normalization and Gram refresh, with the arithmetic of
// als_solve_wave_kernel, als_normalize_kernel and gram_kernel in the same
// order, except that the substitutions multiply by the reciprocals of L's
// diagonal instead of dividing by it (results within a rounding of the
// divisions).
//  - Substitutions: a lane per row (64 rows per wave and pass), the row's
//    unknowns in registers in a frame that shifts by one per step and narrows
//    in steps of 16 as the unsolved part shrinks; L's entries of a step are
//    the same for every row and come from LDS as broadcast reads (L^T rows
//    for the forward pass, L rows backward, zero padding past both ends).
//    There is no exchange between lanes, so the only serial chain per step
//    is one product and one fused multiply-add.
//  - Normalization: a thread per column forms the norm (rows in order); then
//    every thread scales a share of the entries.
//  - Gram: a thread per 4 x 4 block of entries (rows in order).
// A non-positive pivot sets the flag to 1 and writes nothing else.
template <typename T, int RM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
als_update_small_kernel(const double *__restrict__ Gall, int order, int n,
                        const double *__restrict__ M, int64_t I64, int64_t R64,
                        T *__restrict__ Uout, double *__restrict__ lam64,
                        T *__restrict__ lamT, double *__restrict__ G, int *__restrict__ flag)
{
    extern __shared__ __align__(16) unsigned char smem[];
    if (*flag) return;
    const int I = (int)I64, R = (int)R64;  // R <= RM, sizes checked by the host
    const int RR = R * R;
    constexpr int PV = RM + 1;  // pitch of V
    double *col = reinterpret_cast<double *>(smem);      // 256: factorization's column buffers
    double *Lr = col + 256 + 64;                         // L, rows; 64 zeros before
    double *Lt = Lr + RR;                                // L^T, rows; 64 zeros after
    double *x = Lt + RR + 64;                            // V (pitch PV), then the I x R solution, then U
    const int nx = RM * PV > I * R ? RM * PV : I * R;
    double *rd = x + nx;                                 // 1 / L_jj, then lambda
    double *spare = rd + 64;                             // writes of rows past the end
    int &fail = *reinterpret_cast<int *>(spare + 1);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    hadamard_to_lds<RM, 256>(Gall, order, n, R, x, PV);
    col[tid] = 0.0;
    if (tid < 64) {
        Lr[tid - 64] = 0.0;
        Lt[RR + tid] = 0.0;
    }
    __syncthreads();
    if (tid < 64) {
        const bool bad = chol_wave_factor<RM>(x, R, col, Lr, R, 1, Lt, 1, R, spare);
        if (tid == 0) fail = bad;
    }
    __syncthreads();
    if (fail) {
        if (tid == 0) *flag = 1;
        return;
    }
    if (tid < R) rd[tid] = 1.0 / Lr[tid * R + tid];
    __syncthreads();
    {
        const int q = lane & 3;  // quarter of the row's frame this lane holds
        constexpr int RQ = RM / 4;
        for (int r0 = 16 * wave; r0 < I; r0 += 64) {
            const int row = r0 + (lane >> 2);
            const bool ok = row < I;
            double *xrow = x + (size_t)(ok ? row : 0) * R;
            // quarter 0 of a valid row stores the unknowns; other lanes the
            // spare entry
            const bool st = ok && q == 0;
            double *xout = st ? xrow : spare;
            const int xs = st ? 1 : 0;
            // the row of M into its LDS storage, a quarter per block
#pragma unroll
            for (int t = 0; t < RQ; ++t) {
                const int c = q * RQ + t;
                if (ok && c < R) xrow[c] = M[(size_t)row * R + c];
            }
            subst_pass4<1, RQ>(xrow, xout, xs, Lt, rd, R, ok, q);
            __builtin_amdgcn_wave_barrier();
            subst_pass4<-1, RQ>(xrow, xout, xs, Lr, rd, R, ok, q);
        }
    }
    __syncthreads();
    // column norms (rows in order), then the normalized factor; the LDS copy
    // keeps the stored (element-type) values for the Gram below
    if (tid < R) {
        double sq = 0.0;
        for (int i = 0; i < I; ++i) sq += x[i * R + tid] * x[i * R + tid];
        const double lam = sqrt(sq);
        rd[tid] = lam;
        lam64[tid] = lam;
        if (lamT) lamT[tid] = (T)lam;
    }
    __syncthreads();
    for (int e = tid; e < I * R; e += 256) {
        const double lam = rd[e - (e / R) * R];
        const T u = (T)(lam > 0.0 ? x[e] / lam : x[e]);
        Uout[e] = u;
        x[e] = (double)u;
    }
    __syncthreads();
    // G = U^T U: a thread takes a 4 x 4 block of entries (each summed over i
    // in order), so a pair of LDS reads feeds four products
    const int nb4 = (R + 3) / 4;
    for (int blk = tid; blk < nb4 * nb4; blk += 256) {
        const int a0 = (blk / nb4) * 4, c0 = (blk - (blk / nb4) * nb4) * 4;
        double g[4][4] = {};
#pragma unroll 4
        for (int i = 0; i < I; ++i) {
            double ua[4], uc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ua[t] = a0 + t < R ? x[i * R + a0 + t] : 0.0;
                uc[t] = c0 + t < R ? x[i * R + c0 + t] : 0.0;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int u = 0; u < 4; ++u) g[t][u] += ua[t] * uc[u];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (a0 + t < R && c0 + u < R) G[(a0 + t) * R + c0 + u] = g[t][u];
    }
}

// The mode update split in two, for R <= RM <= 64 and a mode whose I x R
// solution fits in LDS (the same sizes as the one-workgroup update above):
//
//  - als_side_chol_kernel (on a second stream, beside the mode's MTTKRP,
//    which it does not need): V = Hadamard of the other Grams, V = L L^T (the
//    one-wave factorization above), W = L^{-1} and V^{-1} = W^T W.  It is launched with eight workgroups, of which the
//    first to be dispatched does the work, so it runs wherever a compute
//    unit is free.
//  - als_apply_small_kernel (after the MTTKRP, on the caller's stream):
//    U_new = M V^{-1}, then the column norms, the normalized factor and its
//    Gram as in the one-workgroup update.
//
// W = L^{-1} column by column (a lane per column c): forward substitution of
// the unit vector e_c, w_j = b_j / L_jj and b_i -= L_ij w_j for i > j, with
// the updates of an entry applied in the order j = 0, 1, ....  Lane c keeps
// the unsolved part of its column in registers, in a frame that moves one
// entry per step (at step j register k holds entry j + k) and narrows in
// steps of 16 as the unsolved part shrinks, so the update is a fixed set of
// fused multiply-adds whose destinations carry the shift (a loop per frame
// width: the code stays small).  L's column j comes from LDS as broadcast
// reads of L^T's row j (RM zeros after the last row).
template <int W, int RM>
__device__ __forceinline__ void inv_step(double (&b)[RM], int j, int R, int c,
                                         const double *__restrict__ Lt,
                                         const double *__restrict__ rd, double *__restrict__ Wout,
                                         int wp)
{
    double lv[W];
#pragma unroll
    for (int k = 1; k < W; ++k) lv[k] = Lt[j * R + j + k];
    const double x = b[0] * rd[j];
    if (c < R) Wout[j * wp + c] = x;
#pragma unroll
    for (int k = 1; k < W; ++k) b[k - 1] = __builtin_fma(-lv[k], x, b[k]);
    b[W - 1] = 0.0;  // entries past the frame are past R - 1
}

template <int RM>
__device__ __forceinline__ void tri_inverse_wave(const double *__restrict__ Lt,
                                                 const double *__restrict__ rd, int R,
                                                 double *__restrict__ Wout, int wp)
{
    const int c = threadIdx.x & 63;
    double b[RM];
#pragma unroll
    for (int k = 0; k < RM; ++k) b[k] = (k == c && c < R) ? 1.0 : 0.0;
    int j = 0;
    if constexpr (RM >= 64)
        for (; j < R - 48; ++j) inv_step<64>(b, j, R, c, Lt, rd, Wout, wp);
    if constexpr (RM >= 48)
        for (; j < R - 32; ++j) inv_step<48>(b, j, R, c, Lt, rd, Wout, wp);
    if constexpr (RM >= 32)
        for (; j < R - 16; ++j) inv_step<32>(b, j, R, c, Lt, rd, Wout, wp);
    for (; j < R; ++j) inv_step<16>(b, j, R, c, Lt, rd, Wout, wp);
}

// Dense products of 4 x 4 blocks with every sum over an index in increasing
// order: G(a, c) += sum_i x(i, a) x(i, c) over rows i of x (pitch given),
// for V^{-1} = W^T W in the side kernel and the Gram in the apply kernel.
__device__ __forceinline__ void gram4_accumulate(const double *__restrict__ x, int pitch, int rows,
                                                 int a0, int c0, double (&g)[4][4])
{
#pragma unroll 4
    for (int i = 0; i < rows; ++i) {
        double ua[4], uc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ua[t] = x[i * pitch + a0 + t];
            uc[t] = x[i * pitch + c0 + t];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int u = 0; u < 4; ++u) g[t][u] += ua[t] * uc[u];
    }
}

// Dynamic LDS of the side kernel: the column buffers and the failure word,
// then V (then L, in place, pitch RM + 1, one spare entry), L^T rows with RM
// zeros after, 1 / L_jj and W (pitch RM + 1).
template <int RM>
constexpr size_t side_chol_lds()
{
    return (size_t)(256 + 1 + (RM * (RM + 1) + 1) + (RM * RM + RM) + RM + RM * (RM + 1)) *
           sizeof(double);
}
template <int RM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
als_side_chol_kernel(const double *__restrict__ Gall, int order, int n, int R,
                     double *__restrict__ Vinv, double *__restrict__ Vout,
                     int *__restrict__ flag, unsigned *__restrict__ ticket, SeqArgs q)
{
    constexpr int P = RM + 1;
    extern __shared__ __align__(16) unsigned char smem[];
    double *col = reinterpret_cast<double *>(smem);  // 256
    int &fail = *reinterpret_cast<int *>(col + 256);
    double *A = col + 257;                           // RM x P (+ 1 spare)
    double *Lt = A + RM * P + 1;                     // RM x RM, RM zeros after
    double *rd = Lt + RM * RM + RM;                  // RM
    double *Wl = rd + RM;                            // RM x P
    const int tid = threadIdx.x;
    // Eight workgroups take a ticket each (one vector atomic per workgroup);
    // the first to run does the work, so it runs on whichever XCD had a
    // compute unit free.  Every launch takes exactly eight tickets and the
    // counter starts at zero, so the first ticket of a launch is 0 mod 8.
    if (tid == 0) fail = (int)(atomicAdd(ticket, 1u) & 7u);
    __syncthreads();
    if (fail != 0) return;
    __syncthreads();  // every thread has read the ticket before fail is reused
    // the previous mode's update (or the previous sweep's end)
    if (seq_enter(q, flag, &fail) == 0) {
        constexpr int nb4 = RM / 4;
        const int a0 = (tid / nb4) * 4, c0 = (tid - (tid / nb4) * nb4) * 4;
        const bool own = tid < nb4 * nb4;  // a thread per 4 x 4 block
        hadamard_to_lds<RM, 256>(Gall, order, n, R, A, P);
        col[tid] = 0.0;
        if (tid < RM) Lt[R * R + tid] = 0.0;
        for (int e = tid; e < RM * P; e += 256) Wl[e] = 0.0;
        __syncthreads();
        if (Vout)  // V itself, for the fit (before L overwrites it)
            for (int e = tid; e < R * R; e += 256) Vout[e] = A[(e / R) * P + e - (e / R) * R];
        if (tid < 64) {
            // L overwrites V in place (a row's entries are read into
            // registers before any is written), and its transpose goes to Lt
            const bool bad = chol_wave_factor<RM>(A, R, col, A, P, 1, Lt, 1, R, A + RM * P);
            if (tid == 0) fail = bad;
        }
        __syncthreads();
        if (fail) {
            if (tid == 0) atomicCAS(flag, 0, 1);
        } else {
            if (tid < R) rd[tid] = 1.0 / A[tid * P + tid];
            __syncthreads();
            if (tid < 64) tri_inverse_wave<RM>(Lt, rd, R, Wl, P);
            __syncthreads();
            // V^{-1}(a, c) = sum_k W(k, a) W(k, c), k increasing (W's zero
            // upper triangle adds exact zeros)
            if (own) {
                double g[4][4] = {};
                gram4_accumulate(Wl, P, RM, a0, c0, g);
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (a0 + t < R && c0 + u < R) Vinv[(a0 + t) * R + c0 + u] = g[t][u];
            }
        }
    }
    seq_leave(q);
}

// Dynamic LDS of the apply kernel for I x R (0: not usable): V^{-1} (RM rows
// of RM + 1), M and U (each I rounded up to 16 rows of RM + 1), lambda and
// its reciprocals.
size_t apply_small_lds(int64_t I, int64_t R)
{
    if (R > 64 || I > (1 << 20)) return 0;
    const int64_t rm = R <= 16 ? 16 : R <= 32 ? 32 : 64;
    const int64_t i16 = (I + 15) / 16 * 16;
    const size_t b = (size_t)(rm * (rm + 1) + 2 * i16 * (rm + 1) + 128) * sizeof(double);
    return b <= 150 * 1024 ? b : 0;
}

typedef double adx4 __attribute__((ext_vector_type(4)));

// U = M V^{-1} and the Gram on the fp64 matrix cores (v_mfma_f64_16x16x4f64:
// lane (r, q) = (lane % 16, lane / 16) supplies A(r, k + q) and B(k + q, r);
// element e of the result holds row 4 e + q, column r).  The raw Gram
// U^T U gives the column norms (its diagonal), so no serial pass over the
// rows is needed; the Gram of the normalized factor is the raw one scaled by
// 1 / (lambda_a lambda_c).  A zero column keeps its values (scale 1).
template <typename T, int RM>
__device__ __forceinline__ void apply_small_body(const double *__restrict__ M, int64_t I64,
                                                 int64_t R64, const double *__restrict__ Vinv,
                                                 T *__restrict__ Uout, double *__restrict__ lam64,
                                                 T *__restrict__ lamT, double *__restrict__ G,
                                                 int *__restrict__ flag, const FitArgs &fa)
{
    extern __shared__ __align__(16) unsigned char smem[];
    const int I = (int)I64, R = (int)R64;
    // row pitches RM + 1: the sixteen rows a matrix-core operand reads fall on
    // distinct banks
    constexpr int PW = RM + 1, XP = RM + 1;
    constexpr int CT = RM / 16;  // 16-column tiles
    const int I16 = (I + 15) / 16 * 16;
    double *W = reinterpret_cast<double *>(smem);  // V^{-1}: RM x PW, zero past R
    double *x = W + RM * PW;                         // M: I16 x XP, zero past I and R
    double *y = x + I16 * XP;                        // U: I16 x XP
    double *lam = y + I16 * XP;                      // 64, then 64 reciprocals
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r16 = lane & 15, q = lane >> 4;
    // V^{-1} and M into LDS: a thread's loads of a batch are all in flight
    // before any is stored, and M's first batch goes out with V^{-1}'s (one
    // memory round trip for both when M fits in it)
    {
        constexpr int NW = (RM * PW + 255) / 256;
        double v[NW], m[16];
#pragma unroll
        for (int t = 0; t < NW; ++t) {
            const int e = tid + 256 * t;
            const int j = e / PW, c = e - (e / PW) * PW;
            const bool in = e < RM * PW && j < R && c < R;
            v[t] = Vinv[in ? j * R + c : 0];
            v[t] = in ? v[t] : 0.0;
        }
        for (int e0 = 0; e0 < I16 * RM; e0 += 256 * 16) {
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int e = e0 + tid + 256 * t;
                const int i = e / RM, c = e - (e / RM) * RM;
                const bool in = i < I && c < R;
                m[t] = M[in ? i * R + c : 0];
                m[t] = in ? m[t] : 0.0;
            }
            if (e0 == 0) {
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    const int e = tid + 256 * t;
                    if (e < RM * PW) W[e] = v[t];
                }
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int e = e0 + tid + 256 * t;
                const int i = e / RM, c = e - (e / RM) * RM;
                if (e < I16 * RM) x[i * XP + c] = m[t];
            }
        }
    }
    __syncthreads();
    // U(i, c) = sum_k M(i, k) V^{-1}(k, c): 16 x 16 tiles, four to a wave at a
    // time, their matrix-core chains interleaved and each step's operands
    // read before its products
    const int ntile = (I16 / 16) * CT;
    for (int t0 = wave; t0 < ntile; t0 += 16) {
        adx4 acc[4];
        int xo[4], wo[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc[u] = adx4{0.0, 0.0, 0.0, 0.0};
            const int t = t0 + 4 * u < ntile ? t0 + 4 * u : t0;  // (spare tiles redo t0)
            const int rt = t / CT, ct = t - (t / CT) * CT;
            xo[u] = (rt * 16 + r16) * XP + q;
            wo[u] = q * PW + ct * 16 + r16;
        }
#pragma unroll
        for (int kk = 0; kk < RM; kk += 4) {
            double av[4], bv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                av[u] = x[xo[u] + kk];
                bv[u] = W[wo[u] + kk * PW];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[u], bv[u], acc[u], 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + 4 * u;
            if (t < ntile) {
                const int rt = t / CT, ct = t - (t / CT) * CT;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[(rt * 16 + 4 * e + q) * XP + ct * 16 + r16] = acc[u][e];
            }
        }
    }
    __syncthreads();
    // the raw Gram U^T U (rows past I are zero): CT x CT tiles, a wave's
    // tiles interleaved the same way
    constexpr int NG = CT * CT, GPW = (NG + 3) / 4;
    adx4 g[GPW];
    int ga[GPW], gc[GPW];
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        g[j] = adx4{0.0, 0.0, 0.0, 0.0};
        const int t = wave + 4 * j < NG ? wave + 4 * j : 0;
        ga[j] = (t / CT) * 16 + r16;
        gc[j] = (t - (t / CT) * CT) * 16 + r16;
    }
    for (int k0 = 0; k0 < I16; k0 += 16) {
#pragma unroll
        for (int kk = k0; kk < k0 + 16; kk += 4) {
            double av[GPW], bv[GPW];
#pragma unroll
            for (int j = 0; j < GPW; ++j) {
                av[j] = y[(kk + q) * XP + ga[j]];
                bv[j] = y[(kk + q) * XP + gc[j]];
            }
#pragma unroll
            for (int j = 0; j < GPW; ++j)
                g[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[j], bv[j], g[j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int t = wave + 4 * j;
        if (t < NG && t / CT == t - (t / CT) * CT)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (4 * e + q == r16) lam[(t / CT) * 16 + r16] = sqrt(g[j][e]);
    }
    __syncthreads();
    // 1 / lambda per column (1 for a zero column, which keeps its values)
    double *rlam = lam + 64;
    if (tid < RM) rlam[tid] = lam[tid] > 0.0 ? 1.0 / lam[tid] : 1.0;
    __syncthreads();
    if (tid < R) {
        lam64[tid] = lam[tid];
        if (lamT) lamT[tid] = (T)lam[tid];
    }
    // the normalized factor; the LDS copy keeps the stored (element-type)
    // values for the fit
    for (int e = tid; e < I * R; e += 256) {
        const int i = e / R, c = e - (e / R) * R;
        const T u = (T)(y[i * XP + c] * rlam[c]);
        Uout[e] = u;
        y[i * XP + c] = (double)u;
    }
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const int t = wave + 4 * j;
        if (t < NG) {
            const int at = t / CT, ct = t - (t / CT) * CT;
            const int c = ct * 16 + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = at * 16 + 4 * e + q;
                if (a < R && c < R) G[a * R + c] = g[j][e] * rlam[a] * rlam[c];
            }
        }
    }
    if (!fa.out_seq) return;
    // The sweep's last mode: its fit, from M (x), the stored factor (y) and
    // lambda, and ||model||^2 = sum_{a,c} lambda_a lambda_c V(a, c) G(a, c),
    // with V = the Hadamard product of the other modes' Grams (stored by this
    // mode's side kernel) and G this mode's Gram (still in the accumulators).
    __shared__ double sh[4];
    __syncthreads();
    double inner = 0.0;
    if (tid < R) {
        double sm = 0.0;
        for (int i = 0; i < I; ++i) sm += x[i * XP + tid] * y[i * XP + tid];
        inner = lam[tid] * sm;
    }
    inner = block_sum(inner, sh);
    double nrm2 = 0.0;
    {
        double vv[GPW][4];
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int t = wave + 4 * j < NG ? wave + 4 * j : 0;
            const int at = t / CT, ct = t - (t / CT) * CT;
            const int c = ct * 16 + r16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int a = at * 16 + 4 * e + q;
                vv[j][e] = fa.V[a < R && c < R ? a * R + c : 0];
            }
        }
#pragma unroll
        for (int j = 0; j < GPW; ++j) {
            const int t = wave + 4 * j;
            if (t < NG) {
                const int at = t / CT, ct = t - (t / CT) * CT;
                const int c = ct * 16 + r16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int a = at * 16 + 4 * e + q;
                    if (a < R && c < R)
                        nrm2 += lam[a] * lam[c] * vv[j][e] * (g[j][e] * rlam[a] * rlam[c]);
                }
            }
        }
    }
    nrm2 = block_sum(nrm2, sh);
    if (tid == 0) fit_finish(inner, nrm2, flag, fa);
}

// The apply waits for its mode's side kernel (V^{-1} and the failure word),
// and stores its word when done, for the next mode's side kernel.  With
// fa.out_seq set it also ends the sweep (the fit).
template <typename T, int RM>
__global__ __launch_bounds__(256) void als_apply_small_kernel(
    const double *__restrict__ M, int64_t I64, int64_t R64, const double *__restrict__ Vinv,
    T *__restrict__ Uout, double *__restrict__ lam64, T *__restrict__ lamT,
    double *__restrict__ G, int *__restrict__ flag, FitArgs fa, SeqArgs q)
{
    __shared__ int sflag;
    const int f = seq_enter(q, flag, &sflag);
    if (f == 0)
        apply_small_body<T, RM>(M, I64, R64, Vinv, Uout, lam64, lamT, G, flag, fa);
    else if (fa.out_seq && threadIdx.x == 0)
        fit_skip(f, fa);
    seq_leave(q);
}

template <typename T>
__global__ __launch_bounds__(256) void fill_kernel(T *__restrict__ p, int64_t n, T v)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Fit after the last mode of a sweep (when its update is not the split one,
// which forms the fit itself); one workgroup.
template <typename T>
__device__ __forceinline__ void fit_body(const double *__restrict__ M, const T *__restrict__ Ulast,
                                         int64_t Ilast, const double *__restrict__ lam64, int64_t R,
                                         int *__restrict__ flag, const double *__restrict__ mparts,
                                         int nmparts, const double *__restrict__ colsum,
                                         const FitArgs &fa)
{
    __shared__ double sh[kRedThreads / 64];
    double inner = 0.0;
    for (int64_t r = threadIdx.x; r < R; r += kRedThreads) {
        double s = 0.0;
        if (colsum)
            s = colsum[r];  // (large R: the same sums, formed by als_colsum_kernel)
        else
            for (int64_t i = 0; i < Ilast; ++i) s += M[i * R + r] * (double)Ulast[i * R + r];
        inner += lam64[r] * s;
    }
    inner = block_sum(inner, sh);
    double nrm2 = 0.0;
    if (nmparts > 0) {
        // (large R: the sum comes in partials from als_model_norm_kernel)
        for (int i = threadIdx.x; i < nmparts; i += kRedThreads) nrm2 += mparts[i];
    } else {
        nrm2 = model_norm_part(lam64, fa.Gall, fa.order, R);
    }
    nrm2 = block_sum(nrm2, sh);
    if (threadIdx.x == 0) fit_finish(inner, nrm2, flag, fa);
}

// The fit kernel stores its sequence word when done, for the next sweep's
// first side kernel (which then sees the stop decision).
template <typename T>
__global__ __launch_bounds__(kRedThreads) void als_fit_kernel(
    const double *__restrict__ M, const T *__restrict__ Ulast, int64_t Ilast,
    const double *__restrict__ lam64, int64_t R, int *__restrict__ flag,
    const double *__restrict__ mparts, int nmparts, const double *__restrict__ colsum, FitArgs fa,
    SeqArgs q)
{
    __shared__ int sflag;
    const int f0 = flag_once(flag, &sflag);
    if (f0) {
        if (threadIdx.x == 0) fit_skip(f0, fa);
    } else {
        fit_body<T>(M, Ulast, Ilast, lam64, R, flag, mparts, nmparts, colsum, fa);
    }
    seq_leave(q);
}

// ---------------------------------------------------------------------------
// Blocked R x R work for ranks past what one workgroup holds (R > 64): the
// Cholesky factorization in 64-wide column blocks, the diagonal blocks by
// one workgroup, carried out on V with the rows of M and of the
// identity appended, so that the forward substitution and the factor's
// inverse come out of the same block steps; the back substitution is then
// one product with that inverse.  Within a diagonal block every entry gets
// the textbook operations; across blocks the updates are summed per block
// (through the block's inverse) before they are applied, so the result
// differs from the one-entry-at-a-time order by rounding only.
// ---------------------------------------------------------------------------

// Set-up of the blocked update in one launch: entries e < R^2 form V =
// Hadamard_{m != n} G_m (modes in order) on and below the diagonal 64 x 64
// tiles (the tiles above are never read), the rest copy M into its working
// rows CM.
__global__ __launch_bounds__(256) void als_aug_setup_kernel(const double *__restrict__ Gall,
                                                            int order, int n, int64_t R,
                                                            double *__restrict__ CV,
                                                            const double *__restrict__ M,
                                                            double *__restrict__ CM, int64_t IR,
                                                            const int *__restrict__ flag)
{
    if (*flag) return;
    const int64_t RR = R * R;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e < RR) {
        const int64_t i = e / R, c = e - i * R;
        if ((c >> 6) > (i >> 6)) return;
        double v = 1.0;
        for (int m = 0; m < order; ++m)
            if (m != n) v *= Gall[(int64_t)m * RR + e];
        CV[e] = v;
    } else if (e - RR < IR) {
        CM[e - RR] = M[e - RR];
    }
}

// Pivot p = 16 pq + PP of the diagonal kernel below (PP a compile-time
// constant, so that the registers of column p, the LDS buffer and the next
// pivot's column are fixed at compile time; pq, the wave holding column p, is
// uniform).  Lane i holds row i of B (b) and of the identity rows (c) in the
// wave's 16 columns.
template <int PP>
__device__ __forceinline__ void chol_aug_pivot(double (&b)[16], double (&c)[16], bool &bad, int pq,
                                               int i, int wave, double (*colB)[64],
                                               double (*colI)[64])
{
    constexpr int buf = PP & 1, pn = (PP + 1) & 15;
    const int p = 16 * pq + PP;
    const int owner_next = pq + (PP == 15 ? 1 : 0);
    __syncthreads();
    const double d = colB[buf][p];
    double lp[16];  // B(j, p) = B(p, j) for this wave's columns (zero before p)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) lp[jj] = colB[buf][16 * wave + jj];
    const double ownb = colB[buf][i], ownc = colI[buf][i];
    bad = bad || !(d > 0.0);
    // 1 / sqrt(d) from the hardware estimate and two Newton steps
    // (y <- y + y (1 - d y^2) / 2), then 1 / d as its square
    double y = __builtin_amdgcn_rsq(d);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const double e = __builtin_fma(-d * y, y, 1.0);
        y = __builtin_fma(0.5 * y, e, y);
    }
    const double rd = y * y;
    const double tb = ownb * rd, tc = ownc * rd;
    // the next pivot's column first, so that its owner's LDS writes are on
    // their way while the other columns are updated
    b[pn] = __builtin_fma(-tb, lp[pn], b[pn]);
    c[pn] = __builtin_fma(-tc, lp[pn], c[pn]);
    if (p + 1 < 64 && wave == owner_next) {
        colB[buf ^ 1][i] = i >= p + 1 ? b[pn] : 0.0;
        colI[buf ^ 1][i] = c[pn];
    }
    // columns before p read zeros (finished); entry p of an identity row is
    // set below (B's entry p is not needed again)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
        if (jj != pn) {
            b[jj] = __builtin_fma(-tb, lp[jj], b[jj]);
            c[jj] = __builtin_fma(-tc, lp[jj], c[jj]);
        }
    if (wave == pq) c[PP] = ownc * y;
    // the pivot's updates are done here, not deferred to where the values are
    // next read (which would keep every pivot's operands live)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        asm volatile("" : "+v"(b[jj]));
        asm volatile("" : "+v"(c[jj]));
    }
}
template <int... PP>
__device__ __forceinline__ void chol_aug_pivots(std::integer_sequence<int, PP...>, double (&b)[16],
                                                double (&c)[16], bool &bad, int pq, int i,
                                                int wave, double (*colB)[64], double (*colI)[64])
{
    (chol_aug_pivot<PP>(b, c, bad, pq, i, wave, colB, colI), ...);
}

// The diagonal block B = A(k0 .. k0 + nb - 1, same columns) of A (R x R,
// row-major: the current Schur complement), nb = min(64, R - k0), at Ab with
// row stride lda (global memory, or LDS when the block step below runs it;
// 64 x 64 entries are read, so a block narrower than 64 comes padded with the
// identity's rows and columns, whose pivots are 1): its Cholesky factor's
// inverse transpose X = L_kk^{-T} to W rows k0 .. k0 + nb - 1 (pitch 64;
// zero in columns past nb) and Z = X X^T = B^{-1} to Z (64 x 64, pitch 64,
// zero outside nb x nb), so that the block step needs products only.  X is
// found as the rows of the identity appended below B and carried through
// B's right-looking factorization (their forward substitution), so one chain
// of 64 pivots gives both: pivot p with d = B(p, p) takes B(i, j) -=
// B(i, p) B(p, j) / d and C(i, j) -= C(i, p) B(p, j) / d for j > p, and sets
// C(i, p) to C(i, p) / sqrt(d).  Wave w holds columns 16 w .. 16 w + 15 of
// both B's row and the identity row of its lane; pivot p's column of each
// goes to every wave through LDS (two buffers, one barrier per pivot), so a
// lane reads 16 of B's entries per pivot.  A pivot that is not positive sets
// the flag to 1.  LDS: colB, colI (2 x 64 each), Xs (64 x 65, which may be
// the block's own LDS copy).
__device__ __forceinline__ void chol_diag_block(const double *Ab, int64_t lda, int nb, int64_t k0,
                                                double *__restrict__ W, double *__restrict__ Z,
                                                int *__restrict__ flag, double (*colB)[64],
                                                double (*colI)[64], double *Xs)
{
    const int i = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    double b[16], c[16];
    {
        const double *Ar = Ab + i * lda + 16 * wave;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
            b[jj] = Ar[jj];
            c[jj] = i == 16 * wave + jj ? 1.0 : 0.0;
        }
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
        asm volatile("" : "+v"(b[jj]));
        asm volatile("" : "+v"(c[jj]));
    }
    // pivot 0's column
    if (wave == 0) {
        colB[0][i] = b[0];
        colI[0][i] = c[0];
    }
    bool bad = false;
    for (int pq = 0; pq < 4; ++pq)
        chol_aug_pivots(std::make_integer_sequence<int, 16>(), b, c, bad, pq, i, wave, colB, colI);
    __syncthreads();  // (every wave is past its last read of Xs's memory)
    if (bad) {
        if (threadIdx.x == 0) *flag = 1;
        return;
    }
    {
        const bool rin = i < nb;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) Xs[i * 65 + 16 * wave + jj] = c[jj];
        if (rin) {
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) W[(k0 + i) * 64 + 16 * wave + jj] = c[jj];
        }
    }
    __syncthreads();
    // Z = X X^T on the matrix cores: wave w forms the 32 x 32 quarter at
    // (wr, wc) as 2 x 2 blocks of 16 x 16 (lane (r16, q) supplies A(r16, t + q)
    // and B(t + q, r16); element e of a block holds row 4 e + q).
    {
        const int r16 = i & 15, q = i >> 4;
        const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
        adx4 acc[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y) acc[x][y] = adx4{0.0, 0.0, 0.0, 0.0};
        for (int t0 = 0; t0 < nb; t0 += 4) {
            const int t = t0 + q;
            double av[2], bv[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = wr + 16 * x + r16;
                av[x] = (r < nb && t < nb) ? Xs[r * 65 + t] : 0.0;
                const int cc = wc + 16 * x + r16;
                bv[x] = (cc < nb && t < nb) ? Xs[cc * 65 + t] : 0.0;
            }
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < 2; ++y)
                    acc[x][y] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[x], bv[y], acc[x][y], 0, 0, 0);
        }
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Z[(wr + 16 * x + 4 * e + q) * 64 + wc + 16 * y + r16] = acc[x][y][e];
    }
}

__global__ __launch_bounds__(256) void als_chol_diag_kernel(const double *__restrict__ A,
                                                            int64_t R, int64_t k0,
                                                            double *__restrict__ W,
                                                            double *__restrict__ Z,
                                                            int *__restrict__ flag)
{
    __shared__ double colB[2][64];  // B(:, p), zero above the pivot
    __shared__ double colI[2][64];  // C(:, p) of the identity rows
    __shared__ double Xs[64 * 65];
    if (*flag) return;
    // (a whole 64-wide block: the caller launches it for R - k0 >= 64 only)
    chol_diag_block(A + k0 * R + k0, R, 64, k0, W, Z, flag, colB, colI, Xs);
}

// One block step k of the factorization V = L L^T carried out on the
// augmented rows [V; M; I] (V's own factor is never stored: its column blocks
// enter in product form through Z_k and W_k from the diagonal kernel).
//   trailing, every active row block i and column block j > k:
//       C(i, j) -= C(i, k) Z_k C_V(j, k)^T    (V rows: tiles j <= i only)
//   panel, the M rows and the identity rows:
//       Y(i, k) = C(i, k) W_k
// The identity rows' block b is active from step b on (column blocks before
// b of L^{-T} are zero); until then its entries are the identity's, so at
// step b they are formed rather than read (CI needs no set-up).  After the
// last step Y_M = M L^{-T} (the forward
// substitution) and Y_I = L^{-T}, so U = M V^{-1} = Y_M Y_I^T.  Each task is
// a 64 x 64 tile, two 64 x 64 x 64 products on the matrix cores (the panel
// one), operands staged in LDS as in the tiled product below; column block k
// is only read during step k, so the tasks of a step are independent.  The
// task of the next diagonal block, tile (k + 1, k + 1), then runs that
// block's diagonal kernel on the tile it has just formed (W_{k+1} and
// Z_{k+1}, into the other Z buffer) while the step's other tasks go on, so
// the chain of diagonal blocks overlaps the trailing updates.
struct AugStep {
    double *CV, *CM, *CI;  // working rows: V (R x R), M (I x R), identity (R x R)
    double *YM, *YI;       // outputs: M L^{-T} (I x R), L^{-T} (R x R)
    double *W;             // W_k at rows k0 .. (pitch 64)
    double *Z;             // Z_k at Z + (k & 1) 4096 (64 x 64 each)
    int64_t R, I;
    int k, nblk, mblk;
    int *flag;
};
constexpr int kAugPitch = 68;
constexpr size_t kAugLds = 2 * 64 * kAugPitch * sizeof(double);
static_assert(kAugLds >= (2 * 64 * 65 + 4 * 64) * sizeof(double),
              "the step's LDS also holds the diagonal kernel's buffers");

__global__ __launch_bounds__(256) void als_aug_step_kernel(AugStep a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    double(*As)[kAugPitch] = reinterpret_cast<double(*)[kAugPitch]>(smem);  // As[t][r] = A(r, t)
    double(*Bs)[kAugPitch] =
        reinterpret_cast<double(*)[kAugPitch]>(smem + 64 * kAugPitch * sizeof(double));
    __shared__ int sflag;
    const int k = a.k;
    const int x = blockIdx.x, y = blockIdx.y;
    const int j = k + x;
    const int nA = a.nblk - 1 - k;
    int sec;
    int64_t rb;
    if (y < nA) {
        sec = 0;
        rb = k + 1 + y;
        if (x == 0 || j > rb) return;  // V rows: trailing lower tiles only
    } else if (y < nA + k + 1) {
        sec = 1;
        rb = y - nA;
    } else {
        sec = 2;
        rb = y - nA - (k + 1);
    }
    const int64_t R = a.R;
    double *C = sec == 0 ? a.CV : sec == 1 ? a.CI : a.CM;
    const int64_t r0 = rb * 64, k0 = (int64_t)k * 64, j0 = (int64_t)j * 64;
    const int nr = (int)min<int64_t>(64, (sec == 2 ? a.I : R) - r0);
    const int kn = (int)min<int64_t>(64, R - k0);
    const int jn = (int)min<int64_t>(64, R - j0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;
    const int r16 = lane & 15, q = lane >> 4;
    const int tl = tid & 63, th = tid >> 6;  // load mapping: 64 along the row, 4 rows per pass
    // A operand: C(r0 + r, k0 + t); B operand: W_k (panel) or Z_k (trailing),
    // both read along their rows by consecutive threads.  (The failure word
    // is read once for the workgroup while these loads are in flight; they
    // stay inside the matrices either way, and nothing is stored past it.)
    {
        double va[16], vb[16];
        const double *Bsrc = x == 0 ? a.W + k0 * 64 : a.Z + (k & 1) * 4096;
        // (an identity row block at its own step is still the identity)
        const bool eye = sec == 1 && rb == k;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = th + 4 * u;
            va[u] = (r < nr && tl < kn) ? (eye ? (r == tl ? 1.0 : 0.0) : C[(r0 + r) * R + k0 + tl])
                                        : 0.0;
            vb[u] = (r < kn && tl < kn) ? Bsrc[r * 64 + tl] : 0.0;
        }
        if (flag_once(a.flag, &sflag)) return;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int r = th + 4 * u;
            As[tl][r] = va[u];
            Bs[r][tl] = vb[u];
        }
    }
    __syncthreads();
    adx4 acc[2][2];
    auto product = [&]() {
#pragma unroll
        for (int xx = 0; xx < 2; ++xx)
#pragma unroll
            for (int yy = 0; yy < 2; ++yy) acc[xx][yy] = adx4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int kk = 0; kk < 64; kk += 4) {
            const int kq = kk + q;
            const double a0 = As[kq][wr + r16], a1 = As[kq][wr + 16 + r16];
            const double b0 = Bs[kq][wc + r16], b1 = Bs[kq][wc + 16 + r16];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
    };
    if (x == 0) {
        // panel: Y(r0 + r, k0 + c) = (C(i, k) W_k)(r, c)
        product();
        double *Y = sec == 1 ? a.YI : a.YM;
#pragma unroll
        for (int xx = 0; xx < 2; ++xx)
#pragma unroll
            for (int yy = 0; yy < 2; ++yy)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = wr + 16 * xx + 4 * e + q, c = wc + 16 * yy + r16;
                    if (r < nr && c < kn) Y[(r0 + r) * R + k0 + c] = acc[xx][yy][e];
                }
        return;
    }
    // trailing: T = C(i, k) Z_k, then C(i, j) -= T C_V(j, k)^T.  The second
    // operand's loads and this thread's entries of C(i, j) go out before the
    // first product (an identity row block's entries right of its own block
    // are still zero at its own step).
    double vb[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const int c = th + 4 * u;
        vb[u] = (c < jn && tl < kn) ? a.CV[(j0 + c) * R + k0 + tl] : 0.0;
    }
    const bool zero_old = sec == 1 && rb == k;
    double cv[16];
#pragma unroll
    for (int xx = 0; xx < 2; ++xx)
#pragma unroll
        for (int yy = 0; yy < 2; ++yy)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wr + 16 * xx + 4 * e + q, c = wc + 16 * yy + r16;
                cv[(xx * 2 + yy) * 4 + e] =
                    (r < nr && c < jn && !zero_old) ? C[(r0 + r) * R + j0 + c] : 0.0;
            }
    product();
    __syncthreads();  // every wave is done with the first operands
#pragma unroll
    for (int xx = 0; xx < 2; ++xx)
#pragma unroll
        for (int yy = 0; yy < 2; ++yy)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                As[wc + 16 * yy + r16][wr + 16 * xx + 4 * e + q] = acc[xx][yy][e];
#pragma unroll
    for (int u = 0; u < 16; ++u) Bs[tl][th + 4 * u] = vb[u];
    __syncthreads();
    product();
    // the next diagonal block's tile: its new values also go to LDS (after
    // every wave is done with the operands there) for the diagonal kernel
    const bool next_diag = sec == 0 && x == 1 && rb == k + 1;
    double *Ts = reinterpret_cast<double *>(smem);  // 64 x 65
    if (next_diag) __syncthreads();
#pragma unroll
    for (int xx = 0; xx < 2; ++xx)
#pragma unroll
        for (int yy = 0; yy < 2; ++yy)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = wr + 16 * xx + 4 * e + q, c = wc + 16 * yy + r16;
                if (r < nr && c < jn) {
                    const double v = cv[(xx * 2 + yy) * 4 + e] - acc[xx][yy][e];
                    C[(r0 + r) * R + j0 + c] = v;
                    if (next_diag) Ts[r * 65 + c] = v;
                } else if (next_diag) {
                    Ts[r * 65 + c] = r == c ? 1.0 : 0.0;  // a narrow last block's padding
                }
            }
    if (next_diag) {
        __syncthreads();
        double(*colB)[64] = reinterpret_cast<double(*)[64]>(Ts + 64 * 65);
        double(*colI)[64] = colB + 2;
        // (the block is read into registers before Xs, at Ts, is written)
        chol_diag_block(Ts, 65, jn, j0, a.W, a.Z + ((k + 1) & 1) * 4096, a.flag, colB, colI, Ts);
    }
}

// C (m x n, leading dimension ldc) = beta C + alpha A B on the fp64 matrix
// cores, with A(i, t) at A[i sai + t sat] and B(t, j) at B[t sbt + j sbj]
// (element type TA for both, widened to fp64; beta = 0 writes alpha A B
// without reading C).  A workgroup owns a 64 x 64 tile of C, each of its
// four waves a 32 x 32 quarter as 2 x 2 blocks of v_mfma_f64_16x16x4f64
// accumulators; K is staged through LDS in chunks of 64, the next chunk's
// loads in flight while the matrix cores work on the current one.  shape:
// kGemmFull; kGemmSym (C symmetric, m = n: the tiles on and below the
// diagonal are formed, each one below also stored transposed above); or
// kGemmUpperB (B(t, j) = 0 for t below j's 64-column tile: the sum for that
// tile starts there).  kseg > 0 (kGemmFull or kGemmUpperB, beta = 0): the
// sum of a tile is cut into segments of kseg chunks, workgroup z taking
// segment z and storing its partial sum to part + z m n (m x n, pitch n);
// als_gemm_segments_kernel then adds a tile's segments in order.  C must not
// overlap A or B.  The sums over t follow the matrix cores' fixed order, so
// results are deterministic.
constexpr int kGemmFull = 0, kGemmSym = 1, kGemmUpperB = 2;
typedef double gdx4 __attribute__((ext_vector_type(4)));

// (Chunks of 32: the operands take 35 KB of LDS and the registers are held
// to three waves per SIMD, so three workgroups share a compute unit.)
constexpr int kGemmKC = 32;
template <typename TA>
__global__ __launch_bounds__(256, 3) void als_mfma_gemm_kernel(double *__restrict__ C, int64_t ldc,
                                                            const TA *__restrict__ A,
                                                            int64_t sai, int64_t sat,
                                                            const TA *__restrict__ B, int64_t sbt,
                                                            int64_t sbj, int64_t m, int64_t n,
                                                            int64_t K, double alpha, double beta,
                                                            int shape, int kseg,
                                                            double *__restrict__ part,
                                                            const int *__restrict__ flag)
{
    constexpr int TM = 64, TN = 64, KC = kGemmKC, PA = TM + 4, NL = TM * KC / 256;
    static_assert(KC == 32 && NL == 8, "the load mapping below assumes chunks of 32");
    extern __shared__ __align__(16) unsigned char smem[];
    double(*As)[PA] = reinterpret_cast<double(*)[PA]>(smem);                  // KC x PA
    double(*Bs)[PA] = reinterpret_cast<double(*)[PA]>(smem + KC * PA * sizeof(double));
    if (*flag) return;
    const int64_t ti = blockIdx.y, tj = blockIdx.x;
    if (shape == kGemmSym && tj > ti) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wr = (wave >> 1) * 32, wc = (wave & 1) * 32;  // the wave's quarter
    const int r16 = lane & 15, q = lane >> 4;
    const int64_t i0 = ti * TM, j0 = tj * TN;
    gdx4 acc[2][2];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y) acc[x][y] = gdx4{0.0, 0.0, 0.0, 0.0};
    // The unit-stride dimension of each operand runs across consecutive
    // threads: along a 64-long dimension (rows of A, columns of B) thread tid
    // takes index tid % 64 and tid / 64 + 4 u along the chunk's 32; along the
    // chunk, index tid % 32 and tid / 32 + 8 u along the other (u = 0 .. NL -
    // 1).  Its byte offset inside the chunk's tile is a fixed 32-bit part (per
    // thread) plus u times a uniform step, so the loads need no per-thread
    // 64-bit addresses.
    const bool a_t = sat == 1, b_c = sbj == 1;
    const int lo = tid & 63, hi = tid >> 6, lo32 = tid & 31, hi32 = tid >> 5;
    const int ra = a_t ? hi32 : lo, ta = a_t ? lo32 : hi;   // A's (row, t) at u = 0
    const int tb0 = b_c ? hi : lo32, cb = b_c ? lo : hi32;  // B's (t, column) at u = 0
    const int dra = a_t ? 8 : 0, dta = a_t ? 0 : 4, dtb = b_c ? 4 : 0, dcb = b_c ? 0 : 8;
    const uint32_t voffA = (uint32_t)((ra * sai + ta * sat) * (int64_t)sizeof(TA));
    const uint32_t voffB = (uint32_t)((tb0 * sbt + cb * sbj) * (int64_t)sizeof(TA));
    const int64_t stepA = dra * sai + dta * sat, stepB = dtb * sbt + dcb * sbj;
    double va[NL], vb[NL];
    // a chunk's operands into registers (zero outside the matrices)
    auto fetch = [&](int64_t t0) {
        const TA *Ab = A + i0 * sai + t0 * sat;
        const TA *Bb = B + t0 * sbt + j0 * sbj;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int r = ra + dra * u, t = ta + dta * u;
            const bool ok = i0 + r < m && t0 + t < K;
            const char *pa = reinterpret_cast<const char *>(Ab + u * stepA) + voffA;
            va[u] = ok ? (double)*reinterpret_cast<const TA *>(pa) : 0.0;
            const int c = cb + dcb * u, tb = tb0 + dtb * u;
            const bool okb = t0 + tb < K && j0 + c < n;
            const char *pb = reinterpret_cast<const char *>(Bb + u * stepB) + voffB;
            vb[u] = okb ? (double)*reinterpret_cast<const TA *>(pb) : 0.0;
        }
    };
    const int64_t kfirst = shape == kGemmUpperB ? (j0 < K ? j0 : K) : 0;
    const int64_t kbeg = kseg > 0 ? kfirst + (int64_t)blockIdx.z * kseg * KC : kfirst;
    if (blockIdx.z > 0 && kbeg >= K) return;  // past this tile's sum
    const int64_t kend = kseg > 0 ? min(K, kbeg + (int64_t)kseg * KC) : K;
    fetch(kbeg);
    for (int64_t t0 = kbeg; t0 < kend; t0 += KC) {
        __syncthreads();  // the previous chunk's operands are read
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            As[ta + dta * u][ra + dra * u] = va[u];
            Bs[tb0 + dtb * u][cb + dcb * u] = vb[u];
        }
        __syncthreads();
        // the next chunk's loads go out before this chunk's matrix-core work
        if (t0 + KC < kend) fetch(t0 + KC);
#pragma unroll 4
        for (int kk = 0; kk < KC; kk += 4) {
            const int k = kk + q;
            const double a0 = As[k][wr + r16], a1 = As[k][wr + 16 + r16];
            const double b0 = Bs[k][wc + r16], b1 = Bs[k][wc + 16 + r16];
            acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
        }
    }
    // element e of a block holds row 4 e + lane / 16, column lane % 16
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 2; ++y)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t i = i0 + wr + 16 * x + 4 * e + q, j = j0 + wc + 16 * y + r16;
                if (i < m && j < n) {
                    const double v = acc[x][y][e];
                    if (kseg > 0) {
                        part[(int64_t)blockIdx.z * m * n + i * n + j] = v;
                    } else {
                        double *c = C + i * ldc + j;
                        *c = beta == 0.0 ? alpha * v : __builtin_fma(alpha, v, beta * *c);
                    }
                }
            }
    if (shape == kGemmSym && ti != tj) {
        // the transposed tile above the diagonal, through LDS so that
        // consecutive threads store consecutive entries of a row (As and Bs
        // together hold the 64 x 64 tile)
        double(*Ts)[PA] = As;  // Ts[j - j0][i - i0]
        __syncthreads();       // every wave is done with the operands
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int y = 0; y < 2; ++y)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    Ts[wc + 16 * y + r16][wr + 16 * x + 4 * e + q] = acc[x][y][e];
        __syncthreads();
        for (int u = 0; u < TN * TM / 256; ++u) {
            const int jr = hi + 4 * u, ic = lo;  // row j0 + jr of C, column i0 + ic
            const int64_t j = j0 + jr, i = i0 + ic;
            if (j < n && i < m) {
                double *c = C + j * ldc + i;
                const double v = Ts[jr][ic];
                *c = beta == 0.0 ? alpha * v : __builtin_fma(alpha, v, beta * *c);
            }
        }
    }
}
constexpr size_t kGemmLds = 2 * kGemmKC * (64 + 4) * sizeof(double);
static_assert(2 * kGemmKC >= 64, "the mirrored tile fits the operands' LDS");

hipError_t allow_large_lds(const void *k);

// C(i, j) = alpha sum_{z < segments of j's tile} part[z m n + i n + j], the
// segments added in order.
__global__ __launch_bounds__(256) void als_gemm_segments_kernel(double *__restrict__ C, int64_t ldc,
                                                                const double *__restrict__ part,
                                                                int64_t m, int64_t n, int64_t K,
                                                                int shape, int kseg, double alpha,
                                                                const int *__restrict__ flag)
{
    if (*flag) return;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= m * n) return;
    const int64_t i = e / n, j = e - (e / n) * n;
    const int64_t j0 = j / 64 * 64;
    const int64_t kfirst = shape == kGemmUpperB ? (j0 < K ? j0 : K) : 0;
    const int64_t seg = (int64_t)kseg * kGemmKC;
    const int64_t nz = kfirst < K ? (K - kfirst + seg - 1) / seg : 1;
    double v = 0.0;
    for (int64_t z = 0; z < nz; ++z) v += part[z * m * n + e];
    C[i * ldc + j] = alpha * v;
}

// Launches the product above on 64 x 64 tiles.  part, part_elems: room for
// segment partial sums (nullptr / 0: none).  With
// room for at least two m x n partials, a long sum (kGemmFull or kGemmUpperB
// with beta = 0) is cut into segments so that the launch has enough
// workgroups of balanced length.
template <typename TA>
hipError_t launch_gemm(double *C, int64_t ldc, const TA *A, int64_t sai, int64_t sat, const TA *B,
                       int64_t sbt, int64_t sbj, int64_t m, int64_t n, int64_t K, double alpha,
                       double beta, int shape, const int *flag, hipStream_t s,
                       double *part = nullptr, int64_t part_elems = 0)
{
    const int64_t gx = (n + 63) / 64, gy = (m + 63) / 64;
    if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;  // grid limits
    const hipError_t a = allow_large_lds(reinterpret_cast<const void *>(als_mfma_gemm_kernel<TA>));
    if (a != hipSuccess) return a;
    // up to four segments when fewer than 768 tiles would each run a long sum
    // (as many as the partial space holds)
    int kseg = 0;
    int64_t nseg = 1;
    const int64_t nchunk = (K + kGemmKC - 1) / kGemmKC;
    if (part && shape != kGemmSym && beta == 0.0 && gx * gy < 768 && nchunk > 16 && m * n > 0) {
        const int64_t ns = std::min<int64_t>({(int64_t)4, part_elems / (m * n), nchunk / 4});
        if (ns >= 2) {
            kseg = (int)((nchunk + ns - 1) / ns);
            nseg = (nchunk + kseg - 1) / kseg;
        }
    }
    hipLaunchKernelGGL(als_mfma_gemm_kernel<TA>, dim3((unsigned)gx, (unsigned)gy, (unsigned)nseg),
                       dim3(256), kGemmLds, s, C, ldc, A, sai, sat, B, sbt, sbj, m, n, K, alpha, beta,
                       shape, kseg, part, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || kseg == 0) return e;
    hipLaunchKernelGGL(als_gemm_segments_kernel, dim3((unsigned)((m * n + 255) / 256)), dim3(256), 0,
                       s, C, ldc, part, m, n, K, shape, kseg, alpha, flag);
    return hipGetLastError();
}

// sum_i M(i, r) U(i, r) for every column r.  A workgroup takes 16 columns;
// thread (c, g) sums rows g, g + 16, ... of column c in order, and the 16
// group sums are added in group order (a fixed order).
template <typename T>
__global__ __launch_bounds__(256) void als_colsum_kernel(const double *__restrict__ M,
                                                         const T *__restrict__ U, int64_t I,
                                                         int64_t R, double *__restrict__ out,
                                                         const int *__restrict__ flag)
{
    __shared__ double part[16][17];
    if (*flag) return;
    const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
    const int64_t r = (int64_t)blockIdx.x * 16 + c;
    double s = 0.0;
    if (r < R) {
#pragma unroll 4
        for (int64_t i = g; i < I; i += 16) s += M[i * R + r] * (double)U[i * R + r];
    }
    part[g][c] = s;
    __syncthreads();
    if (g == 0 && r < R) {
        double t = part[0][c];
        for (int h = 1; h < 16; ++h) t += part[h][c];
        out[r] = t;
    }
}

// ||model||^2 partials for large R: workgroup w sums the entries
// e = w * 256 + tid + k * 256 * gridDim in increasing k per thread, then
// over the workgroup in a fixed order; als_fit_kernel adds the partials in
// workgroup order.
__global__ __launch_bounds__(kRedThreads) void als_model_norm_kernel(
    const double *__restrict__ lam64, const double *__restrict__ Gall, int order, int64_t R,
    double *__restrict__ parts, const int *__restrict__ flag)
{
    __shared__ double sh[kRedThreads / 64];
    if (*flag) return;
    const int64_t RR = R * R;
    double s = 0.0;
    for (int64_t e = (int64_t)blockIdx.x * kRedThreads + threadIdx.x; e < RR;
         e += (int64_t)gridDim.x * kRedThreads) {
        const int64_t a = e / R, b = e - (e / R) * R;
        double v = lam64[a] * lam64[b];
        for (int m = 0; m < order; ++m) v *= Gall[(int64_t)m * RR + e];
        s += v;
    }
    s = block_sum(s, sh);
    if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

// ---------------------------------------------------------------------------
// Host launchers (used by the C-ABI driver)
// ---------------------------------------------------------------------------

template <typename T>
hipError_t launch_sumsq(const T *X, int64_t N, double *partial, int nparts, double *out,
                        hipStream_t s)
{
    hipLaunchKernelGGL(sumsq_partial_kernel<T>, dim3(nparts), dim3(kRedThreads), 0, s, X, N,
                       partial);
    hipLaunchKernelGGL(sum_final_kernel, dim3(1), dim3(kRedThreads), 0, s, (const double *)partial,
                       nparts, out);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gram(const T *U, int64_t I, int64_t R, double *G, const int *flag, hipStream_t s)
{
    if (R > 64) {
        // G = U^T U as a tiled product (the same per-entry order over i)
        return launch_gemm<T>(G, R, U, (int64_t)1, R, U, R, (int64_t)1, R, R, I, 1.0, 0.0, kGemmSym,
                              flag, s);
    }
    const int64_t n = R * R;
    hipLaunchKernelGGL(gram_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, U, I, R,
                       G, flag);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_gram_all(const T *const *U, const int64_t *dims, int order, int64_t R, double *G,
                           const int *flag, hipStream_t s)
{
    if (R > 64 || order > 5) {
        for (int m = 0; m < order; ++m) {
            const hipError_t e = launch_gram<T>(U[m], dims[m], R, G + (size_t)m * R * R, flag, s);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    GramAllArgs g{};
    for (int m = 0; m < order; ++m) {
        g.U[m] = U[m];
        g.I[m] = dims[m];
    }
    hipLaunchKernelGGL(gram_all_kernel<T>, dim3((unsigned)((R * R + 255) / 256), (unsigned)order),
                       dim3(256), 0, s, g, R, G, flag);
    return hipGetLastError();
}

hipError_t launch_chol(const double *Gall, int order, int n, int64_t R, double *L, int *flag,
                       hipStream_t s)
{
    if (R > 64) return hipErrorInvalidValue;  // larger ranks: launch_update_blocked
    auto k = R <= 16 ? als_chol_wave_kernel<16>
             : R <= 32 ? als_chol_wave_kernel<32>
                       : als_chol_wave_kernel<64>;
    hipLaunchKernelGGL(k, dim3(1), dim3(256), 0, s, Gall, order, n, (int)R, L, flag);
    return hipGetLastError();
}

hipError_t launch_solve(const double *M, const double *L, int64_t I, int64_t R, double *Unew,
                        const int *flag, hipStream_t s)
{
    if (R > 64) return hipErrorInvalidValue;  // larger ranks: launch_update_blocked
    hipLaunchKernelGGL(als_solve_wave_kernel, dim3((unsigned)((I + 3) / 4)), dim3(256), 0, s, M, L,
                       I, R, Unew, flag);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_normalize(const double *Unew, int64_t I, int64_t R, T *Uout, double *lam64,
                            T *lamT, const int *flag, hipStream_t s)
{
    hipLaunchKernelGGL(als_normalize_kernel<T>, dim3((unsigned)((R + 15) / 16)), dim3(256), 0, s,
                       Unew, I, R, Uout, lam64, lamT, flag);
    return hipGetLastError();
}

// Bytes of LDS the one-workgroup update of a mode needs (0: not usable).
size_t update_small_lds(int64_t I, int64_t R)
{
    if (R > 64 || I > (1 << 20)) return 0;
    const int64_t rm = R <= 16 ? 16 : R <= 32 ? 32 : 64;
    const int64_t nx = std::max(rm * (rm + 1), I * R);
    const size_t b = (size_t)(256 + 128 + 2 * R * R + nx + 64 + 2) * sizeof(double);
    return b <= 150 * 1024 ? b : 0;
}

hipError_t allow_large_lds(const void *k);

template <typename T>
hipError_t launch_update_small(const double *Gall, int order, int n, const double *M, int64_t I,
                               int64_t R, T *Uout, double *lam64, T *lamT, double *G, int *flag,
                               hipStream_t s)
{
    const size_t lds = update_small_lds(I, R);
    if (!lds) return hipErrorInvalidValue;
    auto k = R <= 16 ? als_update_small_kernel<T, 16>
             : R <= 32 ? als_update_small_kernel<T, 32>
                       : als_update_small_kernel<T, 64>;
    if (lds > 64 * 1024) {
        const hipError_t a = allow_large_lds(reinterpret_cast<const void *>(k));
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3(1), dim3(256), lds, s, Gall, order, n, M, I, R, Uout, lam64, lamT,
                       G, flag);
    return hipGetLastError();
}

hipError_t launch_side_chol(const double *Gall, int order, int n, int64_t R, double *Vinv,
                            double *Vout, int *flag, unsigned *ticket, const unsigned *wait_on,
                            unsigned wait_for, unsigned *done, unsigned done_val, hipStream_t s)
{
    if (R > 64) return hipErrorInvalidValue;
    auto k = R <= 16 ? als_side_chol_kernel<16>
             : R <= 32 ? als_side_chol_kernel<32>
                       : als_side_chol_kernel<64>;
    const size_t lds = R <= 16 ? side_chol_lds<16>() : R <= 32 ? side_chol_lds<32>()
                                                                : side_chol_lds<64>();
    if (lds > 64 * 1024) {
        const hipError_t a = allow_large_lds(reinterpret_cast<const void *>(k));
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3(8), dim3(256), lds, s, Gall, order, n, (int)R, Vinv, Vout, flag,
                       ticket, SeqArgs{wait_on, wait_for, done, done_val});
    return hipGetLastError();
}

template <typename T>
hipError_t launch_apply_small(const double *M, int64_t I, int64_t R, const double *Vinv, T *Uout,
                              double *lam64, T *lamT, double *G, int *flag,
                              const unsigned *wait_on, unsigned wait_for, unsigned *done,
                              unsigned done_val, const AlsFitOut *fit, hipStream_t s)
{
    FitArgs fa{};
    if (fit)
        fa = FitArgs{fit->V,       fit->Gall,     fit->order,   fit->scal,   fit->tol,
                     fit->have_prev, fit->out_fit, fit->out_flag, fit->out_seq, fit->seq_val};
    const size_t lds = apply_small_lds(I, R);
    if (!lds) return hipErrorInvalidValue;
    auto k = R <= 16 ? als_apply_small_kernel<T, 16>
             : R <= 32 ? als_apply_small_kernel<T, 32>
                       : als_apply_small_kernel<T, 64>;
    if (lds > 64 * 1024) {
        const hipError_t a = allow_large_lds(reinterpret_cast<const void *>(k));
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3(1), dim3(256), lds, s, M, I, R, Vinv, Uout, lam64, lamT, G, flag,
                       fa, SeqArgs{wait_on, wait_for, done, done_val});
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fill(T *p, int64_t n, T v, hipStream_t s)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(fill_kernel<T>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n, v);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_fit(const double *M, const T *Ulast, int64_t Ilast, const double *lam64,
                      int64_t R, int *flag, const AlsFitOut &fit, double *parts, int max_parts,
                      double *colsum_buf, unsigned *done, unsigned done_val, hipStream_t s)
{
    const double *Gall = fit.Gall;
    const int order = fit.order;
    const FitArgs fa{fit.V,         fit.Gall,     fit.order,    fit.scal,   fit.tol,
                     fit.have_prev, fit.out_fit, fit.out_flag, fit.out_seq, fit.seq_val};
    const double *colsum = nullptr;
    if (R > 256) {
        hipLaunchKernelGGL(als_colsum_kernel<T>, dim3((unsigned)((R + 15) / 16)), dim3(256), 0, s,
                           M, Ulast, Ilast, R, colsum_buf, flag);
        colsum = colsum_buf;
    }
    int np = 0;
    if (R * R > 65536) {
        np = (int)std::min<int64_t>(max_parts, (R * R + 2047) / 2048);
        hipLaunchKernelGGL(als_model_norm_kernel, dim3(np), dim3(kRedThreads), 0, s, lam64, Gall,
                           order, R, parts, flag);
    }
    hipLaunchKernelGGL(als_fit_kernel<T>, dim3(1), dim3(kRedThreads), 0, s, M, Ulast, Ilast, lam64,
                       R, flag, parts, np, colsum, fa, SeqArgs{nullptr, 0u, done, done_val});
    return hipGetLastError();
}

// U_new = M V^{-1} for ranks past the one-workgroup update (R > 64), by
// 64-wide column blocks: V = Hadamard_{m != n} G_m into CV (its tiles on and
// below the diagonal) and M into CM in one launch, then
// the first diagonal block (W_0, Z_0) and per block
// k one step launch (panels and trailing updates of every row block, and
// block k + 1's diagonal kernel), and at the end U = Y_M Y_I^T into CM
// (which the caller passes as U_new).
hipError_t launch_update_blocked(const double *Gall, int order, int n, int64_t R, const double *M,
                                 int64_t I, double *CV, double *CI, double *CM, double *YI,
                                 double *YM, double *W, double *Z, int *flag, hipStream_t s)
{
    // (the first diagonal block is a whole one only for R > 64)
    if (R <= 64) return hipErrorInvalidValue;
    const int nblk = (int)((R + 63) / 64);
    const int64_t mblk = (I + 63) / 64;
    if (mblk + 2 * (int64_t)nblk > 65535) return hipErrorInvalidValue;  // grid limit
    hipError_t e = allow_large_lds(reinterpret_cast<const void *>(als_aug_step_kernel));
    if (e != hipSuccess) return e;
    const int64_t RR = R * R, IR = I * R;
    if ((RR + IR + 255) / 256 > INT32_MAX) return hipErrorInvalidValue;  // grid limit
    hipLaunchKernelGGL(als_aug_setup_kernel, dim3((unsigned)((RR + IR + 255) / 256)), dim3(256), 0,
                       s, Gall, order, n, R, CV, M, CM, IR, flag);
    AugStep a{CV, CM, CI, YM, YI, W, Z, R, I, 0, nblk, (int)mblk, flag};
    // the first diagonal block; each step forms the next one's
    hipLaunchKernelGGL(als_chol_diag_kernel, dim3(1), dim3(256), 0, s, CV, R, (int64_t)0, W, Z,
                       flag);
    for (int k = 0; k < nblk; ++k) {
        a.k = k;
        const unsigned gy = (unsigned)((nblk - 1 - k) + (k + 1) + mblk);
        hipLaunchKernelGGL(als_aug_step_kernel, dim3((unsigned)(nblk - k), gy), dim3(256), kAugLds,
                           s, a);
    }
    // U = Y_M Y_I^T: A(i, t) = Y_M[i R + t], B(t, j) = Y_I[j R + t]
    // (L^{-T} is upper triangular: B(t, j) = Y_I(j, t) = 0 for t < j)
    // (the identity rows' working copy is free after the last step: it holds
    // the segment partial sums)
    e = launch_gemm<double>(CM, R, YM, R, (int64_t)1, YI, (int64_t)1, R, I, R, R, 1.0, 0.0,
                            kGemmUpperB, flag, s, CI, R * R);
    if (e != hipSuccess) return e;
    return hipGetLastError();
}

template hipError_t launch_sumsq<double>(const double *, int64_t, double *, int, double *, hipStream_t);
template hipError_t launch_sumsq<float>(const float *, int64_t, double *, int, double *, hipStream_t);
template hipError_t launch_gram<double>(const double *, int64_t, int64_t, double *, const int *, hipStream_t);
template hipError_t launch_gram<float>(const float *, int64_t, int64_t, double *, const int *, hipStream_t);
template hipError_t launch_gram_all<double>(const double *const *, const int64_t *, int, int64_t, double *, const int *, hipStream_t);
template hipError_t launch_gram_all<float>(const float *const *, const int64_t *, int, int64_t, double *, const int *, hipStream_t);
template hipError_t launch_update_small<double>(const double *, int, int, const double *, int64_t, int64_t, double *, double *, double *, double *, int *, hipStream_t);
template hipError_t launch_update_small<float>(const double *, int, int, const double *, int64_t, int64_t, float *, double *, float *, double *, int *, hipStream_t);
template hipError_t launch_normalize<double>(const double *, int64_t, int64_t, double *, double *, double *, const int *, hipStream_t);
template hipError_t launch_normalize<float>(const double *, int64_t, int64_t, float *, double *, float *, const int *, hipStream_t);
template hipError_t launch_apply_small<double>(const double *, int64_t, int64_t, const double *, double *, double *, double *, double *, int *, const unsigned *, unsigned, unsigned *, unsigned, const AlsFitOut *, hipStream_t);
template hipError_t launch_apply_small<float>(const double *, int64_t, int64_t, const double *, float *, double *, float *, double *, int *, const unsigned *, unsigned, unsigned *, unsigned, const AlsFitOut *, hipStream_t);
template hipError_t launch_fill<double>(double *, int64_t, double, hipStream_t);
template hipError_t launch_fill<float>(float *, int64_t, float, hipStream_t);
template hipError_t launch_fill<int>(int *, int64_t, int, hipStream_t);
template hipError_t launch_fit<double>(const double *, const double *, int64_t, const double *, int64_t, int *, const AlsFitOut &, double *, int, double *, unsigned *, unsigned, hipStream_t);
template hipError_t launch_fit<float>(const double *, const float *, int64_t, const double *, int64_t, int *, const AlsFitOut &, double *, int, double *, unsigned *, unsigned, hipStream_t);

}  // namespace mttkrp
