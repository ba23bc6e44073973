// C ABI of the matrix-free MTTKRP library (declared in include/mttkrp.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// plans the decomposition (plan.cpp), fills the kernel parameter block and
// enqueues the kernels on the caller's stream.  The library allocates no
// device memory: partial sums and CP-ALS state live in the caller's
// workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <mutex>
#include <vector>

#include "../../include/mttkrp.h"
#include "als_kernels.hpp"
#include "plan.hpp"
#include "tile_select.hpp"

namespace mttkrp {

template <typename T>
hipError_t launch_mttkrp(const Plan &pl, hipStream_t stream, bool with_reduce);
template <typename T>
hipError_t launch_mttkrp_multi(const Plan *const *pls, int np, hipStream_t stream);

namespace {

constexpr int kSumsqParts = 1024;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Second stream of the current device for the all-mode call: created on first
// use (default priority, not synchronising with the null stream) and kept
// until the process ends.
hipError_t side_stream(hipStream_t *out)
{
    constexpr int kMaxDev = 64;
    static std::mutex mu;
    static hipStream_t ss[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ss[dev]) {
        e = hipStreamCreateWithFlags(&ss[dev], hipStreamNonBlocking);
        if (e != hipSuccess) {
            ss[dev] = nullptr;
            return e;
        }
    }
    *out = ss[dev];
    return hipSuccess;
}

// Host-visible slots for the fit and failure word of a CP-ALS run's last two
// sweeps.  They are allocated (pinned, coherent) on a host thread's first run
// on a device and kept until the thread ends: a thread runs one call at a
// time (a call returns only after its kernels are done), so calls never share
// a slot, and no call pays for the allocation again.
struct FitSlot {
    double fit;
    int flag;
    unsigned seq;  // the sweep's number plus one, stored last
};

FitSlot *fit_slots()
{
    constexpr int kMaxDev = 64;
    struct Cache {
        FitSlot *p[kMaxDev] = {};
        ~Cache()
        {
            for (FitSlot *q : p)
                if (q) (void)hipHostFree(q);
        }
    };
    thread_local Cache c;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
    if (!c.p[dev]) {
        void *q = nullptr;
        if (hipHostMalloc(&q, 2 * sizeof(FitSlot), hipHostMallocCoherent) != hipSuccess)
            return nullptr;
        c.p[dev] = static_cast<FitSlot *>(q);
    }
    return c.p[dev];
}

// Checks shared by the MTTKRP entry points.  `factors` may hold NULL at `mode`
// (mode < 0: every factor must be present).
int check_common(const void *X, const int64_t *dims, int order, const void *const *factors,
                 int64_t rank, int mode)
{
    if (!X || !dims || !factors) return MTTKRP_EINVAL;
    if (order < 3 || order > kMaxOrder) return MTTKRP_EORDER;
    if (rank < 1) return MTTKRP_EINVAL;
    for (int m = 0; m < order; ++m) {
        if (dims[m] < 1) return MTTKRP_EINVAL;
        if (m != mode && !factors[m]) return MTTKRP_EINVAL;
    }
    if (!aligned16(X)) return MTTKRP_EALIGN;
    for (int m = 0; m < order; ++m)
        if (factors[m] && !aligned16(factors[m])) return MTTKRP_EALIGN;
    return MTTKRP_OK;
}

// Factor pointers by role in the kernel parameter block.
void bind_factors(KParams &k, const void *const *factors)
{
    k.Uk0 = factors[k.k_mode0];
    k.Uk1 = k.k_mode1 >= 0 ? factors[k.k_mode1] : nullptr;
    k.Ur0 = k.r_mode0 >= 0 ? factors[k.r_mode0] : nullptr;
    k.Ur1 = k.r_mode1 >= 0 ? factors[k.r_mode1] : nullptr;
    for (int j = 0; j < 3; ++j) k.Uo[j] = j < k.nouter ? factors[k.o_mode[j]] : nullptr;
}

void bind_reduced(const Plan &pl, KParams &k, const void *const *factors)
{
    k.Ured = pl.red_mode >= 0 ? factors[pl.red_mode] : nullptr;
}

// Plan of one mode with every pointer bound.
template <typename T>
int bound_plan(const T *X, const int64_t *dims, int order, const T *const *factors, int64_t rank,
               int mode, void *out, int out64, void *ws, size_t ws_bytes, Plan &pl)
{
    int st = make_plan(dims, order, rank, mode, (int)sizeof(T), pl);
    if (st) return st;
    if (!plan_launchable(pl)) return MTTKRP_EINVAL;  // a forced tile without a kernel
    if (pl.ws_bytes > ws_bytes) return MTTKRP_EWORKSPACE;
    if (pl.ws_bytes > 0 && !ws) return MTTKRP_EINVAL;
    pl.kp.X = X;
    bind_factors(pl.kp, reinterpret_cast<const void *const *>(factors));
    bind_reduced(pl, pl.kp, reinterpret_cast<const void *const *>(factors));
    pl.kp.out = out;
    pl.kp.out64 = out64;
    pl.kp.partial = reinterpret_cast<double *>(ws);
    return MTTKRP_OK;
}

template <typename T>
int mttkrp_one(const T *X, const int64_t *dims, int order, const T *const *factors, int64_t rank,
               int mode, void *out, int out64, void *ws, size_t ws_bytes, hipStream_t stream)
{
    Plan pl;
    const int st = bound_plan<T>(X, dims, order, factors, rank, mode, out, out64, ws, ws_bytes, pl);
    if (st) return st;
    return launch_mttkrp<T>(pl, stream, true) == hipSuccess ? MTTKRP_OK : MTTKRP_EHIP;
}

// Rough time of an all-mode sweep: each mode bounded by streaming X at
// 5 TB/s or by the matrix cores at 60 (fp64) or 120 (fp32) TFLOP/s.
double sweep_seconds(const Plan *pl, int order)
{
    double t = 0.0;
    for (int m = 0; m < order; ++m) {
        const KParams &k = pl[m].kp;
        const double N = (double)k.x_bytes / pl[m].elem_bytes;
        const double mem = (double)k.x_bytes / 5e12;
        const double mma = 2.0 * N * (double)k.R / (pl[m].elem_bytes == 8 ? 60e12 : 120e12);
        t += std::max(mem, mma);
    }
    return t;
}
// Two streams in the all-mode call only pay off when the sweep hides the
// cost of the cross-stream dependencies (two per call, about 10 us each):
// measured faster on the 4-way fp32 rank-8 tensor (-8%, ~440 us) and the
// 5-way tensor (-1.5%), slower on the 256^3 fp64 rank-32 one (+6%, ~90 us).
// Nor when each mode is long: the two streams' modes then share the chip
// for their whole length, not only at one mode's tail (512^3 fp64 rank 2000,
// 8.3 ms per mode: 25.67 ms per sweep on two streams against 25.04 ms for
// the same modes one after another).
constexpr double kTwoStreamSweep = 200e-6;
constexpr double kTwoStreamModeMax = 3e-3;

// Two form-1 plans one multi-mode launch can run in turn: the same tile
// shape, the same B tile for every workgroup (contraction group, chunking,
// rank tiles, decomposition) and no partials.
bool fusable(const Plan &a, const Plan &b)
{
    const KParams &x = a.kp, &y = b.kp;
    return a.form == 1 && b.form == 1 && a.layout == 0 && b.layout == 0 && a.waves == 8 &&
           b.waves == 8 && a.mb == b.mb && a.nb == b.nb && a.vec == b.vec &&
           a.elem_bytes == b.elem_bytes && !x.to_partial && !y.to_partial && !x.tr && !y.tr &&
           x.k_mode0 == y.k_mode0 && x.k_mode1 == y.k_mode1 && x.K == y.K && x.Kc == y.Kc &&
           x.nkch == y.nkch && x.IkB == y.IkB && x.bpitch == y.bpitch && x.R == y.R &&
           x.grid_real == y.grid_real && x.grid_per_xcd == y.grid_per_xcd &&
           x.nrtiles == y.nrtiles && x.nsplit == y.nsplit && x.nsplit_it == y.nsplit_it &&
           a.grid == b.grid &&
           (a.elem_bytes == 8 ? select_multi_f64(a) : select_multi_f32(a)) != nullptr;
}

// A plain split plan: partials summed by split_reduce_kernel, or by the tile
// kernel of another launch.
// (The partner reads the partials with 32-bit offsets: their span must stay
// below 2^31 bytes.)
bool plain_split(const Plan &pl)
{
    return pl.kp.nsplit > 1 && !pl.kp.tr &&
           pl.kp.nsplit * pl.kp.In * pl.kp.R * 8 < (INT64_C(1) << 31) - 64;
}

}  // namespace

// Argument checks of a single-mode call, without the workspace (host only).
int check_mode_call(const void *X, const int64_t *dims, int order, const void *const *factors,
                    int64_t rank, int mode, const void *out)
{
    const int st = check_common(X, dims, order, factors, rank, mode < 0 ? 0 : mode);
    if (st) return st;
    if (mode < 0 || mode >= order || !out) return MTTKRP_EINVAL;
    if (!aligned16(out)) return MTTKRP_EALIGN;
    return MTTKRP_OK;
}

namespace {

template <typename T>
int mttkrp_entry(const T *X, const int64_t *dims, int order, const T *const *factors,
                 int64_t rank, int mode, T *out, void *ws, size_t ws_bytes, void *stream)
{
    int st = check_common(X, dims, order, reinterpret_cast<const void *const *>(factors), rank,
                          mode < 0 ? 0 : mode);
    if (st) return st;
    if (mode < 0 || mode >= order || !out) return MTTKRP_EINVAL;
    if (!aligned16(out) || (ws && !aligned16(ws))) return MTTKRP_EALIGN;
    return mttkrp_one<T>(X, dims, order, factors, rank, mode, out, 0, ws, ws_bytes,
                         reinterpret_cast<hipStream_t>(stream));
}

// Largest workspace of one mode (each a multiple of 256 bytes).
int mode_ws_max(const int64_t *dims, int order, int64_t rank, int elem, size_t *bytes)
{
    size_t mx = 0;
    for (int m = 0; m < order; ++m) {
        Plan pl;
        const int st = make_plan(dims, order, rank, m, elem, pl);
        if (st) return st;
        mx = std::max(mx, pl.ws_bytes);
    }
    *bytes = mx;
    return MTTKRP_OK;
}

// The all-mode call holds two modes' partials at once (two streams, or one
// mode's partials pending while the next writes its own): two halves of the
// largest mode workspace.
int all_ws(const int64_t *dims, int order, int64_t rank, int elem, size_t *bytes)
{
    size_t mx = 0;
    const int st = mode_ws_max(dims, order, rank, elem, &mx);
    if (st) return st;
    *bytes = 2 * mx;
    return MTTKRP_OK;
}

template <typename T>
int mttkrp_all_entry(const T *X, const int64_t *dims, int order, const T *const *factors,
                     int64_t rank, T *const *outs, void *ws, size_t ws_bytes, void *stream)
{
    int st = check_common(X, dims, order, reinterpret_cast<const void *const *>(factors), rank, -1);
    if (st) return st;
    if (!outs) return MTTKRP_EINVAL;
    for (int m = 0; m < order; ++m) {
        if (!outs[m]) return MTTKRP_EINVAL;
        if (!aligned16(outs[m])) return MTTKRP_EALIGN;
    }
    if (ws && !aligned16(ws)) return MTTKRP_EALIGN;
    size_t need = 0;
    st = all_ws(dims, order, rank, (int)sizeof(T), &need);
    if (st) return st;
    if (need > ws_bytes) return MTTKRP_EWORKSPACE;
    if (need > 0 && !ws) return MTTKRP_EINVAL;
    // Every plan first (so that nothing is launched when one fails), then the
    // launches.  The modes are independent given the factors, so the order is
    // free.
    Plan pl[kMaxOrder];
    for (int m = 0; m < order; ++m) {
        st = bound_plan<T>(X, dims, order, factors, rank, m, outs[m], 0, ws, ws_bytes, pl[m]);
        if (st) return st;
    }
    const size_t half = need / 2;
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto in_half = [&](int h) {
        return reinterpret_cast<double *>(static_cast<char *>(ws) + (size_t)h * half);
    };
    const double est = sweep_seconds(pl, order);
    if (est >= kTwoStreamSweep && est / order < kTwoStreamModeMax) {
        // A long sweep alternates between the caller's stream and a second
        // one, so that one mode's last workgroups, its split reduction and
        // the next mode's first workgroups run side by side.  Each stream has
        // its own half of the workspace.
        hipStream_t side = nullptr;
        if (side_stream(&side) != hipSuccess) return MTTKRP_EHIP;
        hipEvent_t fork = nullptr, join = nullptr;
        if (hipEventCreateWithFlags(&fork, hipEventDisableTiming) != hipSuccess) return MTTKRP_EHIP;
        if (hipEventCreateWithFlags(&join, hipEventDisableTiming) != hipSuccess) {
            (void)hipEventDestroy(fork);
            return MTTKRP_EHIP;
        }
        // The second stream starts after the work already on the caller's
        // stream, and the caller's stream continues after both.
        hipError_t e = hipEventRecord(fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(side, fork, 0);
        for (int m = 0; m < order && e == hipSuccess; ++m) {
            const int lane = m & 1;
            pl[m].kp.partial = in_half(lane);
            e = launch_mttkrp<T>(pl[m], lane ? side : s, true);
        }
        if (e == hipSuccess) e = hipEventRecord(join, side);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, join, 0);
        (void)hipEventDestroy(fork);
        (void)hipEventDestroy(join);
        return e == hipSuccess ? MTTKRP_OK : MTTKRP_EHIP;
    }
    // A short sweep stays on the caller's stream, the modes with a plain split
    // first.  A split mode launches no reduction of its own: the next
    // launch's tile kernel adds its partial sums in split_reduce_kernel's
    // order (so the results do not change and a launch per split mode is
    // saved), while writing its own partials, if any, to the other half of
    // the workspace.  Only the last launch, when it splits, keeps its
    // reduction kernel.
    int ord[kMaxOrder];
    int no = 0;
    for (int m = 0; m < order; ++m)
        if (plain_split(pl[m])) ord[no++] = m;
    for (int m = 0; m < order; ++m)
        if (!plain_split(pl[m])) ord[no++] = m;
    // Consecutive form-1 modes that share their B tile and decomposition and
    // write no partials run as the passes of one multi-mode launch.
    int prev = -1;  // split mode whose partials are pending
    int prev_half = 0;
    for (int i = 0; i < order;) {
        Plan &cur = pl[ord[i]];
        const int h = prev >= 0 ? 1 - prev_half : 0;
        cur.kp.partial = in_half(h);
        if (prev >= 0) {
            const KParams &a = pl[prev].kp;
            cur.kp.pend_partial = a.partial;
            cur.kp.pend_nsplit = a.nsplit;
            cur.kp.pend_count = a.In * a.R;
            cur.kp.pend_out = a.out;
            cur.kp.pend_ng = a.nsplit >= 32 ? 16 : 4;
        }
        const Plan *grp[kMaxPasses] = {&cur};
        int np = 1;
        while (np < kMaxPasses && i + np < order && fusable(cur, pl[ord[i + np]])) {
            grp[np] = &pl[ord[i + np]];
            ++np;
        }
        if (np > 1) {
            if (launch_mttkrp_multi<T>(grp, np, s) != hipSuccess) return MTTKRP_EHIP;
            prev = -1;
            i += np;
            continue;
        }
        const bool hand_on = plain_split(cur) && i + 1 < order;
        if (launch_mttkrp<T>(cur, s, !hand_on) != hipSuccess) return MTTKRP_EHIP;
        prev = hand_on ? ord[i] : -1;
        prev_half = h;
        ++i;
    }
    return MTTKRP_OK;
}

// CP-ALS workspace layout (bytes, each piece 256-aligned):
//   [mttkrp partials][M fp64 maxI x R][Unew fp64 maxI x R][G fp64 d x R x R]
//   [L fp64 R x R][lambda fp64 R][sumsq partials][scalars: ||X||^2, fit][flag]
struct AlsLayout {
    size_t mt, M, Unew, G, L, W, Z, CI, YI, YM, lam, parts, scal, flag, total;
};

int als_layout(const int64_t *dims, int order, int64_t rank, int elem, AlsLayout &L)
{
    size_t mt = 0;
    int st = mode_ws_max(dims, order, rank, elem, &mt);
    if (st) return st;
    int64_t maxI = 0;
    for (int m = 0; m < order; ++m) maxI = std::max<int64_t>(maxI, dims[m]);
    const size_t R = (size_t)rank;
    size_t off = 0;
    L.mt = off;
    off += round256(mt);
    L.M = off;
    off += round256(8 * (size_t)maxI * R);
    L.Unew = off;
    off += round256(8 * (size_t)maxI * R);
    L.G = off;
    off += round256(8 * (size_t)order * R * R);
    L.L = off;
    off += round256(8 * R * R);
    // inverses of the blocked factor's diagonal blocks (R > 64, R x 64), or
    // the last mode's V for the fit (R <= 64, R x R)
    L.W = off;
    off += round256(8 * R * 64);
    // the blocked update (R > 64): Z_k, the identity rows, L^{-T}, M L^{-T}
    const bool blocked = rank > 64;
    L.Z = off;
    off += blocked ? round256(8 * 2 * 64 * 64) : 0;
    L.CI = off;
    off += blocked ? round256(8 * R * R) : 0;
    L.YI = off;
    off += blocked ? round256(8 * R * R) : 0;
    L.YM = off;
    off += blocked ? round256(8 * (size_t)maxI * R) : 0;
    L.lam = off;
    off += round256(8 * R);
    L.parts = off;
    off += round256(8 * (size_t)kSumsqParts);
    L.scal = off;
    off += 256;
    L.flag = off;
    off += 256;
    L.total = off;
    return MTTKRP_OK;
}

template <typename T>
int cp_als_entry(const T *X, const int64_t *dims, int order, int64_t rank, T *const *factors,
                 T *lambda, int iters, double tol, double *fit_hist, int *iters_done, void *ws,
                 size_t ws_bytes, void *stream_)
{
    if (!X || !dims || !factors || !lambda || !fit_hist || !iters_done) return MTTKRP_EINVAL;
    if (order < 3 || order > kMaxOrder) return MTTKRP_EORDER;
    if (rank < 1 || iters < 0) return MTTKRP_EINVAL;
    for (int m = 0; m < order; ++m) {
        if (dims[m] < 1 || !factors[m]) return MTTKRP_EINVAL;
    }
    if (!aligned16(X) || !aligned16(lambda) || (ws && !aligned16(ws))) return MTTKRP_EALIGN;
    for (int m = 0; m < order; ++m)
        if (!aligned16(factors[m])) return MTTKRP_EALIGN;
    if (rank > 4096) return MTTKRP_ERANGE;  // R x R work (blocked factor, Grams) kept to 4096
    AlsLayout L;
    int st = als_layout(dims, order, rank, (int)sizeof(T), L);
    if (st) return st;
    if (L.total > ws_bytes) return MTTKRP_EWORKSPACE;
    if (!ws) return MTTKRP_EINVAL;

    hipStream_t s = reinterpret_cast<hipStream_t>(stream_);
    unsigned char *w = reinterpret_cast<unsigned char *>(ws);
    double *M = reinterpret_cast<double *>(w + L.M);
    double *Unew = reinterpret_cast<double *>(w + L.Unew);
    double *G = reinterpret_cast<double *>(w + L.G);
    double *Lc = reinterpret_cast<double *>(w + L.L);
    double *Winv = reinterpret_cast<double *>(w + L.W);
    double *Zk = reinterpret_cast<double *>(w + L.Z);
    double *CI = reinterpret_cast<double *>(w + L.CI);
    double *YI = reinterpret_cast<double *>(w + L.YI);
    double *YM = reinterpret_cast<double *>(w + L.YM);
    double *lam64 = reinterpret_cast<double *>(w + L.lam);
    double *parts = reinterpret_cast<double *>(w + L.parts);
    double *scal = reinterpret_cast<double *>(w + L.scal);
    int *flag = reinterpret_cast<int *>(w + L.flag);
    const int64_t R = rank;

    for (int it = 0; it < iters; ++it) fit_hist[it] = std::numeric_limits<double>::quiet_NaN();
    *iters_done = 0;

    int64_t N = 1;
    for (int m = 0; m < order; ++m) N *= dims[m];
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    // the flag block: the failure word, then at 32, 64 and 96 bytes on the
    // caller's stream's sequence word, the side kernel's ticket counter and
    // the side stream's sequence word (all zero at the start of a run)
    if (!ok(launch_fill<int>(flag, 32, 0, s))) return MTTKRP_EHIP;
    unsigned *ticket = reinterpret_cast<unsigned *>(flag + 16);
    if (!ok(launch_fill<T>(lambda, R, T(1), s))) return MTTKRP_EHIP;
    if (!ok(launch_sumsq<T>(X, N, parts, kSumsqParts, scal, s))) return MTTKRP_EHIP;
    if (!ok(launch_gram_all<T>(factors, dims, order, R, G, flag, s))) return MTTKRP_EHIP;

    // Each sweep's fit and flag land in host-visible pinned memory (two
    // slots, written at the end of the sweep).  The host polls sweep it - 1's
    // slot only after sweep it is queued, so the device never waits for the
    // host; a sweep queued past a stop (convergence or a failed Cholesky)
    // changes nothing, since its kernels see the flag and return.
    FitSlot *slots = fit_slots();
    if (!slots) return MTTKRP_EHIP;
    for (int j = 0; j < 2; ++j) __atomic_store_n(&slots[j].seq, 0u, __ATOMIC_RELEASE);
    // On every return the caller's stream is drained: queued kernels may still
    // write the slots, which the thread's next call reuses.
    struct Drain {
        hipStream_t s;
        ~Drain() { (void)hipStreamSynchronize(s); }
    } drain{s};

    // Modes with R <= 64 whose I x R solution fits in LDS split their update:
    // V, its Cholesky factor and V^{-1} (which do not depend on the MTTKRP)
    // run on a second stream beside the mode's MTTKRP; the rest (U = M V^{-1},
    // norms, Gram, and after the sweep's last mode the fit) follows the
    // MTTKRP on the caller's stream.  V^{-1} lives in the L
    // buffer: the next side kernel waits for this mode's update.  The streams are ordered by
    // two sequence words in the flag block, not by events (an event record
    // and a stream wait each held the caller's stream for several
    // microseconds per mode):
    //  - seq_main: the apply kernel of sweep it, mode n stores
    //    it * (order + 1) + n + 1, and the end of the sweep (the fit kernel, or
    //    the last mode's apply when it forms the fit) it * (order + 1) +
    //    order + 1;
    //  - seq_side: the side kernel of sweep it, mode n stores the same value
    //    as that mode's apply.
    // A side kernel waits for seq_main to reach the value before its own (the
    // previous mode's apply, or the end of the previous sweep, which has then
    // set the stop flag if it stops); an apply waits for seq_side to reach its
    // own.  When the previous update on the caller's stream stores no word
    // (an unsplit mode, or the start of the run), an event orders the side
    // kernel instead.  Every kernel waits only for one queued before it.
    auto split_mode = [&](int n) { return R <= 64 && apply_small_lds(dims[n], R) != 0; };
    unsigned *seq_main = reinterpret_cast<unsigned *>(flag + 8);
    unsigned *seq_side = reinterpret_cast<unsigned *>(flag + 24);
    struct Side {
        hipStream_t main = nullptr, side = nullptr;
        hipEvent_t fork = nullptr, join = nullptr;
        bool live = false;  // side kernels queued since the last join
        // the caller's stream waits for every side kernel queued so far
        hipError_t join_now()
        {
            if (!live) return hipSuccess;
            live = false;
            hipError_t e = hipEventRecord(join, side);
            if (e == hipSuccess) e = hipStreamWaitEvent(main, join, 0);
            return e;
        }
        ~Side()
        {
            (void)join_now();
            if (fork) (void)hipEventDestroy(fork);
            if (join) (void)hipEventDestroy(join);
        }
    } sd;
    sd.main = s;
    bool any_split = false;
    for (int m = 0; m < order; ++m) any_split = any_split || split_mode(m);
    if (any_split && iters > 0) {
        if (side_stream(&sd.side) != hipSuccess) return MTTKRP_EHIP;
        if (!ok(hipEventCreateWithFlags(&sd.fork, hipEventDisableTiming))) return MTTKRP_EHIP;
        if (!ok(hipEventCreateWithFlags(&sd.join, hipEventDisableTiming))) return MTTKRP_EHIP;
    }

    // Outcome of sweep k: 1 = go on, 0 = stopped after it (converged), or an
    // error status.  The slot's sweep number is polled; every so often the
    // stream is queried, so that a stream that failed or went idle without
    // the store ends the wait.
    auto consume = [&](int k) -> int {
        FitSlot *h = slots + (k & 1);
        const unsigned want = (unsigned)k + 1u;
        for (unsigned spin = 1;; ++spin) {
            if (__atomic_load_n(&h->seq, __ATOMIC_ACQUIRE) == want) break;
            if ((spin & 255u) == 0u) {
                const hipError_t q = hipStreamQuery(s);
                if (q == hipSuccess) {
                    if (__atomic_load_n(&h->seq, __ATOMIC_ACQUIRE) == want) break;
                    return MTTKRP_EHIP;
                }
                if (q != hipErrorNotReady) return MTTKRP_EHIP;
            }
            __builtin_ia32_pause();
        }
        const int f = __atomic_load_n(&h->flag, __ATOMIC_RELAXED);
        if (f == 1 || f == 3) {
            *iters_done = k;
            // 3: a wait between the two streams timed out
            return f == 1 ? MTTKRP_ENOTSPD : MTTKRP_EHIP;
        }
        double fit = 0.0;
        __atomic_load(&h->fit, &fit, __ATOMIC_RELAXED);
        fit_hist[k] = fit;
        *iters_done = k + 1;
        return f == 2 ? 0 : 1;
    };
    auto finish = [&](int r) -> int {
        // later sweeps may still be queued (their kernels return at once)
        if (!ok(sd.join_now())) return MTTKRP_EHIP;
        if (!ok(hipStreamSynchronize(s))) return MTTKRP_EHIP;
        return r;
    };

    const T *cf[kMaxOrder];
    for (int m = 0; m < order; ++m) cf[m] = factors[m];
    bool main_stored = false;  // the last update queued on s stores seq_main
    for (int it = 0; it < iters; ++it) {
        const unsigned base = (unsigned)it * (unsigned)(order + 1);
        const unsigned v_end = base + (unsigned)order + 1u;
        FitSlot *slot = slots + (it & 1);
        const AlsFitOut fo{Winv,       G,           order,      scal,      tol, it > 0 ? 1 : 0,
                           &slot->fit, &slot->flag, &slot->seq, (unsigned)it + 1u};
        bool fit_done = false;
        for (int n = 0; n < order; ++n) {
            const bool split = split_mode(n);
            const unsigned v = base + (unsigned)n + 1u;
            if (split) {
                const unsigned *wait_on = nullptr;
                if (main_stored) {
                    wait_on = seq_main;
                } else {
                    if (!ok(hipEventRecord(sd.fork, s))) return MTTKRP_EHIP;
                    if (!ok(hipStreamWaitEvent(sd.side, sd.fork, 0))) return MTTKRP_EHIP;
                }
                // the last mode's side kernel also keeps V for the fit
                if (!ok(launch_side_chol(G, order, n, R, Lc, n == order - 1 ? Winv : nullptr,
                                         flag, ticket, wait_on, v - 1u, seq_side, v, sd.side)))
                    return MTTKRP_EHIP;
                sd.live = true;
            }
            st = mttkrp_one<T>(X, dims, order, cf, R, n, M, 1, w + L.mt, L.M - L.mt, s);
            if (st) return st;
            if (split) {
                // the sweep's last mode also forms the fit.  (The Gram stays
                // here: formed by the next side kernel from the stored
                // factor, it made that kernel outlast the MTTKRP it hides
                // under, and the side kernel after it then took a compute
                // unit that the next MTTKRP's grid needed.)
                const bool last = n == order - 1;
                if (!ok(launch_apply_small<T>(M, dims[n], R, Lc, factors[n], lam64, lambda,
                                              G + (size_t)n * R * R, flag, seq_side, v, seq_main,
                                              last ? v_end : v, last ? &fo : nullptr, s)))
                    return MTTKRP_EHIP;
                main_stored = true;
                fit_done = last;
                continue;
            }
            main_stored = false;
            if (update_small_lds(dims[n], R)) {
                // Cholesky, solve, normalization and Gram refresh in one
                // workgroup
                if (!ok(launch_update_small<T>(G, order, n, M, dims[n], R, factors[n], lam64,
                                               lambda, G + (size_t)n * R * R, flag, s)))
                    return MTTKRP_EHIP;
                continue;
            }
            if (R <= 64) {
                if (!ok(launch_chol(G, order, n, R, Lc, flag, s))) return MTTKRP_EHIP;
                if (!ok(launch_solve(M, Lc, dims[n], R, Unew, flag, s))) return MTTKRP_EHIP;
            } else {
                // 64-wide column blocks: per block the diagonal block's
                // factor and inverse by one workgroup, then one launch of
                // tiled products for the panels and trailing updates of V, M
                // and the identity
                if (!ok(launch_update_blocked(G, order, n, R, M, dims[n], Lc, CI, Unew, YI, YM,
                                              Winv, Zk, flag, s)))
                    return MTTKRP_EHIP;
            }
            if (!ok(launch_normalize<T>(Unew, dims[n], R, factors[n], lam64, lambda, flag, s)))
                return MTTKRP_EHIP;
            if (!ok(launch_gram<T>(factors[n], dims[n], R, G + (size_t)n * R * R, flag, s)))
                return MTTKRP_EHIP;
        }
        if (!fit_done) {
            if (!ok(launch_fit<T>(M, factors[order - 1], dims[order - 1], lam64, R, flag, fo,
                                  parts, kSumsqParts, Unew, seq_main, v_end, s)))
                return MTTKRP_EHIP;
            main_stored = true;
        }
        if (it > 0) {
            const int r = consume(it - 1);
            if (r != 1) return finish(r);
        }
    }
    if (iters > 0) {
        const int r = consume(iters - 1);
        if (r != 1) return finish(r);
    }
    return MTTKRP_OK;
}

}  // namespace
}  // namespace mttkrp

using namespace mttkrp;

extern "C" {

const char *mttkrp_strerror(int status)
{
    switch (status) {
    case MTTKRP_OK: return "success";
    case MTTKRP_EINVAL: return "invalid argument (null pointer, non-positive size, mode out of range)";
    case MTTKRP_EORDER: return "tensor order must be 3, 4 or 5";
    case MTTKRP_ERANGE: return "problem size exceeds the supported index range";
    case MTTKRP_EALIGN: return "device pointer not 16-byte aligned";
    case MTTKRP_EWORKSPACE: return "workspace smaller than the size the query returns";
    case MTTKRP_EHIP: return "HIP runtime call or kernel launch failed";
    case MTTKRP_ENOTSPD: return "CP-ALS: Cholesky pivot of the R x R system not positive";
    case MTTKRP_ESCRATCH:
        return "the plan needs more partial-sum space than the no-allocation entry point's "
               "fixed scratch array holds";
    default: return "unknown status";
    }
}

int mttkrp_version(void) { return 100; }

int mttkrp_selftest(void)
{
    // Divisors: every value up to 4096, powers of two and their neighbours,
    // and values near 2^31; dividends: the edges around multiples of the
    // divisor, the top of the range and a fixed linear-congruential sample.
    std::vector<int64_t> ds;
    for (int64_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (int k = 12; k <= 30; ++k)
        for (int64_t e = -1; e <= 1; ++e) ds.push_back((INT64_C(1) << k) + e);
    for (int64_t d : {INT64_C(2147483647), INT64_C(2147483646), INT64_C(2147483629), INT64_C(1000000007),
                      INT64_C(65537), INT64_C(46341), INT64_C(99991)})
        ds.push_back(d);
    uint64_t lcg = 0x9e3779b97f4a7c15ull;
    int64_t idx = 0;
    for (int64_t d : ds) {
        const mttkrp::FastDiv f = mttkrp::make_fastdiv(d);
        std::vector<uint32_t> xs = {0u, 1u, 2u, 0x7fffffffu, 0x7ffffffeu};
        for (int64_t k : {INT64_C(1), INT64_C(2), INT64_C(3), INT64_C(1000), (INT64_C(0x7fffffff) / d)}) {
            const int64_t base = k * d;
            for (int64_t e = -1; e <= 1; ++e)
                if (base + e >= 0 && base + e < (INT64_C(1) << 31)) xs.push_back((uint32_t)(base + e));
        }
        for (int j = 0; j < 64; ++j) {
            lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
            xs.push_back((uint32_t)(lcg >> 33));
        }
        for (uint32_t x : xs) {
            ++idx;
            if (mttkrp::fdiv(x, f) != (uint32_t)(x / (uint64_t)d)) return (int)std::min<int64_t>(idx, INT32_MAX);
        }
    }
    return 0;
}

int mttkrp_workspace_bytes(const int64_t *dims, int order, int64_t rank, int mode, int elem_bytes,
                           size_t *bytes)
{
    if (!bytes) return MTTKRP_EINVAL;
    Plan pl;
    const int st = make_plan(dims, order, rank, mode, elem_bytes, pl);
    if (st) return st;
    *bytes = pl.ws_bytes;
    return MTTKRP_OK;
}

int mttkrp_all_workspace_bytes(const int64_t *dims, int order, int64_t rank, int elem_bytes,
                               size_t *bytes)
{
    if (!bytes || !dims) return MTTKRP_EINVAL;
    if (order < 3 || order > kMaxOrder) return MTTKRP_EORDER;
    if (elem_bytes != 4 && elem_bytes != 8) return MTTKRP_EINVAL;
    return all_ws(dims, order, rank, elem_bytes, bytes);
}

int cp_als_workspace_bytes(const int64_t *dims, int order, int64_t rank, int elem_bytes,
                           size_t *bytes)
{
    if (!bytes || !dims) return MTTKRP_EINVAL;
    if (order < 3 || order > kMaxOrder) return MTTKRP_EORDER;
    if (elem_bytes != 4 && elem_bytes != 8) return MTTKRP_EINVAL;
    if (rank > 4096) return MTTKRP_ERANGE;
    AlsLayout L;
    const int st = als_layout(dims, order, rank, elem_bytes, L);
    if (st) return st;
    *bytes = L.total;
    return MTTKRP_OK;
}

int mttkrp_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
               int64_t rank, int mode, double *out, void *ws, size_t ws_bytes, void *stream)
{
    return mttkrp_entry<double>(X, dims, order, factors, rank, mode, out, ws, ws_bytes, stream);
}

int mttkrp_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
               int64_t rank, int mode, float *out, void *ws, size_t ws_bytes, void *stream)
{
    return mttkrp_entry<float>(X, dims, order, factors, rank, mode, out, ws, ws_bytes, stream);
}

int mttkrp_all_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
                   int64_t rank, double *const *outs, void *ws, size_t ws_bytes, void *stream)
{
    return mttkrp_all_entry<double>(X, dims, order, factors, rank, outs, ws, ws_bytes, stream);
}

int mttkrp_all_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                   int64_t rank, float *const *outs, void *ws, size_t ws_bytes, void *stream)
{
    return mttkrp_all_entry<float>(X, dims, order, factors, rank, outs, ws, ws_bytes, stream);
}

int cp_als_f64(const double *X, const int64_t *dims, int order, int64_t rank,
               double *const *factors, double *lambda, int iters, double tol, double *fit_hist,
               int *iters_done, void *ws, size_t ws_bytes, void *stream)
{
    return cp_als_entry<double>(X, dims, order, rank, factors, lambda, iters, tol, fit_hist,
                                iters_done, ws, ws_bytes, stream);
}

int cp_als_f32(const float *X, const int64_t *dims, int order, int64_t rank, float *const *factors,
               float *lambda, int iters, double tol, double *fit_hist, int *iters_done, void *ws,
               size_t ws_bytes, void *stream)
{
    return cp_als_entry<float>(X, dims, order, rank, factors, lambda, iters, tol, fit_hist,
                               iters_done, ws, ws_bytes, stream);
}

int mttkrp_plan(const int64_t *dims, int order, int64_t rank, int mode, int elem_bytes,
                mttkrp_plan_info *info)
{
    if (!info) return MTTKRP_EINVAL;
    Plan pl;
    const int st = make_plan(dims, order, rank, mode, elem_bytes, pl);
    if (st) return st;
    std::memset(info, 0, sizeof(*info));
    info->form = pl.form;
    info->layout = pl.layout;
    info->k_modes[0] = pl.k_modes[0];
    info->k_modes[1] = pl.k_modes[1];
    info->row_modes[0] = pl.row_modes[0];
    info->row_modes[1] = pl.row_modes[1];
    for (int j = 0; j < 3; ++j) info->outer_modes[j] = pl.outer_modes[j];
    info->mb = pl.mb;
    info->nb = pl.nb;
    info->b_in_lds = pl.b_in_lds ? 1 : 0;
    info->vec = pl.vec ? 1 : 0;
    info->k_len = pl.kp.K;
    info->rows = pl.kp.nrows;
    info->batches = pl.kp.nbatch;
    info->splits = pl.kp.nsplit;
    info->rtiles = pl.kp.nrtiles;
    info->grid = pl.grid;
    info->lds_bytes = pl.lds_bytes;
    info->ws_bytes = pl.ws_bytes;
    info->kchunks = pl.kp.nkch;
    info->waves = pl.waves;
    info->launchable = plan_launchable(pl) ? 1 : 0;
    const PlanModel pm = plan_model(pl, dims, order, mode);
    info->model_flop_s = pm.flop_s;
    info->model_hbm_s = pm.hbm_s;
    info->model_l2_s = pm.l2_s;
    info->model_lds_s = pm.lds_s;
    info->model_s = pm.t_s;
    info->t_inf_s = pm.t_inf_s;
    info->t_0_s = pm.t_0_s;
    return MTTKRP_OK;
}

}  // extern "C"
