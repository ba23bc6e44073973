// Launchers of the CP-ALS kernels (als_kernels.hip), called by the CP-ALS
// driver in capi.cpp.  Every launcher enqueues on the given stream and
// returns the launch status; none allocates memory.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstddef>

namespace mttkrp {

// Where the end of a sweep goes: the fit, the stop decision and the
// host-visible slot (fit, failure word, then the sweep's number, stored last
// with a system-scope release so that the host can poll it).
struct AlsFitOut {
    const double *V;     // (split update) the Hadamard product of the other Grams, R x R
    const double *Gall;  // the Grams of every mode, R x R each
    int order;
    double *scal;        // [0] ||X||^2 in, [1] fit out, [2] the previous fit
    double tol;          // stop when the fit changes by less (0: never)
    int have_prev;       // scal[2] holds a previous sweep's fit
    double *out_fit;
    int *out_flag;
    unsigned *out_seq;
    unsigned seq_val;
};

template <typename T>
hipError_t launch_sumsq(const T *X, int64_t N, double *partial, int nparts, double *out,
                        hipStream_t s);
template <typename T>
hipError_t launch_gram(const T *U, int64_t I, int64_t R, double *G, const int *flag, hipStream_t s);
// The Grams of every mode (G + m * R * R for mode m), in one launch for R <= 64.
template <typename T>
hipError_t launch_gram_all(const T *const *U, const int64_t *dims, int order, int64_t R, double *G,
                           const int *flag, hipStream_t s);
// R > 64: U_new = M V^{-1} into CM by 64-wide column blocks (CV, CI, YI: R x R;
// CM, YM: I x R; W: R x 64; Z: 2 x 64 x 64 -- all workspace).
hipError_t launch_update_blocked(const double *Gall, int order, int n, int64_t R, const double *M,
                                 int64_t I, double *CV, double *CI, double *CM, double *YI,
                                 double *YM, double *W, double *Z, int *flag, hipStream_t s);
hipError_t launch_chol(const double *Gall, int order, int n, int64_t R, double *L, int *flag,
                       hipStream_t s);
hipError_t launch_solve(const double *M, const double *L, int64_t I, int64_t R, double *Unew,
                        const int *flag, hipStream_t s);
template <typename T>
hipError_t launch_normalize(const double *Unew, int64_t I, int64_t R, T *Uout, double *lam64,
                            T *lamT, const int *flag, hipStream_t s);
template <typename T>
hipError_t launch_fill(T *p, int64_t n, T v, hipStream_t s);
size_t update_small_lds(int64_t I, int64_t R);
size_t apply_small_lds(int64_t I, int64_t R);
// The split update's side kernel (V, its Cholesky factor and V^{-1} into
// Vinv; with Vout non-null V itself too, for the fit) and apply kernel (U = M V^{-1}, norms, Gram; with fit non-null also
// the end of the sweep).  Each waits until *wait_on reaches wait_for (none if
// wait_on is null) and stores done_val to *done when finished.
hipError_t launch_side_chol(const double *Gall, int order, int n, int64_t R, double *Vinv,
                            double *Vout, int *flag, unsigned *ticket, const unsigned *wait_on,
                            unsigned wait_for, unsigned *done, unsigned done_val, hipStream_t s);
template <typename T>
hipError_t launch_apply_small(const double *M, int64_t I, int64_t R, const double *Vinv, T *Uout,
                              double *lam64, T *lamT, double *G, int *flag,
                              const unsigned *wait_on, unsigned wait_for, unsigned *done,
                              unsigned done_val, const AlsFitOut *fit, hipStream_t s);
template <typename T>
hipError_t launch_update_small(const double *Gall, int order, int n, const double *M, int64_t I,
                               int64_t R, T *Uout, double *lam64, T *lamT, double *G, int *flag,
                               hipStream_t s);
// The fit kernel (after a last mode whose update is not the split one).
template <typename T>
hipError_t launch_fit(const double *M, const T *Ulast, int64_t Ilast, const double *lam64,
                      int64_t R, int *flag, const AlsFitOut &fit, double *parts, int max_parts,
                      double *colsum_buf, unsigned *done, unsigned done_val, hipStream_t s);

}  // namespace mttkrp
