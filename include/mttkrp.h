/*
 * mttkrp.h -- C ABI of the matrix-free dense MTTKRP library for MI355X (gfx950).
 *
 * The operation ("A Performance Portable Matrix Free Dense MTTKRP in GenTen",
 * abstract and TL;DR): the matricized tensor times Khatri-Rao product, the
 * workhorse kernel of CP decompositions.  For mode n of a d-way dense tensor X
 * with factor matrices U_m (I_m x R),
 *
 *     M(i_n, r) = sum over every i_m, m != n, of  X(i_0..i_{d-1}) * prod_{m != n} U_m(i_m, r),
 *
 * i.e. X_(n) times the Khatri-Rao product of the other factors, with the mode-n
 * unfolding of "An HPC Approach to Accelerate Tensor Decompositions", Sec. 2.
 * The Khatri-Rao matrix is never formed: extra device memory grows like
 * R * sum(I_m), never like R * prod(I_m) (GenTen page, TL;DR).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Pointers   X, factors[m], out, outs[m], lambda and ws point to DEVICE memory.
 *             dims, the factors/outs pointer arrays, fit_hist, iters_done and
 *             info point to HOST memory that is read or written during the call
 *             only.  The library keeps no pointer after it returns.
 *  Layout     X is row-major (C order) over dims: the last mode has unit stride.
 *             U_m is I_m x R row-major.  out is I_n x R row-major.  A column-major
 *             caller passes reversed dims, a reversed factor list and
 *             mode' = order - 1 - mode.
 *  Modes      0-based: mode in [0, order).  order in [3, 5].
 *  Semantics  out is overwritten.  factors[mode] is not read (may be NULL).
 *             out must not alias X, a factor or ws.
 *  Ownership  The caller allocates and frees every buffer, including the
 *             workspace ws, whose size the *_workspace_bytes queries return.
 *             The library allocates no device memory.
 *  Alignment  every device pointer must be 16-byte aligned (EALIGN otherwise).
 *  Streams    `stream` is a hipStream_t (NULL: the default stream).  mttkrp*
 *             calls only enqueue work and return; cp_als* synchronise the
 *             stream once per sweep to read back the fit.
 *  Errors     every argument is checked on the host before any HIP call; a bad
 *             argument returns its code and touches nothing.  A launch failure
 *             returns MTTKRP_EHIP.  A fault during execution surfaces at the
 *             caller's next synchronisation.  Nothing is printed.
 *  Threads    calls are reentrant; calls that share a ws buffer must not overlap.
 */
#ifndef MTTKRP_AMD_MTTKRP_H
#define MTTKRP_AMD_MTTKRP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define MTTKRP_OK 0
#define MTTKRP_EINVAL (-1)     /* null pointer, dims[m] < 1, rank < 1, mode out of range, iters < 0 */
#define MTTKRP_EORDER (-2)     /* order not in [3, 5] */
#define MTTKRP_ERANGE (-3)     /* a size overflows int64 or exceeds the library's index range */
#define MTTKRP_EALIGN (-4)     /* a device pointer is not 16-byte aligned */
#define MTTKRP_EWORKSPACE (-5) /* ws_bytes smaller than the size the query returns */
#define MTTKRP_EHIP (-6)       /* a HIP runtime call or kernel launch failed */
#define MTTKRP_ENOTSPD (-7)    /* CP-ALS: a Cholesky pivot of the R x R system was not positive */
#define MTTKRP_ESCRATCH (-8)   /* mttkrp_noalloc: the plan needs more than MTTKRP_NOALLOC_SCRATCH_BYTES */

/* Text for a status code (static storage; never NULL). */
const char *mttkrp_strerror(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mttkrp_version(void);

/* Host-only self-check of the integer helpers the kernels rely on: the
 * multiply-high division constants the planner computes for the index decode
 * ("Division by Invariant Integers using Multiplication", Granlund and
 * Montgomery, Sec. 4) are checked against plain division over a fixed set of
 * divisors in [1, 2^31) and dividends in [0, 2^31).  Needs no GPU.  Returns 0,
 * or 1 + the index of the first failing (divisor, dividend) pair. */
int mttkrp_selftest(void);

/* ---- workspace queries ----
 * Write to *bytes the device workspace the matching call needs (0 is possible)
 * for elem_bytes = 8 (fp64) or 4 (fp32).  It holds fp64 partial sums of the
 * kernel's output rows from independent chunks of the work (at most
 * max(1024, contraction chunks) of them).  The kernel's rows are the I_n
 * output rows, or, when the output mode is a short unit-stride mode, the
 * block of the last two modes (I_{d-2} * I_{d-1} rows with I_{d-1} < 64).  So
 * the workspace grows like R * I_n (or R * 64 * I_{d-2}) and never with the
 * Khatri-Rao size R * prod_{m != n} I_m.  The all-mode call needs twice the
 * largest mode's workspace: it holds one mode's partials while the next mode
 * writes its own. */
int mttkrp_workspace_bytes(const int64_t *dims, int order, int64_t rank, int mode,
                           int elem_bytes, size_t *bytes);
int mttkrp_all_workspace_bytes(const int64_t *dims, int order, int64_t rank, int elem_bytes,
                               size_t *bytes);
int cp_als_workspace_bytes(const int64_t *dims, int order, int64_t rank, int elem_bytes,
                           size_t *bytes);

/* ---- MTTKRP of one mode ----
 * out (I_mode x R) = X_(mode) times the Khatri-Rao product of every other factor.
 * fp64: arithmetic in fp64.  fp32: fp32 products; the matrix cores sum in
 * fp32 over at most one contraction chunk (the part of the contracted mode(s)
 * whose Khatri-Rao tile fits in LDS: at most 1,840 terms, 288 at the 4-way
 * benchmark tensors), and every longer sum is in fp64; out is rounded to
 * fp32 once.  The expected relative error of a chunk's fp32 sum is about
 * 2^-24 * sqrt(chunk), below 3e-6. */
int mttkrp_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
               int64_t rank, int mode, double *out, void *ws, size_t ws_bytes, void *stream);
int mttkrp_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
               int64_t rank, int mode, float *out, void *ws, size_t ws_bytes, void *stream);

/* ---- MTTKRP of one mode without any allocation ----
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * computation, kernels and result, bit for bit, as mttkrp_f64 (elem_bytes =
 * 8) or mttkrp_f32 (elem_bytes = 4), with X, factors and out as there, but
 * no workspace argument.  The split partial sums go to a scratch array of
 * MTTKRP_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU, from the first call on that GPU until the process ends.  The call
 * allocates nothing (no hipMalloc, no hipFree, no allocating library call).
 * A plan that needs more partial-sum space than the array holds (the size
 * mttkrp_workspace_bytes reports) is refused with MTTKRP_ESCRATCH before any
 * HIP call.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (on different streams, or from different host threads)
 * race and must be serialised by the caller.  Each call rewrites every
 * partial it reads, so nothing is carried over from an earlier call. */
#define MTTKRP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mttkrp_noalloc(const void *X, const int64_t *dims, int order, const void *const *factors,
                   int64_t rank, int mode, void *out, int elem_bytes, void *stream);

/* ---- MTTKRP of every mode (the all-mode sweep of the GenTen page, Fig. 4) ----
 * outs[m] (I_m x R) for m = 0..order-1, in mode order, on one stream.  X is
 * read once per mode. */
int mttkrp_all_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
                   int64_t rank, double *const *outs, void *ws, size_t ws_bytes, void *stream);
int mttkrp_all_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                   int64_t rank, float *const *outs, void *ws, size_t ws_bytes, void *stream);

/* ---- CP-ALS driver (GenTen page, Fig. 5: MTTKRP plus inner product and
 * Cholesky solve per step) ----
 * Gauss-Seidel sweeps over the modes.  For mode n: V = Hadamard of the Grams
 * U_m^T U_m (m != n); M = MTTKRP_n; V = L L^T (Cholesky, no pivoting);
 * U_n <- M V^{-1}; lambda_r = ||U_n(:, r)||_2; columns with lambda_r > 0 are
 * scaled to unit norm.  After the last mode the fit
 *     1 - sqrt(max(0, ||X||^2 + ||model||^2 - 2 <X, model>)) / ||X||
 * is read back to fit_hist[it] (HOST, length iters; NaN past the last sweep
 * run).  factors: in = initial factors, out = final factors (DEVICE).
 * lambda: DEVICE, length R.  tol > 0 stops after the first sweep whose fit
 * changed by less than tol; tol <= 0 runs exactly iters sweeps.
 * *iters_done (HOST) = sweeps run.  A non-positive Cholesky pivot stops the
 * run with MTTKRP_ENOTSPD; the factors then hold the values of the failing
 * step's start.  The R x R solve runs in fp64 for both element types. */
int cp_als_f64(const double *X, const int64_t *dims, int order, int64_t rank,
               double *const *factors, double *lambda, int iters, double tol, double *fit_hist,
               int *iters_done, void *ws, size_t ws_bytes, void *stream);
int cp_als_f32(const float *X, const int64_t *dims, int order, int64_t rank,
               float *const *factors, float *lambda, int iters, double tol, double *fit_hist,
               int *iters_done, void *ws, size_t ws_bytes, void *stream);

/* ---- ablation baselines (comparison only, not the product path) ----
 * The untiled matrix-free strategies the GenTen page improves on (its
 * MTTKRP-ELEM and MTTKRP-SLICE).  Same arguments and result as mttkrp_*, no
 * workspace.  ELEM: one thread per tensor element, one atomic addition per
 * output entry it touches (out is zeroed first; the order of the additions,
 * hence the rounding, is not fixed).  SLICE: one workgroup per output row,
 * partial sums added in a fixed order.  Both compute in the element type. */
int mttkrp_elem_f64(const double *X, const int64_t *dims, int order, const double *const *factors,
                    int64_t rank, int mode, double *out, void *stream);
int mttkrp_elem_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                    int64_t rank, int mode, float *out, void *stream);
int mttkrp_slice_f64(const double *X, const int64_t *dims, int order,
                     const double *const *factors, int64_t rank, int mode, double *out,
                     void *stream);
int mttkrp_slice_f32(const float *X, const int64_t *dims, int order, const float *const *factors,
                     int64_t rank, int mode, float *out, void *stream);

/* ---- measurement probes (not part of the MTTKRP) ----
 * The achievable rates that the roofline fractions are also reported
 * against: the HBM read rate and the matrix-core rate of the device the
 * stream belongs to.  Asynchronous on `stream`; time them with events.
 *
 * mttkrp_probe_read: reads bytes (a multiple of 16) of buf once with 16-byte
 *   loads and writes, per workgroup w < mttkrp_probe_read_grid(), the sum
 *   modulo 2^32 of x ^ y ^ z ^ w over the 32-bit words of the 16-byte groups
 *   it read to sink[w] (DEVICE, mttkrp_probe_read_grid() words), so the host
 *   can check that every byte was read.  buf and sink 16-byte aligned.
 * mttkrp_probe_mfma: elem_bytes = 8 (fp64) or 4 (fp32); every wave of
 *   mttkrp_probe_mfma_grid() workgroups of four waves runs iters rounds of
 *   eight independent 16x16x4 MFMAs (2048 flops each) on register operands,
 *   i.e. mttkrp_probe_mfma_grid() * 4 * 8 * 2048 * iters flops in all, and
 *   writes one finite value per wave to sink (DEVICE, 4 *
 *   mttkrp_probe_mfma_grid() doubles).
 * Both return MTTKRP_EINVAL / MTTKRP_EALIGN for bad arguments, MTTKRP_EHIP
 * for a failed launch. */
int mttkrp_probe_read_grid(void);
int mttkrp_probe_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);
int mttkrp_probe_mfma_grid(void);
int mttkrp_probe_mfma(int elem_bytes, int64_t iters, double *sink, void *stream);

/* ---- plan introspection (no device work) ----
 * The decomposition mttkrp_* would launch for this problem: which modes are
 * contracted on the matrix cores, which index the tile rows, the tile shape and
 * the grid.  For tests and reports. */
typedef struct {
    int form;            /* 0: tile rows are the output mode (direct accumulation);
                            1: the output index is fixed per tile and tile rows are
                               reduced against their factor rows                      */
    int layout;          /* 0: contraction index has unit stride; 1: row index has unit stride */
    int k_modes[2];      /* contracted mode(s); k_modes[1] = -1 when one mode        */
    int row_modes[2];    /* tile-row mode(s); row_modes[1] = -1 when one mode        */
    int outer_modes[3];  /* modes iterated per tile (-1 = unused)                     */
    int mb, nb;          /* wave tile: mb x 16 rows, nb x 16 rank columns            */
    int b_in_lds;        /* 1: contraction-side factor rows staged in LDS             */
    int vec;             /* 1: vectorised (4-element) tensor loads                    */
    int64_t k_len;       /* contraction length                                        */
    int64_t rows;        /* tile-row count per batch                                  */
    int64_t batches;     /* outer tuples                                              */
    int64_t splits;      /* independent chunks per output tile (1: no second pass)   */
    int64_t rtiles;      /* rank tiles                                                */
    int64_t grid;        /* workgroups of the main kernel                             */
    size_t lds_bytes;    /* dynamic LDS of the main kernel                            */
    size_t ws_bytes;     /* workspace of this mode                                    */
    int64_t kchunks;     /* contraction chunks (each sums into its own partial)       */
    int waves;           /* waves per workgroup of the main kernel                    */
    int launchable;      /* 1: a kernel exists for this tile (0 only for a forced tile) */
    /* The plain cache model of this plan on MI355X, in seconds (a reading of
     * the GenTen page's "performance models for an ideal multi-level cache
     * machine", TL;DR and abstract, whose formulas are not given): the time
     * each resource needs for the plan's traffic at its peak rate.  model_s
     * = max(flop, hbm, l2, lds).  t_inf_s: every byte moved once; t_0_s: the
     * factor rows re-read for every tensor element (no reuse). */
    double model_flop_s; /* padded tile flops / matrix-core peak                     */
    double model_hbm_s;  /* X (once per L2-sharing group of rank tiles), factors,
                            output and split partials / 8 TB/s                      */
    double model_l2_s;   /* X per rank tile, staged Khatri-Rao tiles, outer and row
                            factor reads / (8 XCDs x 2 KB/clock)                    */
    double model_lds_s;  /* operand reads and staging stores / (256 CUs x 128 B/clock) */
    double model_s;
    double t_inf_s, t_0_s;
} mttkrp_plan_info;

/* Experiments only: the environment variable MTTKRP_FORCE_TILE="mb,nb" or
 * "mb,nb,waves" (mb in {2,4}, nb in {1,2,4,8}, waves in {4,8}) replaces the
 * planner's wave tile in every plan of the process (the tile-heuristic
 * validation sweeps tiles this way).  A malformed value makes every call that
 * plans return MTTKRP_EINVAL, and so does a forced tile no kernel instantiates
 * (mttkrp_plan then reports launchable = 0 and returns MTTKRP_OK). */
int mttkrp_plan(const int64_t *dims, int order, int64_t rank, int mode, int elem_bytes,
                mttkrp_plan_info *info);

#ifdef __cplusplus
}
#endif

#endif /* MTTKRP_AMD_MTTKRP_H */
