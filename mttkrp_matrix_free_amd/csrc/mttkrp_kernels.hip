// Matrix-free dense MTTKRP kernels for gfx950 (CDNA4).
//
// One mode of M(i_n, r) = sum X(i) prod_{m != n} U_m(i_m, r) ("A Performance
// Portable Matrix Free Dense MTTKRP in GenTen", abstract) is computed as a
// stream of small dense contractions run on the matrix cores, never forming
// the Khatri-Rao matrix:
//
//   for every outer tuple o and tile of rows rho:
//       T(rho, r) = sum_k X(o, rho, k) B(k, r)              (MFMA, 16x16x4)
//   form 0 (rho = i_n):   M(rho, r) += T computed with B scaled by W_o(r)
//   form 1 (i_n in o):    M(i_n, r) += sum_rho Z(rho, r) W_o(r) T(rho, r)
//
// where B is the (at most two-factor) Khatri-Rao tile of the contracted modes
// staged in LDS, W_o the Hadamard product of the outer factor rows and Z that
// of the row factors -- the "tile Hadamard product" of the GenTen page, Fig. 2.
//
// Operand delivery.  Each lane loads four consecutive tensor elements with
// 16-byte global loads straight into registers (no LDS round trip for X):
//   layout 0 (contraction index contiguous): a lane holds X(row, k0+4q..k0+4q+3)
//     and feeds them to four successive MFMA k-steps; the k order inside the
//     matrix-core reduction is permuted consistently for A and B, which leaves
//     the sum unchanged;
//   layout 1 (rows contiguous, output = last mode): a lane holds four
//     consecutive rows at one k and feeds four interleaved 16-row blocks.
// The next step's loads are issued before the current step's MFMAs (register
// double buffering), so HBM latency hides behind matrix-core work.
//
// 16x16x4 MFMA lane layout (CDNA3/CDNA4): lane l supplies A(row l%16, k l/16)
// and B(k l/16, col l%16), and receives D(Mfma<T>::row(l/16, e), l%16) in
// element e.
//
// Workgroups: 256 threads (4 waves) sharing one B tile; the workgroup index is
// remapped so that consecutive logical workgroups run on the same XCD (the
// hardware deals workgroups round-robin over the 8 XCDs), keeping the rank
// tiles of one tensor chunk in one L2.
#include <hip/hip_runtime.h>

#include "plan.hpp"

namespace mttkrp {

typedef double dx4 __attribute__((ext_vector_type(4)));
typedef double dx2 __attribute__((ext_vector_type(2)));
typedef float fx4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma;
// The two instructions share their operand layout but not their result
// layout: element e of lane l holds row 4*(l/16)+e for fp32 and row
// 4*e+(l/16) for fp64 (the fp64 result is interleaved over the four lane
// groups).  `row(q, e)` gives that row for lane group q = l/16.
template <>
struct Mfma<double> {
    typedef dx4 acc_t;
    static __device__ __forceinline__ acc_t mma(double a, double b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int q, int e) { return 4 * e + q; }
};
template <>
struct Mfma<float> {
    typedef fx4 acc_t;
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int row(int q, int e) { return 4 * q + e; }
};

__device__ __forceinline__ void load4(const double *p, double *v)
{
    const dx2 a = *reinterpret_cast<const dx2 *>(p);
    const dx2 b = *reinterpret_cast<const dx2 *>(p + 2);
    v[0] = a[0];
    v[1] = a[1];
    v[2] = b[0];
    v[3] = b[1];
}
__device__ __forceinline__ void load4(const float *p, float *v)
{
    const fx4 a = *reinterpret_cast<const fx4 *>(p);
    v[0] = a[0];
    v[1] = a[1];
    v[2] = a[2];
    v[3] = a[3];
}

// Decoded work item: tensor offset of the tile origin, first tile row,
// outer-mode indices.
struct Item {
    int64_t off;
    int64_t row0;
    int64_t oidx[3];
};

__device__ __forceinline__ Item decode_item(const KParams &p, int64_t it, int64_t unit_off,
                                            int64_t rows_per_tile, bool form1)
{
    Item r;
    int64_t b;
    if (form1) {
        b = it / p.nrowtiles;
        r.row0 = (it - b * p.nrowtiles) * rows_per_tile;
    } else {
        b = it;
        r.row0 = 0;
    }
    // unused outer slots have dimension 1 and stride 0
    const int64_t q2 = b / p.o_dim[2];
    r.oidx[2] = b - q2 * p.o_dim[2];
    const int64_t q1 = q2 / p.o_dim[1];
    r.oidx[1] = q2 - q1 * p.o_dim[1];
    r.oidx[0] = q1;
    r.off = unit_off + r.oidx[0] * p.o_stride[0] + r.oidx[1] * p.o_stride[1] +
            r.oidx[2] * p.o_stride[2] + r.row0 * p.row_stride;
    return r;
}

template <typename T, int MB, int NB, bool RC, bool VEC, bool FORM1, bool BLDS>
__global__ __launch_bounds__(kThreads) void mttkrp_tile_kernel(KParams p)
{
    static_assert(!RC || (MB % 4 == 0), "row-contiguous layout uses 64-row groups");
    static_assert(!RC || !FORM1, "row-contiguous layout has the output as rows");
    typedef typename Mfma<T>::acc_t acc_t;
    constexpr int BN = 16 * NB;
    constexpr int ROWS = 16 * MB;
    constexpr int G = MB / 4;  // 64-row groups (layout 1)

    extern __shared__ __align__(16) unsigned char smem[];
    T *Bs = reinterpret_cast<T *>(smem);
    double *red = reinterpret_cast<double *>(smem);

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int q = lane >> 4;
    const int c16 = lane & 15;

    // XCD-aware remap: hardware workgroup b runs on XCD b % 8.
    const int64_t bid = blockIdx.x;
    const int64_t logical = (bid % kNumXCD) * p.grid_per_xcd + bid / kNumXCD;
    if (logical >= p.grid_real) return;
    const int64_t rtile = logical % p.nrtiles;
    const int64_t rest = logical / p.nrtiles;
    const int64_t split = rest % p.nsplit;
    const int64_t unit = rest / p.nsplit;
    const int64_t r0 = rtile * BN;

    const T *__restrict__ X = reinterpret_cast<const T *>(p.X);
    const int64_t R = p.R;

    // ---- stage the contraction-side Khatri-Rao tile B(k, r0:r0+BN) in LDS ----
    if (BLDS) {
        const T *Ua = reinterpret_cast<const T *>(p.Uk0);
        const T *Ub = reinterpret_cast<const T *>(p.Uk1);
        const int64_t total = p.Kpad * BN;
        for (int64_t idx = tid; idx < total; idx += kThreads) {
            const int64_t kk = idx / BN;
            const int c = (int)(idx - kk * BN);
            const int64_t col = r0 + c;
            T v = T(0);
            if (kk < p.K && col < R) {
                if (Ub == nullptr) {
                    v = Ua[kk * R + col];
                } else {
                    const int64_t a = kk / p.IkB;
                    const int64_t b = kk - a * p.IkB;
                    v = Ua[a * R + col] * Ub[b * R + col];
                }
            }
            Bs[kk * p.bpitch + c] = v;
        }
        __syncthreads();
    }

    // Per-lane rank columns.
    int64_t col[NB];
    bool colok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        col[nb] = r0 + nb * 16 + c16;
        colok[nb] = col[nb] < R;
    }

    // Work range of this workgroup and wave.
    const int64_t it_lo = split * p.chunk;
    const int64_t it_hi = min(p.nitems, it_lo + p.chunk);
    const int64_t my_first = it_lo + wave;
    const int64_t my_items = my_first < it_hi ? (it_hi - my_first + kWaves - 1) / kWaves : 0;
    const int64_t nkc = p.Kpad / 16;
    const int64_t nsteps = my_items * nkc;

    // Unit: form 1 -> output row i_n; form 0 -> tile of output rows.
    int64_t unit_off, out_row0;
    if (FORM1) {
        unit_off = unit * p.n_stride;
        out_row0 = unit;
    } else {
        out_row0 = unit * ROWS;
        unit_off = out_row0 * p.row_stride;
    }
    const int64_t nrows_lim = FORM1 ? p.nrows : p.In;

    acc_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = acc_t{};
    // form 1: running per-column sums; form 0 with fp32: fp64 flush of acc
    double accrow[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) accrow[j] = 0.0;
    constexpr bool FLUSH64 = (!FORM1) && sizeof(T) == 4;
    double acc64[FLUSH64 ? MB : 1][FLUSH64 ? NB : 1][FLUSH64 ? 4 : 1];
    if (FLUSH64) {
#pragma unroll
        for (int i = 0; i < (FLUSH64 ? MB : 1); ++i)
#pragma unroll
            for (int j = 0; j < (FLUSH64 ? NB : 1); ++j)
#pragma unroll
                for (int e = 0; e < (FLUSH64 ? 4 : 1); ++e) acc64[i][j][e] = 0.0;
    }

    // ---- loads of one 16-wide contraction step ----
    auto load_step = [&](T *a, const Item &itm, int64_t kc) {
        if (!RC) {
            const int64_t kk = kc * 16 + 4 * q;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t rr = (FORM1 ? itm.row0 : out_row0) + mb * 16 + c16;
                const T *src = X + itm.off + (int64_t)(mb * 16 + c16) * p.row_stride + kk;
                if (VEC) {
                    if (rr < nrows_lim && kk < p.K) {
                        load4(src, a + mb * 4);
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[mb * 4 + e] = T(0);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a[mb * 4 + e] = (rr < nrows_lim && kk + e < p.K) ? src[e] : T(0);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int64_t kk = kc * 16 + 4 * s + q;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const int64_t rr = out_row0 + 64 * g + 4 * c16;
                    const T *src = X + itm.off + kk * p.k_stride + 64 * g + 4 * c16;
                    T *dst = a + (s * G + g) * 4;
                    if (VEC) {
                        if (kk < p.K && rr < p.In) {
                            load4(src, dst);
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) dst[e] = T(0);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            dst[e] = (kk < p.K && rr + e < p.In) ? src[e] : T(0);
                    }
                }
            }
        }
    };

    // Outer multiplier of an item (product of the outer factor rows).
    auto outer_w = [&](const Item &itm, T *w) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) w[nb] = T(1);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            if (j < p.nouter) {
                const T *Uo = reinterpret_cast<const T *>(p.Uo[j]) + itm.oidx[j] * R;
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
                    if (colok[nb]) w[nb] *= Uo[col[nb]];
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            if (!colok[nb]) w[nb] = T(0);
    };

    // ---- matrix-core work of one step ----
    const T *Ug = reinterpret_cast<const T *>(p.Uk0);
    auto compute_step = [&](const T *a, int64_t kc, const T *wb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int64_t kk = RC ? (kc * 16 + 4 * s + q) : (kc * 16 + 4 * q + s);
            T b[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                if (BLDS) {
                    b[nb] = Bs[kk * p.bpitch + nb * 16 + c16];
                } else {
                    b[nb] = (kk < p.K && colok[nb]) ? Ug[kk * R + col[nb]] : T(0);
                }
                if (!FORM1) b[nb] *= wb[nb];
            }
            if (!RC) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
                        acc[mb][nb] = Mfma<T>::mma(a[mb * 4 + s], b[nb], acc[mb][nb]);
            } else {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            acc[4 * g + jj][nb] =
                                Mfma<T>::mma(a[(s * G + g) * 4 + jj], b[nb], acc[4 * g + jj][nb]);
            }
        }
    };

    // ---- end of a work item ----
    auto finish_item = [&](const Item &itm, const T *w) {
        if (FORM1) {
            // Reduce the tile rows against their factor rows and the outer multiplier.
            const T *Ura = reinterpret_cast<const T *>(p.Ur0);
            const T *Urb = reinterpret_cast<const T *>(p.Ur1);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t rr = itm.row0 + mb * 16 + Mfma<T>::row(q, e);
                    if (rr < p.nrows) {
                        int64_t ia = rr, ib = 0;
                        if (Urb) {
                            ia = rr / p.IrB;
                            ib = rr - ia * p.IrB;
                        }
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            if (colok[nb]) {
                                double z = (double)Ura[ia * R + col[nb]] * (double)w[nb];
                                if (Urb) z *= (double)Urb[ib * R + col[nb]];
                                accrow[nb] += z * (double)acc[mb][nb][e];
                            }
                        }
                    }
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = acc_t{};
            }
        } else if (FLUSH64) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc64[mb][nb][e] += (double)acc[mb][nb][e];
                    acc[mb][nb] = acc_t{};
                }
        }
    };

    // ---- main loop: steps over (item, k-chunk), loads one step ahead ----
    if (nsteps > 0) {
        T abuf0[MB * 4], abuf1[MB * 4];
        // load cursor
        int64_t l_it = my_first, l_kc = 0;
        Item l_itm = decode_item(p, l_it, unit_off, ROWS, FORM1);
        // compute cursor
        int64_t c_kc = 0;
        Item c_itm = l_itm;
        T w[NB];
        outer_w(c_itm, w);

        auto advance_load = [&]() {
            if (++l_kc == nkc) {
                l_kc = 0;
                l_it += kWaves;
                if (l_it < it_hi) l_itm = decode_item(p, l_it, unit_off, ROWS, FORM1);
            }
        };
        // Items of the compute cursor are re-decoded from a counter.
        int64_t c_it = my_first;
        load_step(abuf0, l_itm, l_kc);
        advance_load();
        for (int64_t j = 0; j < nsteps; j += 2) {
            if (j + 1 < nsteps) {
                load_step(abuf1, l_itm, l_kc);
                advance_load();
            }
            compute_step(abuf0, c_kc, w);
            if (++c_kc == nkc) {
                finish_item(c_itm, w);
                c_kc = 0;
                c_it += kWaves;
                if (c_it < it_hi) {
                    c_itm = decode_item(p, c_it, unit_off, ROWS, FORM1);
                    outer_w(c_itm, w);
                }
            }
            if (j + 1 >= nsteps) break;
            if (j + 2 < nsteps) {
                load_step(abuf0, l_itm, l_kc);
                advance_load();
            }
            compute_step(abuf1, c_kc, w);
            if (++c_kc == nkc) {
                finish_item(c_itm, w);
                c_kc = 0;
                c_it += kWaves;
                if (c_it < it_hi) {
                    c_itm = decode_item(p, c_it, unit_off, ROWS, FORM1);
                    outer_w(c_itm, w);
                }
            }
        }
    }

    // ---- workgroup reduction and store ----
    const bool split_out = p.nsplit > 1;
    __syncthreads();  // every wave is done with the B tile: LDS is reused below
    if (FORM1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            double v = accrow[nb];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            accrow[nb] = v;
        }
        if (q == 0) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) red[wave * BN + nb * 16 + c16] = accrow[nb];
        }
        __syncthreads();
        if (tid < BN) {
            double v = red[tid];
#pragma unroll
            for (int w2 = 1; w2 < kWaves; ++w2) v += red[w2 * BN + tid];
            const int64_t c = r0 + tid;
            if (c < R) {
                if (split_out) {
                    p.partial[(split * p.In + out_row0) * R + c] = v;
                } else if (p.out64) {
                    reinterpret_cast<double *>(p.out)[out_row0 * R + c] = v;
                } else {
                    reinterpret_cast<T *>(p.out)[out_row0 * R + c] = (T)v;
                }
            }
        }
    } else {
        // Lane-private layout: element (mb, nb, e) of lane l at ((mb*NB+nb)*4+e)*64 + l.
        auto val = [&](int mb, int nb, int e) -> double {
            return FLUSH64 ? acc64[FLUSH64 ? mb : 0][FLUSH64 ? nb : 0][FLUSH64 ? e : 0]
                           : (double)acc[mb][nb][e];
        };
        for (int w2 = kWaves - 1; w2 >= 1; --w2) {
            if (wave == w2) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int idx = ((mb * NB + nb) * 4 + e) * 64 + lane;
                            red[idx] = (w2 == kWaves - 1) ? val(mb, nb, e) : red[idx] + val(mb, nb, e);
                        }
            }
            __syncthreads();
        }
        if (wave == 0) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int idx = ((mb * NB + nb) * 4 + e) * 64 + lane;
                        const double v = val(mb, nb, e) + (kWaves > 1 ? red[idx] : 0.0);
                        int64_t row;
                        if (!RC)
                            row = out_row0 + mb * 16 + Mfma<T>::row(q, e);
                        else
                            row = out_row0 + 64 * (mb / 4) + 4 * Mfma<T>::row(q, e) + (mb % 4);
                        if (row < p.In && colok[nb]) {
                            if (split_out) {
                                p.partial[(split * p.In + row) * R + col[nb]] = v;
                            } else if (p.out64) {
                                reinterpret_cast<double *>(p.out)[row * R + col[nb]] = v;
                            } else {
                                reinterpret_cast<T *>(p.out)[row * R + col[nb]] = (T)v;
                            }
                        }
                    }
        }
    }
}

// Fixed-order sum of the split partials: out[i] = sum_{s=0}^{S-1} partial[s][i].
template <typename T>
__global__ __launch_bounds__(256) void split_reduce_kernel(const double *__restrict__ partial,
                                                           int64_t nsplit, int64_t count,
                                                           void *out, int out64)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    double v = 0.0;
    for (int64_t s = 0; s < nsplit; ++s) v += partial[s * count + i];
    if (out64)
        reinterpret_cast<double *>(out)[i] = v;
    else
        reinterpret_cast<T *>(out)[i] = (T)v;
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

typedef void (*TileKernel)(KParams);

template <typename T, int MB, int NB, bool RC, bool VEC, bool FORM1, bool BLDS>
TileKernel pick()
{
    return mttkrp_tile_kernel<T, MB, NB, RC, VEC, FORM1, BLDS>;
}

template <typename T, int MB, int NB, bool RC, bool FORM1, bool BLDS>
TileKernel pick_vec(bool vec)
{
    return vec ? pick<T, MB, NB, RC, true, FORM1, BLDS>() : pick<T, MB, NB, RC, false, FORM1, BLDS>();
}

template <typename T, int MB, bool RC, bool FORM1, bool BLDS>
TileKernel pick_nb(int nb, bool vec)
{
    switch (nb) {
    case 1: return pick_vec<T, MB, 1, RC, FORM1, BLDS>(vec);
    case 2: return pick_vec<T, MB, 2, RC, FORM1, BLDS>(vec);
    case 4: return pick_vec<T, MB, 4, RC, FORM1, BLDS>(vec);
    default: return nullptr;
    }
}

template <typename T>
TileKernel select_kernel(const Plan &pl)
{
    if (pl.layout == 1) {
        if (pl.mb != 4 || pl.form != 0) return nullptr;
        return pl.b_in_lds ? pick_nb<T, 4, true, false, true>(pl.nb, pl.vec)
                           : pick_nb<T, 4, true, false, false>(pl.nb, pl.vec);
    }
    if (pl.form == 0) {
        if (pl.mb != 2 || !pl.b_in_lds) return nullptr;
        return pick_nb<T, 2, false, false, true>(pl.nb, pl.vec);
    }
    if (!pl.b_in_lds) {
        if (pl.mb != 2) return nullptr;
        if (pl.nb == 8) return pick_vec<T, 2, 8, false, true, false>(pl.vec);
        return pick_nb<T, 2, false, true, false>(pl.nb, pl.vec);
    }
    if (pl.nb == 8) return pl.mb == 2 ? pick_vec<T, 2, 8, false, true, true>(pl.vec) : nullptr;
    if (pl.mb == 4) return pick_nb<T, 4, false, true, true>(pl.nb, pl.vec);
    if (pl.mb == 2) return pick_nb<T, 2, false, true, true>(pl.nb, pl.vec);
    return nullptr;
}

template <typename T>
hipError_t launch_mttkrp(const Plan &pl, hipStream_t stream)
{
    TileKernel k = select_kernel<T>(pl);
    if (!k) return hipErrorInvalidConfiguration;
    if (pl.lds_bytes > 64 * 1024) {
        // gfx950 has 160 KB of LDS per CU; dynamic sizes above 64 KB are opted into.
        hipError_t a = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)pl.lds_bytes);
        if (a != hipSuccess) return a;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)pl.grid), dim3(kThreads), pl.lds_bytes, stream, pl.kp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (pl.kp.nsplit > 1) {
        const int64_t count = pl.kp.In * pl.kp.R;
        const unsigned blocks = (unsigned)((count + 255) / 256);
        hipLaunchKernelGGL(split_reduce_kernel<T>, dim3(blocks), dim3(256), 0, stream,
                           (const double *)pl.kp.partial, pl.kp.nsplit, count, pl.kp.out,
                           pl.kp.out64);
        e = hipGetLastError();
    }
    return e;
}

template hipError_t launch_mttkrp<double>(const Plan &, hipStream_t);
template hipError_t launch_mttkrp<float>(const Plan &, hipStream_t);

}  // namespace mttkrp
