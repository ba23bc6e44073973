// Matrix-free dense MTTKRP tile kernel for gfx950 (CDNA4) -- template, included by the
// instantiation units tile_*.hip.
//
//
// One mode of M(i_n, r) = sum X(i) prod_{m != n} U_m(i_m, r) ("A Performance
// Portable Matrix Free Dense MTTKRP in GenTen", abstract) is computed as a
// stream of small dense contractions run on the matrix cores, never forming
// the Khatri-Rao matrix:
//
//   for every outer tuple o and tile of rows rho:
//       T(rho, r) = sum_k X(o, rho, k) B(k, r)              (MFMA, 16x16x4)
//   form 0 (rho = i_n):   M(rho, r) += T computed with B scaled by W_o(r)
//                         (fp32: M += W_o(r) T, once per item, in fp64)
//   form 1 (i_n in o):    M(i_n, r) += sum_rho Z(rho, r) W_o(r) T(rho, r)
//
// where B is the (at most two-factor) Khatri-Rao tile of the contracted modes,
// W_o the Hadamard product of the outer factor rows and Z that of the row
// factors -- the "tile Hadamard product" of the GenTen page, Fig. 2.
//
// Tensor loads.  X is read with buffer loads whose per-lane byte offsets are
// fixed for a wave and whose per-step advance is a scalar offset.  A lane
// whose element lies outside the tile (ragged rows, the tail of the
// contraction, steps past the end of the wave's work) gets an offset past the
// buffer's range, for which the hardware returns zero without touching memory.
// The loads therefore carry no branches, and the loop keeps the loads of the
// next steps (two when the registers allow) in flight while the matrix cores
// work on the current one:
//   layout 0 (contraction index contiguous): a lane holds X(row, k0+4q..k0+4q+3)
//     and feeds them to four successive MFMA k-steps; the k order inside the
//     matrix-core reduction is permuted consistently for A and B, which leaves
//     the sum unchanged;
//   layout 1 (rows contiguous, output = last mode): a lane holds RL = 4 (or,
//     for 32-row tiles, 2) consecutive rows at one k and feeds RL interleaved
//     16-row blocks.
//
// 16x16x4 MFMA lane layout (CDNA3/CDNA4): lane l supplies A(row l%16, k l/16)
// and B(k l/16, col l%16), and receives D(Mfma<T>::row(l/16, e), l%16) in
// element e.
//
// Workgroups: four or eight waves sharing one B tile (eight waves per compute
// unit in either case); the workgroup index is remapped so that consecutive logical
// workgroups run on the same XCD (the hardware deals workgroups round-robin
// over the 8 XCDs), keeping the rank tiles of one tensor chunk in one L2.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "plan.hpp"
#include "tile_select.hpp"

namespace mttkrp {

typedef double dx4 __attribute__((ext_vector_type(4)));
typedef double dx2 __attribute__((ext_vector_type(2)));
typedef float fx4 __attribute__((ext_vector_type(4)));
typedef float fx2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Third descriptor word of a raw (unstructured) buffer on gfx9-family parts.
constexpr unsigned kRsrcWord3 = 0x00020000u;
// Byte offset past every descriptor's range (ranges are kept below 2^31):
// a load at this offset returns zero.
constexpr unsigned kOOB = 0x80000000u;

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

// Descriptor of [base, base + bytes) (range capped below 2^31).  The base and
// the range are wave-uniform; they are read from the first lane so that the
// compiler keeps the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes >= 0x7fffffff ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(lo | (hi << 32)), 0,
                                             __builtin_amdgcn_readfirstlane(n), kRsrcWord3);
}

// Four consecutive elements at byte offset voff (+ soff).
__device__ __forceinline__ void bload4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                       double *v)
{
    const dx2 a = __builtin_bit_cast(dx2, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    const dx2 b =
        __builtin_bit_cast(dx2, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
    v[0] = a[0];
    v[1] = a[1];
    v[2] = b[0];
    v[3] = b[1];
}
__device__ __forceinline__ void bload4(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                       float *v)
{
    const fx4 a = __builtin_bit_cast(fx4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    v[0] = a[0];
    v[1] = a[1];
    v[2] = a[2];
    v[3] = a[3];
}
// Two consecutive elements at byte offset voff (+ soff).
__device__ __forceinline__ void bload2(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                       double *v)
{
    const dx2 a = __builtin_bit_cast(dx2, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    v[0] = a[0];
    v[1] = a[1];
}
__device__ __forceinline__ void bload2(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                       float *v)
{
    const fx2 a = __builtin_bit_cast(fx2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
    v[0] = a[0];
    v[1] = a[1];
}
// One element at byte offset voff (+ soff).
__device__ __forceinline__ double bload1(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                         double)
{
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff,
                                        float)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Element offset of tile row r: r * stride, or, for two row modes that are
// not adjacent, ia * stride_a + ib * stride_b with (ia, ib) = divmod(r, I_b).
__device__ __forceinline__ int64_t row_offset(const KParams &p, int64_t r)
{
    if (!p.row_split) return r * p.row_stride;
    const uint32_t ia = fdiv((uint32_t)r, p.fd_IrB);
    return (int64_t)ia * p.row_stride_a + (int64_t)((uint32_t)r - ia * p.fd_IrB.d) * p.row_stride;
}

// Decoded work item: tensor offset of the tile origin, first tile row,
// outer-mode indices.
struct Item {
    int64_t off;
    int64_t row0;
    int64_t oidx[3];
};

__device__ __forceinline__ Item decode_item(const KParams &p, uint32_t it, int64_t unit_off,
                                            int64_t rows_per_tile, bool form1)
{
    // (item indices are below 2^31: 32-bit divisions by planner constants)
    Item r;
    uint32_t b;
    if (form1) {
        b = fdiv(it, p.fd_nrowtiles);
        r.row0 = (int64_t)(it - b * p.fd_nrowtiles.d) * rows_per_tile;
    } else {
        b = it;
        r.row0 = 0;
    }
    // unused outer slots have dimension 1 and stride 0
    const uint32_t q2 = fdiv(b, p.fd_odim2);
    r.oidx[2] = b - q2 * p.fd_odim2.d;
    const uint32_t q1 = fdiv(q2, p.fd_odim1);
    r.oidx[1] = q2 - q1 * p.fd_odim1.d;
    r.oidx[0] = q1;
    r.off = unit_off + r.oidx[0] * p.o_stride[0] + r.oidx[1] * p.o_stride[1] +
            r.oidx[2] * p.o_stride[2] + row_offset(p, r.row0);
    return r;
}

// One mode's work for the calling workgroup.  stage_b = false: the B tile of
// this pass is already in LDS (staged by an earlier pass of the same launch
// with the same contraction chunk and rank tile); red_off: byte offset of the
// cross-wave reduction space in LDS.
template <typename T, int MB, int NB, bool RC, bool VEC, bool FORM1, int W, int S>
__device__ __forceinline__ void tile_pass(const KParams &p, unsigned char *smem, bool stage_b,
                                          size_t red_off)
{
    // S: outer-factor slots carried per step (0: no outer mode; else one per
    // outer mode, with unused slots counting as 1).
    static_assert(S >= 0 && S <= 3, "outer slots");
    static_assert(!FORM1 || S == 0, "form 1 reads its outer factors once per item");
    constexpr int SS = S > 0 ? S : 1;  // array extent
    constexpr int NT = 64 * W;  // threads of the workgroup (W waves)
    static_assert(!RC || MB == 2 || MB % 4 == 0, "row-contiguous layout: 32- or 64-row groups");
    static_assert(!RC || !FORM1, "row-contiguous layout has the output as rows");
    static_assert(W == 4 || W == 8, "four or eight waves");
    typedef typename Mfma<T>::acc_t acc_t;
    constexpr int BN = 16 * NB;
    constexpr int ROWS = 16 * MB;
    // layout 1: a lane holds RL consecutive rows of each 16*RL-row group
    constexpr int RL = MB < 4 ? MB : 4;
    constexpr int G = MB / RL;  // row groups
    constexpr int NA = 4 * MB;  // tensor elements per lane per step
    constexpr unsigned SZ = sizeof(T);

    T *Bs = reinterpret_cast<T *>(smem);
    double *red = reinterpret_cast<double *>(smem + red_off);

    const int tid = threadIdx.x;
    // The wave index is uniform across the wave: keep it (and everything
    // derived from it) in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int q = lane >> 4;
    const int c16 = lane & 15;

    // XCD-aware remap: hardware workgroup b runs on XCD b % 8.
    const int64_t bid = blockIdx.x;
    const int64_t logical = (bid % kNumXCD) * p.grid_per_xcd + bid / kNumXCD;
    if (logical >= p.grid_real) return;
    // Workgroup decode in 32 bits (the grid is below 2^31).
    const uint32_t lg = (uint32_t)logical;
    const uint32_t rest = fdiv(lg, p.fd_nrtiles);
    const int64_t rtile = lg - rest * p.fd_nrtiles.d;
    // unit-major (the splits of one unit adjacent) or split-major (the units
    // of one split adjacent: row tiles that share cache lines then run on one
    // XCD and walk the same contraction steps together)
    uint32_t unit32, split32;
    if (p.split_major) {
        split32 = fdiv(rest, p.fd_nunits);
        unit32 = rest - split32 * p.fd_nunits.d;
    } else {
        unit32 = fdiv(rest, p.fd_nsplit);
        split32 = rest - unit32 * p.fd_nsplit.d;
    }
    const int64_t split = split32;  // output partial written by this workgroup
    const int64_t unit = unit32;
    const uint32_t kch32 = fdiv((uint32_t)split, p.fd_nsplit_it);
    const int64_t kch = kch32;                                   // contraction chunk
    const int64_t isplit = split - (int64_t)kch32 * p.fd_nsplit_it.d;  // chunk of the work items
    const int64_t r0 = rtile * BN;
    const int64_t kbase = kch * p.Kc;
    const int64_t Kloc = min(p.Kc, p.K - kbase);
    // steps per item (the last contraction chunk may be shorter)
    const FastDiv fd_nkc = kch == p.nkch - 1 ? p.fd_nkc_last : p.fd_nkc_full;
    const int nkc = (int)fd_nkc.d;

    const T *__restrict__ X = reinterpret_cast<const T *>(p.X);
    const int64_t R = p.R;

    // Per-lane rank columns (R < 2^24, so 32 bits suffice).
    int col[NB];
    bool colok[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        col[nb] = (int)r0 + nb * 16 + c16;
        colok[nb] = col[nb] < R;
    }

    // Work range of this workgroup: steps [g_lo, g_lo + wg_steps) of the
    // unit's sequence of (item, step) pairs, nkc steps per item.  Form 0 cuts
    // the sequence into nsplit_it equal ranges; form 1 into ranges of whole
    // items (p.chunk items each), because every item a range touches costs a
    // row reduction.  The waves split the workgroup's range evenly in turn.  A
    // range may start or end inside an item (every item result is linear in
    // its steps, so a partial item is reduced like a whole one).
    // (below 2^31: the planner bounds the unit's steps)
    const int tot_steps = (int)p.nitems * nkc;
    int g_lo, wg_steps;
    if (FORM1) {
        const int it_lo = min((int)p.nitems, (int)(isplit * p.chunk));
        const int it_hi = min((int)p.nitems, it_lo + (int)p.chunk);
        g_lo = it_lo * nkc;
        wg_steps = (it_hi - it_lo) * nkc;
    } else {
        const int wg_chunk =
            (int)fdiv((uint32_t)(tot_steps + (int)p.fd_nsplit_it.d - 1), p.fd_nsplit_it);
        g_lo = min(tot_steps, (int)isplit * wg_chunk);
        wg_steps = min(tot_steps, g_lo + wg_chunk) - g_lo;
    }
    const int per_wave = (wg_steps + W - 1) / W;
    const int s_lo = min(wg_steps, wave * per_wave);
    const int s_hi = min(wg_steps, s_lo + per_wave);
    const int nsteps = s_hi - s_lo;

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

    // ---- per-lane byte offsets of the tensor elements inside a tile ----
    // layout 0: row block mb, elements 4q..4q+3 of the contraction step;
    // layout 1: substep s, 64-row group g, rows 4*c16..4*c16+3.
    constexpr int NV = RC ? 4 * G : MB;
    unsigned vbase[NV];
    if (!RC) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
            vbase[mb] = (unsigned)(((int64_t)(mb * 16 + c16) * p.row_stride + 4 * q) * SZ);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int g = 0; g < G; ++g)
                vbase[s * G + g] = (unsigned)(((int64_t)(16 * RL * g + RL * c16) +
                                               (int64_t)(4 * s + q) * p.k_stride) *
                                              SZ);
    }
    // Row validity (form 0: fixed for the workgroup; form 1: per item).
    // With two non-adjacent row modes the offsets depend on the item's first
    // row and are recomputed per item.
    auto row_offsets = [&](int64_t row0, unsigned *vo) {
        if (!RC) {
            const int64_t base0 = FORM1 && p.row_split ? row_offset(p, row0) : 0;
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int64_t rr = row0 + mb * 16 + c16;
                unsigned v = vbase[mb];
                if (FORM1 && p.row_split)
                    v = (unsigned)((row_offset(p, rr < nrows_lim ? rr : row0) - base0 + 4 * q) * SZ);
                vo[mb] = rr < nrows_lim ? v : kOOB;
            }
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    vo[s * G + g] =
                        (out_row0 + 16 * RL * g + RL * c16 < p.In) ? vbase[s * G + g] : kOOB;
        }
    };

    // Load cursor state: descriptor of the current item and its offsets.
    struct LoadCursor {
        int64_t base;  // element offset of the descriptor's start in X
        unsigned vo[NV];
        int it, kc, step;      // item, step in the item, step in the workgroup
        int64_t orow[3];       // element offsets of the outer factor rows (i_o * R)
        bool live;             // step < s_hi: past it, loads return zeros
    };
    const int64_t x_elems = p.x_bytes / SZ;
    const int64_t kshift = RC ? kbase * p.k_stride : kbase;  // start of the chunk
    auto enter_item = [&](LoadCursor &lc) {
        if (lc.step < s_hi) {
            const Item itm = decode_item(p, lc.it, unit_off, ROWS, FORM1);
            lc.base = itm.off + kshift;
            row_offsets(FORM1 ? itm.row0 : out_row0, lc.vo);
#pragma unroll
            for (int j = 0; j < 3; ++j) lc.orow[j] = j < p.nouter ? itm.oidx[j] * R : 0;
            lc.live = true;
        } else {
            lc.live = false;
        }
    };
    // Columns of this lane clamped into the factor (loads need no branch).
    int colc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) colc[nb] = colok[nb] ? col[nb] : 0;
    // Outer factors, read through buffer descriptors: the lane's column is a
    // fixed vector offset and the item's row a scalar offset, so a step's
    // factor loads need no address arithmetic.  Unused slots have an empty
    // range (their loads return zero) and count as 1 in the product.
    __amdgpu_buffer_rsrc_t ro[SS];
#pragma unroll
    for (int j = 0; j < SS; ++j)
        ro[j] = make_rsrc(j < p.nouter ? p.Uo[j] : p.Uk0,
                          j < p.nouter ? p.o_dim[j] * R * (int64_t)SZ : 0);
    unsigned ocol[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) ocol[nb] = (unsigned)colc[nb] * SZ;

    // Issue the loads of the cursor's step: its three outer factor values
    // (whose product is the multiplier W_o of the step's item) into wq, then
    // its tensor elements into a.  Each step carries the factor values of its
    // own item, so they are buffered with the tensor and no load depends on a
    // branch; the product is formed only when the step is used.
    auto load_step = [&](T *a, T (*wq)[NB], const LoadCursor &lc) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            const unsigned srow = (unsigned)(lc.orow[j] * SZ);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wq[j][nb] = bload1(ro[j], ocol[nb], srow, T(0));
        }
        const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(X + lc.base, (x_elems - lc.base) * (int64_t)SZ);
        const int krem = (int)Kloc - lc.kc * 16;  // contraction elements left in this item
        if (!RC) {
            const unsigned soff = (unsigned)(lc.kc * 16 * SZ);
            const bool kin = lc.live && (4 * q < krem);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                if (VEC) {
                    bload4(rsrc, kin ? lc.vo[mb] : kOOB, soff, a + mb * 4);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        a[mb * 4 + e] = bload1(
                            rsrc, (lc.live && 4 * q + e < krem) ? lc.vo[mb] + e * SZ : kOOB,
                            soff, T(0));
                }
            }
        } else {
            const unsigned soff = (unsigned)(lc.kc * 16 * p.k_stride * SZ);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bool kin = lc.live && (4 * s + q < krem);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    T *dst = a + (s * G + g) * RL;
                    const unsigned vo = kin ? lc.vo[s * G + g] : kOOB;
                    if (VEC) {
                        if (RL == 4)
                            bload4(rsrc, vo, soff, dst);
                        else
                            bload2(rsrc, vo, soff, dst);
                    } else {
#pragma unroll
                        for (int e = 0; e < RL; ++e)
                            dst[e] = bload1(rsrc,
                                            (vo != kOOB && out_row0 + 16 * RL * g + RL * c16 + e < p.In)
                                                ? vo + e * SZ
                                                : kOOB,
                                            soff, T(0));
                    }
                }
            }
        }
    };
    auto advance = [&](LoadCursor &lc) {
        ++lc.step;
        if (++lc.kc == nkc) {
            lc.kc = 0;
            ++lc.it;
            enter_item(lc);
        } else if (lc.step == s_hi) {
            lc.live = false;
        }
    };

    // ---- matrix-core work of one step ----
    // Multiplier of a step from its buffered factor values.  The empty asm
    // pins the values to this point, so the product (and the wait for its
    // loads) is not moved up to where the loads are issued.
    auto multiplier = [&](T (*wq)[NB], T *w) {
#pragma unroll
        for (int j = 0; j < S; ++j)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(wq[j][nb]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            T v = colok[nb] ? T(1) : T(0);
#pragma unroll
            for (int j = 0; j < S; ++j) v *= j < p.nouter ? wq[j][nb] : T(1);
            w[nb] = v;
        }
    };
    // fp32 form 0 applies the outer multiplier once per item instead (at the
    // item end, with the fp64 flush), so its steps use B as staged.
    constexpr bool SCALE_B = !FORM1 && !FLUSH64;
    auto compute_step = [&](const T *a, int kc, T (*wq)[NB]) {
        T wb[NB];
        if (SCALE_B) multiplier(wq, wb);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int kk = RC ? (kc * 16 + 4 * s + q) : (kc * 16 + 4 * q + s);
            T b[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                b[nb] = Bs[kk * p.bpitch + nb * 16 + c16];
                if (SCALE_B) b[nb] *= wb[nb];
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
                        for (int jj = 0; jj < RL; ++jj)
                            acc[RL * g + jj][nb] =
                                Mfma<T>::mma(a[(s * G + g) * RL + jj], b[nb], acc[RL * g + jj][nb]);
            }
        }
    };

    // ---- end of a work item ----
    // Outer factors of the form-1 item reduction; unused slots read the first
    // row of the contraction factor and count as 1.
    const T *Uf[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) Uf[j] = reinterpret_cast<const T *>(j < p.nouter ? p.Uo[j] : p.Uk0);
    auto finish_item = [&](int64_t row0, const int64_t *orow, T (*wq)[NB]) {
        if (FORM1) {
            // The item's outer multiplier W_o (needed once per item, so read
            // here rather than with every step's tensor loads).
            // (Only the outer modes the plan has are read.)
            T wv[3][NB];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) wv[j][nb] = T(1);
                if (j < p.nouter) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) wv[j][nb] = Uf[j][orow[j] + colc[nb]];
                }
            }
            // Reduce the tile rows against their factor rows and the outer
            // multiplier, one accumulator row g = (mb, e) at a time.  The
            // factor loads use 32-bit offsets from the factor's base (its
            // span is below 2^31 bytes); indices are clamped (rows past the
            // tile's end are masked afterwards), so no load depends on its
            // lane's row.
            const bool two = p.Ur1 != nullptr;
            const unsigned IrB = (unsigned)p.IrB;
            const unsigned RS = (unsigned)(R * SZ);
            const char *za_base = reinterpret_cast<const char *>(p.Ur0);
            const char *zb_base = reinterpret_cast<const char *>(two ? p.Ur1 : p.Ur0);
            unsigned cofs_z[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) cofs_z[nb] = (unsigned)(colc[nb] * SZ);
            constexpr int NG = MB * 4;
            T w[NB];
            auto outer_weight = [&]() {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    T v = T(1);
#pragma unroll
                    for (int j = 0; j < 3; ++j) v *= j < p.nouter ? wv[j][nb] : T(1);
                    w[nb] = v;
                }
            };
            if constexpr (sizeof(T) == 8) {
                // fp64: with at most 16 values of a factor per lane the loads
                // of all rows go out at once (one round trip); otherwise the
                // loads of row g + 1 are issued before row g is used, so only
                // two rows are held.  An absent second factor reads the first
                // and counts as 1 (no load sits under a branch).
                constexpr bool ZALL = NG * NB <= 16;
                constexpr int ZR = ZALL ? NG : 2;
                T za[ZR][NB], zb[ZR][NB];
                auto zload = [&](int g, T *a, T *b) {
                    const int64_t rr = row0 + (g >> 2) * 16 + Mfma<T>::row(q, g & 3);
                    const unsigned rc = rr < p.nrows ? (unsigned)rr : 0u;
                    const unsigned ia = two ? fdiv(rc, p.fd_IrB) : rc;
                    const unsigned ib = two ? rc - ia * IrB : 0u;
                    const unsigned oa = ia * RS, ob = ib * RS;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        a[nb] = *reinterpret_cast<const T *>(za_base + (oa + cofs_z[nb]));
                        b[nb] = *reinterpret_cast<const T *>(zb_base + (ob + cofs_z[nb]));
                    }
                };
                if (ZALL) {
#pragma unroll
                    for (int g = 0; g < NG; ++g) zload(g, za[g % ZR], zb[g % ZR]);
                } else {
                    zload(0, za[0], zb[0]);
                }
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    asm volatile("" ::: "memory");
                    if (!ZALL && g + 1 < NG) zload(g + 1, za[(g + 1) % ZR], zb[(g + 1) % ZR]);
                    if (g == 0) outer_weight();
                    const int mb = g >> 2, e = g & 3;
                    const bool rok = row0 + mb * 16 + Mfma<T>::row(q, e) < p.nrows;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const double zbv = two ? (double)zb[g % ZR][nb] : 1.0;
                        const double z = (double)za[g % ZR][nb] * zbv * (double)w[nb];
                        const double t = z * (double)acc[mb][nb][e];
                        accrow[nb] += (rok && colok[nb]) ? t : 0.0;
                    }
                }
            } else {
                // fp32: one copy of the row loop with a second row factor
                // (TWO) and one without (its values are not read).  The
                // factor values of ZR rows are loaded together: one round trip
                // per batch of rows, at most 16 values of a factor per lane.
                // The weights and their products with the tile are formed in
                // fp32, the row sums in fp64 (columns past the rank are never
                // stored: no mask).
                auto rows = [&](auto two_c) {
                    constexpr bool TWO = decltype(two_c)::value;
                    constexpr int ZR = NG * NB <= 16 ? NG : 16 / NB;
                    static_assert(NG % ZR == 0 && ZR >= 1, "whole batches of rows");
                    T za[ZR][NB], zb[TWO ? ZR : 1][NB];
                    auto zload = [&](int g, int u) {
                        const int64_t rr = row0 + (g >> 2) * 16 + Mfma<T>::row(q, g & 3);
                        const unsigned rc = rr < p.nrows ? (unsigned)rr : 0u;
                        const unsigned ia = TWO ? fdiv(rc, p.fd_IrB) : rc;
                        const unsigned oa = ia * RS;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            za[u][nb] = *reinterpret_cast<const T *>(za_base + (oa + cofs_z[nb]));
                            if constexpr (TWO)
                                zb[u][nb] = *reinterpret_cast<const T *>(
                                    zb_base + ((rc - ia * IrB) * RS + cofs_z[nb]));
                        }
                    };
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        if (g % ZR == 0) {
                            asm volatile("" ::: "memory");
#pragma unroll
                            for (int u = 0; u < ZR; ++u) zload(g + u, u);
                        }
                        if (g == 0) outer_weight();  // (after the first batch's loads)
                        const int mb = g >> 2, e = g & 3, u = g % ZR;
                        const bool rok = row0 + mb * 16 + Mfma<T>::row(q, e) < p.nrows;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            T z = TWO ? za[u][nb] * zb[TWO ? u : 0][nb] * w[nb] : za[u][nb] * w[nb];
                            z = rok ? z : T(0);
                            accrow[nb] += (double)(z * acc[mb][nb][e]);
                        }
                    }
                };
                if (two)
                    rows(std::integral_constant<bool, true>());
                else
                    rows(std::integral_constant<bool, false>());
            }
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = acc_t{};
        } else if (FLUSH64) {
            // The item's tile, weighted by its outer multiplier (from the
            // factor values buffered with its last step), joins the fp64 sums
            // (the product formed in fp64).
            T w[NB];
            multiplier(wq, w);
            double wd[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) wd[nb] = (double)w[nb];
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc64[mb][nb][e] =
                            __builtin_fma((double)acc[mb][nb][e], wd[nb], acc64[mb][nb][e]);
                    acc[mb][nb] = acc_t{};
                }
        }
    };

    // ---- main loop: steps over (item, k-chunk); the loads of the next PD
    // steps are in flight while a step runs on the matrix cores ----
    constexpr int PD = tile_prefetch(sizeof(T), MB, NB, FORM1, S, RC, W);
    T abuf[PD + 1][NA];
    T wbuf[PD + 1][SS][NB];
    LoadCursor lc;
    lc.base = 0;  // with every offset out of range until an item is entered
#pragma unroll
    for (int v = 0; v < NV; ++v) lc.vo[v] = kOOB;
#pragma unroll
    for (int j = 0; j < 3; ++j) lc.orow[j] = 0;
    lc.it = (int)fdiv((uint32_t)(g_lo + s_lo), fd_nkc);
    lc.kc = g_lo + s_lo - lc.it * nkc;
    lc.step = s_lo;
    lc.live = false;
    enter_item(lc);
    // compute cursor
    int c_it = lc.it, c_kc = lc.kc, c_step = s_lo;
    int64_t c_row0 = 0, c_orow[3] = {0, 0, 0};
    auto compute_item = [&]() {  // form 1: first row and outer rows of item c_it
        const Item itm = decode_item(p, c_it, unit_off, ROWS, FORM1);
        c_row0 = itm.row0;
#pragma unroll
        for (int j = 0; j < 3; ++j) c_orow[j] = j < p.nouter ? itm.oidx[j] * R : 0;
    };
    if (FORM1 && nsteps > 0) compute_item();

    // ---- stage the contraction-side Khatri-Rao tile B(kbase + k, r0:r0+BN)
    // in LDS, rows past the chunk zero-filled to a multiple of 16.  A thread
    // owns VW consecutive columns (16 bytes) of every RPP-th row; SP rows are
    // loaded before any is stored (one memory round trip per SP * RPP rows).
    // Factor values are read with buffer loads, elements outside the chunk or
    // the rank range at an offset past the descriptor (they read as zero),
    // so no load sits under a branch; a two-factor tile takes one index
    // division per row.  The tensor loads of the first PD steps are issued
    // right after the first batch's factor loads: loads return in order, so
    // that batch's stores wait for the factor values only, while the tensor
    // loads stay in flight. ----
    {
        constexpr int VW = 16 / (int)SZ;
        constexpr int TPR = BN / VW;  // threads per tile row
        static_assert(NT % TPR == 0, "tile row split over whole threads");
        constexpr int RPP = NT / TPR;  // rows per pass
        constexpr int SP = 8;          // rows per thread per batch
        typedef typename std::conditional<sizeof(T) == 8, dx2, fx4>::type vec_t;
        const int scol = (tid % TPR) * VW;
        const int srow = tid / TPR;
        const int nstage = (int)(nkc * 16);
        const bool two = p.Uk1 != nullptr;
        const unsigned IkB = (unsigned)p.IkB;
        // Descriptors: the first factor from the chunk's first row on, the
        // second (if any) whole; spans are kept below 2^31 bytes by the planner.
        const int64_t ia0 = two ? kbase / (int64_t)IkB : kbase;
        const int64_t na = two ? p.K / (int64_t)IkB : p.K;
        const __amdgpu_buffer_rsrc_t ra =
            make_rsrc(reinterpret_cast<const T *>(p.Uk0) + ia0 * R, (na - ia0) * R * (int64_t)SZ);
        const __amdgpu_buffer_rsrc_t rb2 =
            make_rsrc(two ? p.Uk1 : p.Uk0, two ? (int64_t)IkB * R * (int64_t)SZ : 0);
        unsigned cofs[VW];
        bool cok[VW];
#pragma unroll
        for (int v = 0; v < VW; ++v) {
            cok[v] = r0 + scol + v < R;
            cofs[v] = (unsigned)((r0 + scol + v) * SZ);
        }
        auto stage = [&](auto two_c, auto vec_c) {
            constexpr bool TWO = decltype(two_c)::value;
            constexpr bool V16 = decltype(vec_c)::value;
            T sv[SP][VW];
            auto load_batch = [&](int rbase) {
#pragma unroll
                for (int j = 0; j < SP; ++j) {
                    const int kk = rbase + j * RPP + srow;
                    const bool rok = kk < Kloc;
                    const unsigned kg = (unsigned)(kbase + kk);
                    const unsigned ia = TWO ? fdiv(kg, p.fd_IkB) : kg;
                    const unsigned ib = TWO ? kg - ia * IkB : 0u;
                    const unsigned oa = (unsigned)((int64_t)(ia - (unsigned)ia0) * R * SZ);
                    const unsigned ob = (unsigned)((int64_t)ib * R * SZ);
                    if (V16) {
                        // R is a multiple of VW: a 16-byte group is wholly in or out.
                        const bool ok = rok && cok[0];
                        const vec_t xa = __builtin_bit_cast(
                            vec_t, __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? oa + cofs[0] : kOOB, 0, 0));
                        vec_t xb;
                        if (TWO)
                            xb = __builtin_bit_cast(vec_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                               rb2, ok ? ob + cofs[0] : kOOB, 0, 0));
#pragma unroll
                        for (int v = 0; v < VW; ++v) sv[j][v] = TWO ? xa[v] * xb[v] : xa[v];
                    } else {
#pragma unroll
                        for (int v = 0; v < VW; ++v) {
                            const bool ok = rok && cok[v];
                            T x = bload1(ra, ok ? oa + cofs[v] : kOOB, 0, T(0));
                            if (TWO) x *= bload1(rb2, ok ? ob + cofs[v] : kOOB, 0, T(0));
                            sv[j][v] = x;
                        }
                    }
                }
            };
            auto store_batch = [&](int rbase) {
#pragma unroll
                for (int j = 0; j < SP; ++j) {
                    const int kk = rbase + j * RPP + srow;
                    if (kk < nstage) {
                        vec_t t;
#pragma unroll
                        for (int v = 0; v < VW; ++v) t[v] = sv[j][v];
                        *reinterpret_cast<vec_t *>(&Bs[kk * p.bpitch + scol]) = t;
                    }
                }
            };
            // First batch, then the tensor loads of the first PD steps, then
            // the first batch's stores (which wait for its loads only).
            load_batch(0);
            asm volatile("" ::: "memory");
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                load_step(abuf[u], wbuf[u], lc);
                advance(lc);
            }
            store_batch(0);
            for (int rbase = SP * RPP; rbase < nstage; rbase += SP * RPP) {
                load_batch(rbase);
                store_batch(rbase);
            }
        };
        typedef std::integral_constant<bool, true> yes;
        typedef std::integral_constant<bool, false> no;
        const bool v16 = (R % VW) == 0;
        if (!stage_b) {
            // B is in LDS already: only the tensor loads of the first steps.
#pragma unroll
            for (int u = 0; u < PD; ++u) {
                load_step(abuf[u], wbuf[u], lc);
                advance(lc);
            }
        } else if (two) {
            if (v16) stage(yes(), yes()); else stage(yes(), no());
        } else {
            if (v16) stage(no(), yes()); else stage(no(), no());
        }
    }
    __syncthreads();

    // After each step: reduce the item when it ends or when the wave's
    // range ends inside it.
    auto after_compute = [&](T (*wq)[NB]) {
        ++c_step;
        const bool item_end = ++c_kc == nkc;
        if (c_step <= s_hi && (item_end || c_step == s_hi)) {
            finish_item(c_row0, c_orow, wq);
            if (item_end) {
                c_kc = 0;
                ++c_it;
                if (FORM1 && c_step < s_hi) compute_item();
            }
        }
    };

    // PD + 1 steps per iteration over a ring of PD + 1 register buffers
    // indexed by compile-time constants, so each buffer keeps its own
    // registers.  Steps past the wave's range load zeros and skip the
    // matrix cores.
    for (int t = 0; t < nsteps; t += PD + 1) {
#pragma unroll
        for (int u = 0; u <= PD; ++u) {
            load_step(abuf[(u + PD) % (PD + 1)], wbuf[(u + PD) % (PD + 1)], lc);
            advance(lc);
            if (c_step < s_hi) compute_step(abuf[u], c_kc, wbuf[u]);
            after_compute(wbuf[u]);
        }
    }

    // ---- a split reduction of another mode (all-mode sweep) ----
    // Done here, before the workgroup barrier, so that waves which finish
    // their steps early do it while the others still run.  Thread gid takes
    // group g = gid mod NG of output gid / NG and sums partials g, g + NG, ...
    // in blocks of eight (as split_reduce_kernel does); the NG group sums of
    // an output sit in consecutive lanes and are added in group order.
    // The partials are read through a buffer descriptor (their span is below
    // 2^31 bytes): a slot past the last split reads as zero, so the eight
    // loads of a block go out together with no branch.
    if (p.pend_partial != nullptr) {
        const int NGp = p.pend_ng;  // 4 or 16
        const int lg = NGp == 16 ? 4 : 2;
        const int64_t total = p.pend_count * NGp;
        const int64_t stride = p.grid_real * (int64_t)NT;
        const int64_t npass = (total + stride - 1) / stride;
        const __amdgpu_buffer_rsrc_t rp =
            make_rsrc(p.pend_partial, p.pend_nsplit * p.pend_count * (int64_t)sizeof(double));
        for (int64_t k = 0; k < npass; ++k) {
            const int64_t gid = k * stride + logical * NT + tid;
            const bool ok = gid < total;
            const int64_t i = ok ? (gid >> lg) : 0;
            const int g = (int)(gid & (NGp - 1));
            double v = 0.0;
            for (int64_t s0 = g; s0 < p.pend_nsplit; s0 += 8 * NGp) {
                double t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int64_t sp = s0 + (int64_t)u * NGp;
                    const unsigned off =
                        (ok && sp < p.pend_nsplit) ? (unsigned)((sp * p.pend_count + i) * 8) : kOOB;
                    t[u] = bload1(rp, off, 0u, 0.0);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) v += t[u];
            }
            // every shuffle is issued before the sums are added (in group order)
            double tot = v;
            auto combine = [&](auto ng_c) {
                constexpr int NG = decltype(ng_c)::value;
                double o[NG];
#pragma unroll
                for (int j = 1; j < NG; ++j) o[j] = __shfl(v, (lane & ~(NG - 1)) + j);
#pragma unroll
                for (int j = 1; j < NG; ++j) tot += o[j];
            };
            if (NGp == 16)
                combine(std::integral_constant<int, 16>());
            else
                combine(std::integral_constant<int, 4>());
            if (ok && g == 0) reinterpret_cast<T *>(p.pend_out)[i] = (T)tot;
        }
    }

    // ---- workgroup reduction and store ----
    const bool split_out = p.to_partial != 0;
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
            for (int w2 = 1; w2 < W; ++w2) v += red[w2 * BN + tid];
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
        auto add_val = [&](int mb, int nb, int e, double x) {
            if (FLUSH64)
                acc64[FLUSH64 ? mb : 0][FLUSH64 ? nb : 0][FLUSH64 ? e : 0] += x;
            else
                acc[mb][nb][e] += (T)x;
        };
        constexpr int SLOT = MB * NB * 4 * 64;
        // Output element (mb, nb, e) of lane ln: its row and column.
        auto put = [&](int mb, int nb, int e, int ln, double v) {
            const int64_t c = r0 + nb * 16 + (ln & 15);
            int64_t row;
            if (!RC)
                row = out_row0 + mb * 16 + Mfma<T>::row(ln >> 4, e);
            else
                row = out_row0 + 16 * RL * (mb / RL) + RL * Mfma<T>::row(ln >> 4, e) + (mb % RL);
            if (row < p.In && c < R) {
                if (split_out) {
                    p.partial[(split * p.In + row) * R + c] = v;
                } else if (p.out64) {
                    reinterpret_cast<double *>(p.out)[row * R + c] = v;
                } else {
                    reinterpret_cast<T *>(p.out)[row * R + c] = (T)v;
                }
            }
        };
        if (p.red_all) {
            // Every wave writes its tile to a slot of its own; after one barrier
            // each thread adds the W slots of its elements in wave order and
            // stores them, so the store is spread over the whole workgroup.
            static_assert(SLOT % NT == 0, "slot split over whole threads");
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        red[wave * SLOT + ((mb * NB + nb) * 4 + e) * 64 + lane] = val(mb, nb, e);
            __syncthreads();
#pragma unroll
            for (int k = 0; k < SLOT / NT; ++k) {
                const int i = k * NT + tid;
                double v = red[i];
#pragma unroll
                for (int w2 = 1; w2 < W; ++w2) v += red[w2 * SLOT + i];
                const int g = i >> 6;
                put(g / (4 * NB), (g >> 2) % NB, g & 3, i & 63, v);
            }
        } else {
            // Fixed-order pairwise tree over the waves: in the round with h
            // slots, waves h..2h-1 write their sums and waves 0..h-1 add them, so
            // W waves take log2(W) rounds and W/2 slots of LDS.
#pragma unroll
            for (int h = W / 2; h >= 1; h /= 2) {
                if (wave >= h && wave < 2 * h) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                red[(wave - h) * SLOT + ((mb * NB + nb) * 4 + e) * 64 + lane] =
                                    val(mb, nb, e);
                }
                __syncthreads();
                if (wave < h) {
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                add_val(mb, nb, e,
                                        red[wave * SLOT + ((mb * NB + nb) * 4 + e) * 64 + lane]);
                }
                if (h > 1) __syncthreads();
            }
            if (wave == 0) {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) put(mb, nb, e, lane, val(mb, nb, e));
            }
        }
    }
}

template <typename T, int MB, int NB, bool RC, bool VEC, bool FORM1, int W, int S>
__global__ __launch_bounds__(64 * W, (tile_occupancy(sizeof(T), MB, NB, FORM1, S, RC, W))) void
mttkrp_tile_kernel(KParams p)
{
    extern __shared__ __align__(16) unsigned char smem[];
    tile_pass<T, MB, NB, RC, VEC, FORM1, W, S>(p, smem, true, 0);
}

// Two form-1 modes whose plans share the contraction group, the chunking,
// the rank tiles and the workgroup decomposition (so every workgroup needs
// the same B tile in both), one after the other in each workgroup of a
// single launch: the B tile is staged once, and the second mode's work does
// not wait for the first mode's last workgroups.  The reduction space sits
// after the B tile.  (The passes are written out, not indexed at run time,
// so the parameter blocks stay in scalar registers.)
template <typename T, int MB, int NB, bool VEC, int W>
__global__ __launch_bounds__(64 * W, (tile_min_waves(sizeof(T), MB, NB, true, 0))) void
mttkrp_tile_multi_kernel(KPack pk)
{
    extern __shared__ __align__(16) unsigned char smem[];
    tile_pass<T, MB, NB, false, VEC, true, W, 0>(pk.p[0], smem, true, pk.red_off);
    __syncthreads();
    tile_pass<T, MB, NB, false, VEC, true, W, 0>(pk.p[1], smem, false, pk.red_off);
}

}  // namespace mttkrp
