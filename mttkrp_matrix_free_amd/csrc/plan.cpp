// Host planner for the matrix-free MTTKRP (pure host code, no HIP calls).
//
// Chooses, for one mode, the contraction group run on the matrix cores, the
// tile rows, the outer (Hadamard) modes, the wave tile, and the split of the
// work over workgroups.  The split rule follows a plain cache/traffic model:
// X is streamed once per rank tile; a split adds 2 * nsplit * I_n * R * 8
// bytes of partial sums, kept under an eighth of the tensor traffic; the grid
// is sized to fill whole rounds of the workgroups the chip holds at once.
// (The GenTen page names a tile-size heuristic and cache models for this
// choice; their formulas are not given, so this is a reading for gfx950:
// 160 KB LDS and 512 registers per lane per SIMD.)
#include "plan.hpp"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mttkrp.h"

namespace mttkrp {

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t &out)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    out = a * b;
    return true;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// MTTKRP_FORCE_TILE="mb,nb" or "mb,nb,waves" (experiments only).  Returns 0
// when unset, 1 with the values when well formed, -1 otherwise.
int forced_tile(int &mb, int &nb, int &waves)
{
    const char *v = std::getenv("MTTKRP_FORCE_TILE");
    if (!v || !*v) return 0;
    int a = 0, b = 0, w = 0;
    char tail = 0;
    const int got = std::sscanf(v, "%d,%d,%d%c", &a, &b, &w, &tail);
    if (got == 2 || got == 3) {
        if ((a == 2 || a == 4) && (b == 1 || b == 2 || b == 4 || b == 8) &&
            (got == 2 || w == 4 || w == 8)) {
            mb = a;
            nb = b;
            waves = got == 3 ? w : 0;
            return 1;
        }
    }
    return -1;
}

}  // namespace

int make_plan(const int64_t *dims, int order, int64_t rank, int mode, int elem_bytes, Plan &plan)
{
    if (!dims) return MTTKRP_EINVAL;
    if (order < 3 || order > kMaxOrder) return MTTKRP_EORDER;
    if (rank < 1 || mode < 0 || mode >= order) return MTTKRP_EINVAL;
    if (elem_bytes != 4 && elem_bytes != 8) return MTTKRP_EINVAL;
    for (int m = 0; m < order; ++m)
        if (dims[m] < 1) return MTTKRP_EINVAL;

    // Sizes: every element offset and every workspace byte count must fit in
    // int64 with room for the kernels' index arithmetic.
    int64_t N = 1;
    for (int m = 0; m < order; ++m)
        if (!mul_ok(N, dims[m], N)) return MTTKRP_ERANGE;
    int64_t tmp;
    if (!mul_ok(N, 8, tmp) || tmp > (INT64_C(1) << 50)) return MTTKRP_ERANGE;
    for (int m = 0; m < order; ++m)
        if (!mul_ok(dims[m], rank, tmp) || !mul_ok(tmp, 8 * 1024, tmp)) return MTTKRP_ERANGE;
    if (rank > (INT64_C(1) << 24)) return MTTKRP_ERANGE;

    const int d = order;
    const int n = mode;
    int64_t S[kMaxOrder];
    {
        int64_t s = 1;
        for (int m = d - 1; m >= 0; --m) {
            S[m] = s;
            s *= dims[m];
        }
    }

    Plan p;
    p.elem_bytes = elem_bytes;
    KParams &k = p.kp;
    k.R = rank;
    k.In = dims[n];
    k.r_mode0 = k.r_mode1 = -1;
    k.k_mode0 = k.k_mode1 = -1;
    k.IkB = 1;
    k.IrB = 1;

    bool in_k[kMaxOrder] = {false, false, false, false, false};
    bool in_rows[kMaxOrder] = {false, false, false, false, false};

    // A contraction mode shorter than 32 is merged with its left neighbour
    // (when that neighbour is free) so that the matrix-core K dimension is not
    // mostly padding; the merged Khatri-Rao tile must fit in LDS at one
    // 16-column rank block.
    // fp32 at rank 64 and above also merges a last mode of at most 64 into a
    // long contraction, chunked through LDS: an item then spans a chunk of
    // many steps instead of 4, so its per-item work (decode, the multiplier,
    // the fp64 flush) is spread over more matrix-core work (4-way fp32
    // tensor: rank 512 modes 0-1 -5%, rank 64 mode 1 -5%; at rank 64 the
    // output mode with a 4 MiB row stride lost 4%, so that case keeps the
    // short contraction).
    const int64_t kMergeMax = (int64_t)(kLdsBudget / ((16 + 8) * (size_t)elem_bytes));
    auto choose_k = [&](int last) {
        int first = last;
        const bool free_left = last - 1 >= 0 && last - 1 != n;
        const bool short_last =
            free_left && dims[last] < 32 && dims[last - 1] * dims[last] <= kMergeMax;
        const bool long_fp32 = elem_bytes == 4 && dims[last] <= 64 && rank >= 64 &&
                               (rank >= 128 || S[n] <= (INT64_C(1) << 16));
        if (free_left && (short_last || long_fp32)) first = last - 1;
        if (first == last) {
            k.k_mode0 = last;
            k.K = dims[last];
        } else {
            k.k_mode0 = first;
            k.k_mode1 = last;
            k.IkB = dims[last];
            k.K = dims[first] * dims[last];
        }
        k.k_stride = S[last];
        for (int m = first; m <= last; ++m) in_k[m] = true;
        return first;
    };

    // Trailing rows: when the output is the unit-stride mode and shorter than
    // a 64-row tile, or the second-to-last mode while the last mode is too
    // short to be a contraction on its own, the tile rows are the contiguous
    // block of the last two modes (rows have unit stride), the contraction
    // runs over the mode before them (merged with its left neighbour when it
    // is not a multiple of 16), and the reduction pass contracts the row mode
    // that is not the output against its factor.
    // (Tiny tensors keep the plain plan: the extra reduction launch would
    // cost more than the padded rows.)
    const bool trailing = d >= 3 && N >= (INT64_C(1) << 20) &&
                          ((n == d - 1 && dims[d - 1] < 64) || (n == d - 2 && dims[d - 1] < 32));
    k.tr = 0;
    k.tr_div = 0;
    k.tr_inner = 1;
    k.tr_J = 1;
    k.In_out = dims[n];
    if (trailing) {
        p.layout = 1;
        p.form = 0;
        const int last = d - 3;
        int first = last;
        if ((dims[last] % 16 != 0 || dims[last] < 32) && last - 1 >= 0) first = last - 1;
        k.k_mode0 = first;
        k.K = dims[last];
        if (first != last) {
            k.k_mode1 = last;
            k.IkB = dims[last];
            k.K = dims[first] * dims[last];
        }
        k.k_stride = S[last];
        for (int m = first; m <= last; ++m) in_k[m] = true;
        k.nrows = dims[d - 2] * dims[d - 1];
        k.row_stride = 1;
        in_rows[d - 2] = in_rows[d - 1] = true;
        k.tr = 1;
        k.tr_inner = dims[d - 1];
        k.tr_div = n == d - 2;
        p.red_mode = n == d - 2 ? d - 1 : d - 2;
        k.tr_J = dims[p.red_mode];
        k.In = k.nrows;  // the kernel's rows are the block
    } else if (n == d - 1) {
        // Output mode has unit stride: tile rows are the output rows.
        p.layout = 1;
        p.form = 0;
        choose_k(d - 2);
        k.nrows = dims[n];
        k.row_stride = 1;
        in_rows[n] = true;
    } else {
        p.layout = 0;
        const int kq = choose_k(d - 1);
        // Tile rows: the free mode nearest the contraction group on its left
        // (skipping the output mode), merged with the next free mode to its
        // left when it is shorter than 64 rows.  The two need not be adjacent
        // (the output mode may sit between them): row r = (ia, ib) is then
        // addressed as ia * stride_a + ib * stride_b.
        int rlast = -1;
        for (int m = kq - 1; m >= 0 && rlast < 0; --m)
            if (m != n) rlast = m;
        // At high rank the per-tile row reduction of form 1 (one factor load
        // and one fma per accumulator element) costs more than scaling the
        // contraction tile by the outer multiplier, so the output rows become
        // the tile rows (form 0).  That reduction runs on the vector ALUs,
        // which do not overlap the matrix cores, and it weighs twice as much
        // against fp32 MFMAs as against fp64 ones: fp32 takes form 0 already
        // at rank 64, and at lower rank when the output rows lie close
        // together (stride up to 2^16 elements; measured on the 4-way fp32
        // tensor: R=64 modes 0-2 258 -> 202-218 us, R=8 modes 1-2 -15/-23%).
        if (rank >= 256 || (elem_bytes == 4 && (rank >= 64 || S[n] <= (INT64_C(1) << 16))))
            rlast = -1;
        if (rlast >= 0) {
            p.form = 1;
            int rfirst = rlast;
            if (dims[rlast] < 64)
                for (int m = rlast - 1; m >= 0 && rfirst == rlast; --m)
                    if (m != n) rfirst = m;
            k.r_mode0 = rfirst;
            k.nrows = dims[rlast];
            k.IrB = dims[rlast];
            k.row_stride = S[rlast];
            k.row_stride_a = S[rfirst];
            k.row_split = 0;
            if (rfirst != rlast) {
                k.r_mode1 = rlast;
                k.nrows = dims[rfirst] * dims[rlast];
                k.row_split = rfirst != rlast - 1 ? 1 : 0;
            }
            in_rows[rfirst] = in_rows[rlast] = true;
        } else {
            // The output rows are the tile rows; every other mode is contracted
            // or outer.
            p.form = 0;
            k.nrows = dims[n];
            k.row_stride = S[n];
            in_rows[n] = true;
        }
    }

    // Outer modes: everything else except the output mode (and the rows).
    k.nouter = 0;
    k.nbatch = 1;
    for (int m = 0; m < d; ++m) {
        if (in_k[m] || in_rows[m] || m == n) continue;
        k.o_mode[k.nouter] = m;
        k.o_dim[k.nouter] = dims[m];
        k.o_stride[k.nouter] = S[m];
        k.nbatch *= dims[m];
        ++k.nouter;
    }
    for (int j = k.nouter; j < 3; ++j) {
        k.o_mode[j] = -1;
        k.o_dim[j] = 1;
        k.o_stride[j] = 0;
    }
    k.n_stride = S[n];

    // Vectorised loads need every 4-element group inside the tensor and
    // aligned with the row/fibre starts.
    if (p.layout == 0)
        p.vec = (k.K % 4 == 0) && (k.row_stride % 4 == 0) &&
                (!k.row_split || k.row_stride_a % 4 == 0);
    else
        p.vec = (k.nrows % 4 == 0) && (k.k_stride % 4 == 0);
    if (p.layout == 0) {
        for (int j = 0; j < k.nouter; ++j)
            if (k.o_stride[j] % 4 != 0) p.vec = false;
        if (p.form == 1 && k.n_stride % 4 != 0) p.vec = false;
    } else {
        for (int j = 0; j < k.nouter; ++j)
            if (k.o_stride[j] % 4 != 0) p.vec = false;
    }

    // Wave tile: mb x 16 rows, nb x 16 rank columns.  Wide rank tiles (nb = 8)
    // reuse each tensor element for 128 columns when the rank is large; the
    // row tile is 32 rows unless there is work for many more waves than the
    // chip holds.
    // fp32 form-0 tiles keep an fp64 copy of their accumulators, so eight
    // rank blocks leave one wave per SIMD; four blocks with two waves per
    // SIMD keep the matrix cores busier even though X is then read once per
    // 64 rank columns (measured on the 4-way fp32 rank-512 tensor: -19%).
    const int64_t ncb = ceil_div(rank, 16);  // 16-wide rank blocks
    // (fp64 form-0 tiles stay at four blocks too: on the 512^3 rank-2000
    // tensor, modes 0 and 1 took 8.2 ms with four blocks against 9.3 ms with
    // eight, whose registers leave one wave per SIMD.)
    const bool wide_ok =
        p.form == 1 ? elem_bytes == 4
                    : tile_min_waves(elem_bytes, 2, 8, false, plan_slots(0, k.nouter)) == 2;
    if (ncb >= 8 && p.layout == 0 && wide_ok)
        p.nb = 8;
    else
        p.nb = ncb >= 4 ? 4 : (ncb >= 2 ? 2 : 1);
    if (p.layout == 1) {
        p.mb = 4;
        // Trailing-rows tiles (a short block of rows, many contraction steps)
        // keep the matrix cores fed only with two waves per SIMD.  When four
        // rank blocks of 64 rows do not fit the registers for that, 32-row
        // tiles with four rank blocks are taken: every 64 rank columns then
        // read X once, and a short row block is padded less (200 rows: 224
        // instead of 256).  Failing that, 64-row tiles with two rank blocks.
        const int sl = plan_slots(0, k.nouter);
        if (k.tr && p.nb == 4 && tile_min_waves(elem_bytes, 4, 4, false, sl) == 1) {
            if (tile_min_waves(elem_bytes, 2, 4, false, sl) == 2)
                p.mb = 2;
            else if (tile_min_waves(elem_bytes, 4, 2, false, sl) == 2)
                p.nb = 2;
        }
        // Other row-contiguous plans (the output is the unit-stride mode)
        // take two rank blocks: a 64 x 32 tile feeds its MFMAs from fewer
        // registers per step than 64 x 64 (tile sweep: 512^3 rank 2000 mode 2
        // 8.57 -> 8.37 ms, 4-way fp32 rank 64 mode 3 190 -> 176 us).
        if (!k.tr && p.nb > 2) p.nb = 2;
    } else if (p.nb > 4) {
        p.mb = 2;
    } else if (p.form == 1) {
        // (256^3 rank 32 keeps 32-row tiles: 64-row ones won 1-2% per mode
        // alone but lost 2-4% in the all-mode sweep)
        const int64_t tiles64 = k.In * k.nbatch * ceil_div(k.nrows, 64);
        p.mb = (p.nb <= 2 && tiles64 >= 8192) ? 4 : 2;
    } else {
        // (fp32 single-block tiles are 32 rows: tile sweep, 4-way fp32 rank
        // 8 modes 1-2, 110 / 115 us against 114 / 117 us for 64 rows)
        p.mb = (k.In >= 64 && p.nb <= 2 && !(elem_bytes == 4 && p.nb == 1)) ? 4 : 2;
    }

    // Experiments: a forced wave tile (and workgroup size) replaces the
    // choice above; everything below follows from it.
    int f_mb = 0, f_nb = 0, f_waves = 0;
    const int forced = forced_tile(f_mb, f_nb, f_waves);
    if (forced < 0) return MTTKRP_EINVAL;
    if (forced > 0) {
        p.mb = f_mb;
        p.nb = f_nb;
    }

    // Workgroup size: form 1 and the row-contiguous layout run eight waves per
    // workgroup (when a wave's registers allow two waves per SIMD), one
    // workgroup per compute unit, so one staged Khatri-Rao tile serves the
    // whole unit and fewer splits (partial sums) are needed -- when that tile
    // is big enough (32 KiB) for its staging to matter; otherwise four waves,
    // two workgroups per compute unit, which interleave better with the other
    // stream's launch in an all-mode sweep (4-way fp32 rank 8: 442 -> 414 us).
    const bool big_b = ceil_div(k.K, 16) * 16 * (16 * p.nb + 4) * elem_bytes >= 32 * 1024;
    p.waves = ((p.form == 1 || p.layout == 1) && big_b &&
               tile_min_waves(elem_bytes, p.mb, p.nb, p.form == 1, plan_slots(p.form, k.nouter)) == 2)
                  ? 8
                  : 4;
    // Rank-tiled fp64 row-contiguous plans with the 64 x 32 tile: four-wave
    // workgroups, three per compute unit (tile_three_waves), once the rank
    // makes them matrix-core bound
    if (elem_bytes == 8 && p.form == 0 && p.layout == 1 && p.mb == 4 && p.nb == 2 &&
        plan_slots(p.form, k.nouter) == 1 && rank >= 256)
        p.waves = 4;
    if (forced > 0 && f_waves) p.waves = f_waves;
    const int occ = tile_occupancy(elem_bytes, p.mb, p.nb, p.form == 1,
                                   plan_slots(p.form, k.nouter), p.layout == 1, p.waves);
    const size_t lds_budget = p.waves == 8 ? kLdsBudgetWide
                              : occ == 3   ? kLdsBudgetThree
                                           : kLdsBudget;

    // Contraction chunks: the Khatri-Rao tile of one chunk (Kc x 16nb) must
    // fit in the workgroup's LDS; longer contractions are split into chunks
    // whose results are summed by the reduction pass.
    // LDS pitch of B rows: a lane group of four reads rows 4 apart, so the
    // pitch is padded (4 elements) to put those rows on different banks.
    // In the row-contiguous layout the four lane groups read consecutive
    // rows instead: for fp32 a pitch of 16 (mod 32) elements puts each pair
    // of groups on disjoint banks (with a pad of 4, the 4-way fp32 R=64 mode-3
    // kernel stalled half a cycle per MFMA on bank conflicts).
    const int bpitch =
        16 * p.nb + ((p.layout == 1 && elem_bytes == 4) ? (p.nb % 2 ? 32 : 16) : 4);
    const int64_t Kpad = ceil_div(k.K, 16) * 16;
    const int64_t kc_max = (int64_t)(lds_budget / ((size_t)bpitch * elem_bytes)) / 16 * 16;
    if (kc_max < 16) return MTTKRP_ERANGE;
    k.Kc = std::min<int64_t>(Kpad, kc_max);
    k.nkch = ceil_div(k.K, k.Kc);
    k.bpitch = bpitch;
    p.b_in_lds = true;

    // Work decomposition.
    const int64_t rows_per_tile = 16 * p.mb;
    k.nrtiles = ceil_div(rank, 16 * p.nb);
    if (p.form == 1) {
        k.nunits = k.In;
        k.nrowtiles = ceil_div(k.nrows, rows_per_tile);
        k.nitems = k.nbatch * k.nrowtiles;
    } else {
        k.nunits = ceil_div(k.In, rows_per_tile);
        k.nrowtiles = 1;
        k.nitems = k.nbatch;
    }
    // Split the work items of a unit so that the grid holds eight waves per
    // compute unit (sixteen when the staged Khatri-Rao tile is small, so that
    // restaging it is cheap), while the partial sums (written and read once
    // each) stay under an eighth of the tensor traffic.  The waves of a
    // workgroup share its steps evenly, so a chunk may hold any number of
    // items.
    const size_t b_tile = (size_t)k.Kc * k.bpitch * elem_bytes;
    // Workgroups resident at once: by waves (one to three per SIMD, the
    // instantiation's occupancy) and by LDS.  A grid that needs a second, partial round
    // leaves most of the chip idle in it, so the split is rounded down to
    // whole rounds.
    const int slots = plan_slots(p.form, k.nouter);
    const int per_cu_waves = 4 * occ;
    // Cross-wave reduction space: one row of column sums per wave (form 1);
    // for form 0 every wave's tile of fp64 sums when that fits the LDS budget
    // (one round, the store spread over the workgroup), else W/2 tiles (a
    // pairwise tree over the waves).
    const size_t wave_tile = (size_t)rows_per_tile * 16 * p.nb * 8;
    k.red_all = (p.form == 0 && (size_t)p.waves * wave_tile <= lds_budget) ? 1 : 0;
    const size_t red = p.form == 1 ? (size_t)p.waves * 16 * p.nb * 8
                                   : (size_t)(k.red_all ? p.waves : p.waves / 2) * wave_tile;
    const size_t lds_est = std::max((size_t)k.Kc * k.bpitch * elem_bytes, red);
    const int64_t per_cu = std::max<int64_t>(
        1, std::min<int64_t>(per_cu_waves / p.waves, (int64_t)(160 * 1024 / lds_est)));
    const int64_t resident = per_cu * kNumCU;
    p.per_cu = (int)per_cu;
    (void)b_tile;
    // The split that best fills whole rounds of resident workgroups (the
    // smallest one among equals), up to two rounds' worth.  Form 0 cuts the
    // unit's sequence of (item, step) pairs into equal ranges, not whole
    // items, so every workgroup of a round has the same work (each range
    // keeps at least two steps per wave; 5-way trailing rows: 50 items in 6
    // ranges, 90 -> 87 us).  Form 1 keeps whole items per range: every item a
    // range touches costs a row reduction (5-way modes 0-2: +4% otherwise).
    // Trailing-rows plans have few units and few, long items (the outer
    // tuples): their contraction is cut into more chunks than LDS requires
    // when that fills the rounds better (fewer chunks among equals).
    // (Each chunk count is paired with the best split of the items into
    // 1..4 step ranges, up to two rounds of workgroups; among equal fills the
    // fewest partial outputs win, and among those the shortest chunks, whose
    // B tiles are the quickest to stage.)
    if (k.tr) {
        int64_t best_kc = k.Kc, best_parts = 0;
        double best_u = -1.0;
        const int64_t nk0 = k.nkch;
        for (int64_t nk = nk0; nk <= std::max<int64_t>(nk0, 64); ++nk) {
            const int64_t kc = ceil_div(ceil_div(k.K, nk), 16) * 16;
            const int64_t nke = ceil_div(k.K, kc);
            for (int64_t w = 1; w <= 4; ++w) {
                const int64_t g = k.nunits * k.nrtiles * nke * w;
                if (g > 2 * resident && !(nk == nk0 && w == 1)) continue;
                const double u = (double)g / (double)(ceil_div(g, resident) * resident);
                if (u > best_u + 0.01 || (u > best_u - 0.01 && nke * w <= best_parts)) {
                    best_u = std::max(best_u, u);
                    best_kc = kc;
                    best_parts = nke * w;
                }
            }
        }
        k.Kc = best_kc;
        k.nkch = ceil_div(k.K, k.Kc);
    }
    const int64_t base = k.nunits * k.nrtiles * k.nkch;
    const int64_t unit_steps = k.nitems * (k.Kc / 16);
    int64_t want = 1;
    {
        const int64_t wmax =
            p.form == 1
                ? std::max<int64_t>(1, std::min<int64_t>(k.nitems, ceil_div(2 * resident, base)))
                : std::max<int64_t>(1, std::min<int64_t>(unit_steps / (2 * p.waves),
                                                         ceil_div(2 * resident, base)));
        auto util = [&](int64_t w) {
            const int64_t g =
                p.form == 1 ? base * ceil_div(k.nitems, ceil_div(k.nitems, w)) : base * w;
            return (double)g / (double)(ceil_div(g, resident) * resident);
        };
        double best = 0.0;
        for (int64_t w = 1; w <= wmax; ++w) best = std::max(best, util(w));
        for (int64_t w = 1; w <= wmax; ++w)
            if (util(w) >= best - 0.01) {
                want = w;
                break;
            }
    }
    const int64_t out_bytes = k.In * rank * 8;
    const int64_t cap_traffic = std::max<int64_t>(
        1, (N * elem_bytes / 8) / std::max<int64_t>(1, 2 * out_bytes * k.nkch));
    want = std::min<int64_t>(want, std::min<int64_t>(cap_traffic, 1024));
    if (p.form == 1) {
        k.chunk = std::max<int64_t>(1, ceil_div(k.nitems, want));  // items per workgroup
        k.nsplit_it = ceil_div(k.nitems, k.chunk);
    } else {
        k.nsplit_it = want;
        k.chunk = ceil_div(unit_steps, want);  // steps per workgroup (full contraction chunk)
    }
    k.nsplit = k.nsplit_it * k.nkch;
    k.grid_real = k.nunits * k.nsplit * k.nrtiles;
    k.grid_per_xcd = ceil_div(k.grid_real, kNumXCD);
    p.grid = k.grid_per_xcd * kNumXCD;
    if (p.grid > INT_MAX) return MTTKRP_ERANGE;

    // Buffer loads address a tile with 32-bit byte offsets below 2^31: the
    // span of one tile (its rows and its whole contraction) must fit.
    {
        int64_t span;
        if (p.layout == 0 && k.row_split)
            span = ((ceil_div(rows_per_tile, k.IrB) + 1) * k.row_stride_a +
                    k.IrB * k.row_stride + k.Kc) * elem_bytes;
        else if (p.layout == 0)
            span = ((rows_per_tile - 1) * k.row_stride + k.Kc) * elem_bytes;
        else
            span = (rows_per_tile + (k.Kc - 1) * k.k_stride) * elem_bytes;
        if (span >= (INT64_C(1) << 31) - 64) return MTTKRP_ERANGE;
        // The contraction factor rows one chunk stages are read the same
        // way: the first factor from the chunk's first row, the second whole.
        // The row factors of a form-1 reduction likewise.
        if (p.form == 1) {
            const int64_t na = k.r_mode1 >= 0 ? k.nrows / k.IrB : k.nrows;
            if ((na * rank + 16) * elem_bytes >= (INT64_C(1) << 31)) return MTTKRP_ERANGE;
            if (k.r_mode1 >= 0 && (k.IrB * rank + 16) * elem_bytes >= (INT64_C(1) << 31))
                return MTTKRP_ERANGE;
        }
        // Outer factors are read through descriptors over the whole factor.
        for (int j = 0; j < k.nouter; ++j)
            if ((k.o_dim[j] * rank + 16) * elem_bytes >= (INT64_C(1) << 31)) return MTTKRP_ERANGE;
        const int64_t rows_a = (k.k_mode1 >= 0) ? k.Kc / k.IkB + 2 : k.Kc;
        if ((rows_a * rank + 16) * elem_bytes >= (INT64_C(1) << 31)) return MTTKRP_ERANGE;
        if ((k.k_mode1 >= 0) && (k.IkB * rank + 16) * elem_bytes >= (INT64_C(1) << 31))
            return MTTKRP_ERANGE;
    }
    k.x_bytes = N * elem_bytes;

    // Index decode in 32 bits: every dividend and divisor below 2^31.
    {
        const int64_t lim = INT64_C(1) << 31;
        const int64_t nkc_full = k.Kc / 16;
        if (k.K >= lim || k.nrows >= lim || k.nbatch >= lim || k.nitems >= lim ||
            k.nitems * nkc_full + k.nsplit_it >= lim || k.IrB >= lim || k.IkB >= lim)
            return MTTKRP_ERANGE;
        const int64_t klast = k.K - (k.nkch - 1) * k.Kc;
        k.fd_nrtiles = make_fastdiv(k.nrtiles);
        k.fd_nunits = make_fastdiv(k.nunits);
        // Trailing-rows blocks need not be whole cache lines (the 5-way
        // tensor's 200-row fp64 block is 12.5 lines), so neighbouring row
        // tiles share lines.  Split-major order keeps every row tile of a
        // split on one XCD, where the shared lines are fetched once into its
        // L2 (unit-major order spread them over XCDs: 1.28x the tensor
        // fetched).
        k.split_major = k.tr ? 1 : 0;
        k.fd_nsplit = make_fastdiv(k.nsplit);
        k.fd_nsplit_it = make_fastdiv(k.nsplit_it);
        k.fd_nkc_full = make_fastdiv(nkc_full);
        k.fd_nkc_last = make_fastdiv((klast + 15) / 16);
        k.fd_nrowtiles = make_fastdiv(k.nrowtiles);
        k.fd_odim1 = make_fastdiv(k.o_dim[1]);
        k.fd_odim2 = make_fastdiv(k.o_dim[2]);
        k.fd_IrB = make_fastdiv(k.IrB);
        k.fd_IkB = make_fastdiv(k.IkB);
    }

    p.lds_bytes = std::max((size_t)k.Kc * k.bpitch * elem_bytes, red);
    k.to_partial = (k.nsplit > 1 || k.tr) ? 1 : 0;
    p.ws_bytes = k.to_partial ? (size_t)k.nsplit * (size_t)out_bytes : 0;
    p.ws_bytes = (p.ws_bytes + 255) / 256 * 256;

    p.k_modes[0] = k.k_mode0;
    p.k_modes[1] = k.k_mode1;
    if (k.tr) {
        p.row_modes[0] = d - 2;
        p.row_modes[1] = d - 1;
    } else if (p.form == 1) {
        p.row_modes[0] = k.r_mode0;
        p.row_modes[1] = k.r_mode1;
    } else {
        p.row_modes[0] = n;
        p.row_modes[1] = -1;
    }
    for (int j = 0; j < 3; ++j) p.outer_modes[j] = k.o_mode[j];
    plan = p;
    return MTTKRP_OK;
}

PlanModel plan_model(const Plan &p, const int64_t *dims, int order, int mode)
{
    // Rates (MI355X, published): matrix cores 78.6 / 157.3 TFLOP/s, HBM
    // 8 TB/s; L2 8 XCDs x 2048 B/clock and LDS 256 CUs x 128 B/clock at
    // 2.4 GHz.
    const double s = p.elem_bytes;
    const double P = p.elem_bytes == 8 ? 78.6e12 : 157.3e12;
    const double BW = 8.0e12, BW_L2 = 8 * 2048 * 2.4e9, BW_LDS = 256 * 128 * 2.4e9;
    const KParams &k = p.kp;
    double N = 1.0, sumI = 0.0;
    for (int m = 0; m < order; ++m) {
        N *= (double)dims[m];
        sumI += (double)dims[m];
    }
    const double R = (double)k.R;
    const double In = (double)dims[mode];
    PlanModel pm{};
    // plan-free bounds
    const double F = 2.0 * R * N;
    pm.t_inf_s = std::max(F / P, s * (N + R * sumI) / BW);
    pm.t_0_s = std::max(F / P, s * (N + (order - 1) * N * R) / BW);
    // the plan's padded work: rows in whole 16 * mb tiles, the contraction in
    // 16-element steps per chunk, the rank in whole rank tiles
    const int64_t rpt = 16 * p.mb;
    const double rows = (p.form == 1 ? (double)k.nunits * (double)k.nrowtiles
                                     : (double)k.nunits) *
                        (double)rpt * (double)k.nbatch;
    const int64_t klast = k.K - (k.nkch - 1) * k.Kc;
    const double Kpad = (double)((k.nkch - 1) * k.Kc + (klast + 15) / 16 * 16);
    const double Rpad = (double)(k.nrtiles * 16 * p.nb);
    pm.flop_s = 2.0 * rows * Kpad * Rpad / P;
    // wave steps (16 contraction elements of one wave tile) over the launch
    const double wave_steps = rows / (double)rpt * (Kpad / 16.0) * (double)k.nrtiles;
    // HBM: X once for every group of rank tiles that run together on one
    // XCD (the workgroup order keeps a chunk's rank tiles adjacent), the other
    // factors and the output once, partials written and read once
    const double resident_xcd = (double)(kNumCU / kNumXCD) * (double)p.per_cu;
    const double rho_x = std::ceil((double)k.nrtiles / resident_xcd);
    const double rows_k = (double)k.In;  // the kernel's output rows (the block for trailing rows)
    const double part = k.to_partial ? 2.0 * (double)k.nsplit * rows_k * R * 8.0 : 0.0;
    pm.hbm_s = (N * s * rho_x + R * (sumI - In) * s + In * R * s + part) / BW;
    // L2: X once per rank tile; the staged Khatri-Rao tile of every
    // workgroup (two factor rows per element for a two-factor tile); the
    // outer factor values every step carries; the row factors of every
    // form-1 item end
    const double b_stage = (double)k.grid_real * (double)k.Kc * 16.0 * p.nb * s *
                           (k.k_mode1 >= 0 ? 2.0 : 1.0);
    const double outer = (double)plan_slots(p.form, k.nouter) * wave_steps * 64.0 * p.nb * s;
    const double itemend = p.form == 1 ? (double)k.nunits * (double)k.nitems * (double)k.nrtiles *
                                             (double)rpt * 16.0 * p.nb * s *
                                             (k.r_mode1 >= 0 ? 2.0 : 1.0)
                                       : 0.0;
    pm.l2_s = (N * s * (double)k.nrtiles + b_stage + outer + itemend) / BW_L2;
    // LDS: every wave step reads 4 x 16 nb operand values of B per lane; the
    // staging writes each B tile once per workgroup
    const double lds = wave_steps * 4.0 * 64.0 * p.nb * s +
                       (double)k.grid_real * (double)k.Kc * 16.0 * p.nb * s;
    pm.lds_s = lds / BW_LDS;
    pm.t_s = std::max(std::max(pm.flop_s, pm.hbm_s), std::max(pm.l2_s, pm.lds_s));
    return pm;
}

size_t als_extra_bytes(const int64_t *dims, int order, int64_t rank)
{
    int64_t maxI = 0;
    for (int m = 0; m < order; ++m) maxI = std::max<int64_t>(maxI, dims[m]);
    const size_t R = (size_t)rank;
    // M (fp64), Grams of every mode, V, L, lambda, scalars
    size_t b = 8 * ((size_t)maxI * R + (size_t)order * R * R + 2 * R * R + R + 64);
    return (b + 255) / 256 * 256;
}

}  // namespace mttkrp
