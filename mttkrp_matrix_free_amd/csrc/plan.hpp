// Host planner and kernel parameter block for the matrix-free MTTKRP.
//
// Decomposition (one mode n of a d-way row-major tensor):
//   * A contraction group K of one or two consecutive modes is summed on the
//     matrix cores against the factor rows of those modes: T(row, r) =
//     sum_k X(.., row, .., k) * B(k, r), with B(k, r) = U_ka(k / I_kb, r) *
//     U_kb(k % I_kb, r) (a Khatri-Rao tile of at most two factors, built in LDS
//     on the fly).  This is the mode-k product of "An HPC Approach to
//     Accelerate Tensor Decompositions", Eq. (1), with the factor as the
//     matrix.
//   * Tile rows index one or two consecutive modes (layout 0: the contraction
//     index has unit stride, rows are fibres) or the output mode itself when
//     it is the last mode (layout 1: rows have unit stride).
//   * Every remaining mode is an "outer" mode, iterated per tile, whose factor
//     row is a Hadamard multiplier (the tile Hadamard product of the GenTen
//     page, Fig. 2).
//   * form 0: tile rows are the output rows; the outer multiplier scales B and
//     the matrix-core accumulators sum over every outer tuple directly.
//     form 1: the output index is an outer index fixed per workgroup; after
//     each tile the accumulators are reduced over the tile rows against the
//     row factors and the outer multiplier.
// Partial results of independent chunks go to a workspace and are summed in a
// fixed order by a second kernel (deterministic), as the GenTen page's Fig. 2
// allows several workgroups per slice.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace mttkrp {

constexpr int kMaxOrder = 5;

constexpr int kNumCU = 256;            // MI355X compute units
constexpr int kNumXCD = 8;             // accelerator complex dies (L2 domains)
constexpr size_t kLdsBudget = 80 * 1024;       // dynamic LDS of a 4-wave workgroup (2 per CU)
constexpr size_t kLdsBudgetThree = 52 * 1024;  // the same at three workgroups per CU
constexpr size_t kLdsBudgetWide = 144 * 1024;  // dynamic LDS of an 8-wave workgroup (1 per CU)

// Outer-factor slots a tile kernel carries per step: none for form 1 (its
// outer multiplier is read once per item, at the item's reduction), else one
// per outer mode (at least one).
__host__ __device__ constexpr int plan_slots(int form, int nouter)
{
    return form == 1 ? 0 : (nouter <= 1 ? 1 : nouter);
}

// Register estimate of a tile kernel (per lane, 32-bit registers): the
// accumulators, the fp64 flush of form-0 fp32 tiles, `buffers` step buffers
// (tensor elements and `slots` outer factor values per column), per-column
// state and a fixed part.  Shared by the kernels (launch bounds, prefetch
// depth) and the planner (workgroup size).
__host__ __device__ constexpr int tile_regs(int elem, int mb, int nb, bool form1, int slots,
                                            int buffers)
{
    return mb * nb * 4 * elem / 4 +                          // accumulators
           ((!form1 && elem == 4) ? mb * nb * 4 * 2 : 0) +   // fp64 flush
           buffers * (4 * mb + slots * nb) * elem / 4 +      // step buffers
           (form1 ? 16 : 10) * nb +                           // B operand, column, row sum
           (form1 ? 96 : 64);                                 // addresses, cursors, row factors
}
// Waves per SIMD the registers allow: two within 256 registers, else one.
__host__ __device__ constexpr int tile_min_waves(int elem, int mb, int nb, bool form1, int slots)
{
    return tile_regs(elem, mb, nb, form1, slots, 2) <= 256 ? 2 : 1;
}
// Waves per SIMD of a kernel instantiation (its launch bound).  Besides the
// register model's one or two: three for the form-0 tiles of the rank-tiled,
// matrix-core-bound plans -- 32 x 64 tiles of row-major outputs and 64 x 32
// tiles of row-contiguous outputs, four-wave workgroups, one outer slot in
// fp64, one or two in fp32 -- whose kernels fit 168 registers without spills
// once they keep one step of tensor loads in flight (512^3 rank 2000: the
// matrix cores busy 85% of a launch at two waves per SIMD; 8.30 -> 8.05 ms
// per mode; 128 x 128 x 128 x 64 fp32 rank 512: 1.29 -> 1.22 ms, rank 64:
// 0.18 -> 0.17 ms).
__host__ __device__ constexpr bool tile_three_waves(int elem, int mb, int nb, bool form1, int slots,
                                                    bool rc, int w)
{
    return !form1 && w == 4 && (elem == 8 ? slots == 1 : (slots == 1 || slots == 2)) &&
           ((mb == 2 && nb == 4 && !rc) || (mb == 4 && nb == 2 && rc));
}
__host__ __device__ constexpr int tile_occupancy(int elem, int mb, int nb, bool form1, int slots,
                                                bool rc, int w)
{
    return tile_three_waves(elem, mb, nb, form1, slots, rc, w)
               ? 3
               : tile_min_waves(elem, mb, nb, form1, slots);
}
// Steps of tensor loads kept in flight: two when a third buffer fits the
// budget of the instantiation's occupancy, else one.
__host__ __device__ constexpr int tile_prefetch(int elem, int mb, int nb, bool form1, int slots,
                                                bool rc, int w)
{
    return tile_regs(elem, mb, nb, form1, slots, 3) <=
                   512 / tile_occupancy(elem, mb, nb, form1, slots, rc, w)
               ? 2
               : 1;
}

// Division by a divisor d in [1, 2^31) fixed for a launch, for dividends
// below 2^31: q = (mulhi(x, m) + x) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 -- the round-up method of Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication" (1994),
// Sec. 4, with the add kept in 32 bits because x < 2^31.  The constants are
// computed once on the host; a division costs a multiply-high, an add and a
// shift instead of a software 64-bit division.
struct FastDiv {
    uint32_t d, m, s;
};
inline FastDiv make_fastdiv(int64_t d)
{
    FastDiv f;
    f.d = (uint32_t)d;
    f.s = 0;
    while ((UINT64_C(1) << f.s) < (uint64_t)d) ++f.s;
    f.m = (uint32_t)(((UINT64_C(1) << 32) * ((UINT64_C(1) << f.s) - (uint64_t)d)) / (uint64_t)d + 1);
    return f;
}
__host__ __device__ inline uint32_t fdiv(uint32_t x, const FastDiv &f)
{
    const uint32_t t = (uint32_t)(((uint64_t)x * f.m) >> 32);
    return (t + x) >> f.s;
}

struct KParams {
    const void *X;
    int64_t x_bytes;           // bytes of X (bounds of its buffer descriptor)
    // factor rows by role (device): contraction group, tile rows, outer modes
    const void *Uk0, *Uk1;     // Uk1 = null when the contraction group is one mode
    const void *Ur0, *Ur1;     // form 1 only; Ur1 = null for one row mode
    const void *Uo[3];         // null past nouter
    void *out;                 // I_n x R, element type of the problem
    double *partial;           // [nsplit][I_n][R] fp64 partial sums (nsplit > 1)
    int64_t R;
    int64_t In;                // output rows
    // contraction group
    int64_t K;                 // contraction length
    int64_t Kc;                // contraction chunk of one workgroup (multiple of 16)
    int64_t nkch;              // contraction chunks (each writes its own partial)
    int64_t k_stride;          // element stride of k in X
    int k_mode0, k_mode1;      // k = i_{k_mode0} * IkB + i_{k_mode1}; k_mode1 = -1: single mode
    int64_t IkB;
    // tile rows
    int64_t nrows;             // rows per batch
    int64_t row_stride;        // element stride of the row index (of i_{r_mode1} for two row modes)
    int64_t row_stride_a;      // element stride of i_{r_mode0}
    int row_split;             // 1: the two row modes are not adjacent (offsets per item and lane)
    int r_mode0, r_mode1;      // form 1 only; row = i_{r_mode0} * IrB + i_{r_mode1}
    int64_t IrB;
    // outer modes (decoded last-fastest from the batch index)
    int nouter;
    int o_mode[3];
    int64_t o_dim[3];
    int64_t o_stride[3];
    int64_t nbatch;
    int64_t n_stride;          // form 1: stride of the output mode
    // decomposition
    int64_t nunits;            // form 1: I_n; form 0: row tiles of the output
    int64_t nrowtiles;         // form 1: row tiles per batch
    int64_t nitems;            // work items per unit (form 1: batches x row tiles; form 0: batches)
    int64_t chunk;             // form 1: items per workgroup; form 0: steps (full chunk)
    int64_t nsplit;            // partial outputs per unit: nsplit_it * nkch
    int64_t nsplit_it;         // chunks of the work items per unit
    int64_t nrtiles;           // rank tiles
    int64_t grid_real;         // nunits * nsplit * nrtiles
    int64_t grid_per_xcd;      // ceil(grid_real / kNumXCD)
    int bpitch;                // LDS row pitch of B (elements)
    int out64;                 // 1: `out` is fp64 whatever the element type
    int to_partial;            // 1: the tile kernel writes fp64 partials (split or trailing rows)
    int red_all;               // form 0: every wave's tile goes to LDS at once (else a pairwise tree)
    // Trailing rows (layout 1 with the last two modes as tile rows): the kernel
    // rows are the block (i_{d-2}, i_{d-1}); the reduction pass contracts the
    // row mode that is not the output against its factor U_red.
    int tr;                    // 1: trailing-rows plan
    int tr_div;                // 1: output index = row / tr_inner; 0: = row % tr_inner
    int64_t tr_inner;          // I_{d-1}
    int64_t tr_J;              // extent of the reduced row mode
    int64_t In_out;            // output rows I_n (In is the kernel's row count)
    const void *Ured;          // factor of the reduced row mode
    // A split reduction of another mode carried out by this launch (all-mode
    // sweep): pend_out[i] = sum_s pend_partial[s][i] for i < pend_count, in
    // the fixed order of split_reduce_kernel with pend_ng thread groups.
    // pend_partial = null: none.
    const double *pend_partial;
    int64_t pend_nsplit, pend_count;
    void *pend_out;
    int pend_ng;
    // divisors of the index decode (every dividend is below 2^31)
    FastDiv fd_nrtiles, fd_nsplit, fd_nsplit_it, fd_nunits;
    int split_major;           // 1: workgroup order is (split, unit, rank tile), else (unit, split, rank tile)
    FastDiv fd_nkc_full, fd_nkc_last;  // steps per item: full chunk, last chunk
    FastDiv fd_nrowtiles, fd_odim1, fd_odim2, fd_IrB, fd_IkB;
};

struct Plan {
    int elem_bytes = 8;
    int form = 1;
    int layout = 0;   // 0: contraction index contiguous; 1: rows contiguous
    int mb = 4, nb = 2;
    int waves = 4;    // waves per workgroup (4 or 8)
    int per_cu = 1;   // workgroups resident per compute unit (registers and LDS)
    bool b_in_lds = true;
    bool vec = true;
    int k_modes[2] = {-1, -1};
    int row_modes[2] = {-1, -1};
    int outer_modes[3] = {-1, -1, -1};
    int red_mode = -1;  // trailing rows: the row mode reduced after the tile pass
    KParams kp{};
    int64_t grid = 0;        // launched grid (multiple of kNumXCD)
    size_t lds_bytes = 0;
    size_t ws_bytes = 0;
};

// Parameter blocks of the two modes one multi-mode launch runs in turn
// (form 1, same B tile and decomposition); red_off: LDS byte offset of the
// reduction space (after the B tile).
constexpr int kMaxPasses = 2;
struct KPack {
    KParams p[kMaxPasses];
    int64_t red_off;
};

// Fills `plan` for mode `mode`.  Returns 0 or a MTTKRP_* status.  Pure host
// code: no HIP call.  Pointers in plan.kp are left null.
// For experiments, the environment variable MTTKRP_FORCE_TILE="mb,nb" or
// "mb,nb,waves" replaces the planner's wave tile (and workgroup size); the
// contraction chunks, splits and grid then follow from it as usual.  A value
// that is malformed or outside mb in {2,4}, nb in {1,2,4,8}, waves in {4,8}
// makes every plan fail with MTTKRP_EINVAL.  (A forced tile that no kernel
// instantiates is reported by plan_launchable.)
int make_plan(const int64_t *dims, int order, int64_t rank, int mode, int elem_bytes, Plan &plan);

// The plain cache model of one plan (seconds on MI355X): the time each
// resource needs for the plan's traffic at its peak rate, T(p) the largest.
// Matrix cores: the padded tile flops at 78.6 (fp64) / 157.3 (fp32)
// TFLOP/s.  HBM: X once per group of rank tiles that share an L2, the other
// factors and the output once, split partials written and read, at 8 TB/s.
// L2: X once per rank tile, the staged Khatri-Rao tiles, the per-step outer
// factor values and the item-end row factors, at 8 XCDs x 2 KB/clock.  LDS:
// the matrix-core operand reads of B and the staging stores, at 256 CUs x
// 128 B/clock.  T_inf and T_0 are the plan-free bounds (every byte moved
// once; the factor rows re-read for every tensor element).
struct PlanModel {
    double flop_s, hbm_s, l2_s, lds_s, t_s;  // t_s = max of the four
    double t_inf_s, t_0_s;
};
PlanModel plan_model(const Plan &p, const int64_t *dims, int order, int mode);

// Whether a kernel instantiation exists for the plan's tile (always true for
// the planner's own choices; a forced tile may have none).
bool plan_launchable(const Plan &p);

// Workspace of the CP-ALS driver beyond the MTTKRP workspace (bytes).
size_t als_extra_bytes(const int64_t *dims, int order, int64_t rank);

}  // namespace mttkrp
