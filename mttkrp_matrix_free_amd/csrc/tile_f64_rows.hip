// Tile-kernel instantiations: f64, layout 1 (rows contiguous, output = the
// unit-stride mode), form 0; four waves or eight (when two waves per SIMD
// fit the registers), 64-row groups (mb = 4) with nb <= 4, or 32-row
// groups (mb = 2) with nb = 4;
// one to three outer slots.
#include "mttkrp_tile.hpp"

namespace mttkrp {
namespace {

// Eight-wave workgroups exist only for tiles whose registers allow two waves
// per SIMD (the planner asks for them only then).
template <typename T, int MB, int NB, bool RC, bool FORM1, int W, int S>
TileKernel pick_vec(bool vec)
{
    if constexpr (W == 8 && tile_min_waves(sizeof(T), MB, NB, FORM1, S) != 2)
        return nullptr;
    else
        return vec ? mttkrp_tile_kernel<T, MB, NB, RC, true, FORM1, W, S>
                   : mttkrp_tile_kernel<T, MB, NB, RC, false, FORM1, W, S>;
}

// Rank-tile widths instantiated up to MAXNB (the planner never asks for more).
template <typename T, int MB, bool RC, bool FORM1, int MAXNB, int W, int S>
TileKernel pick_nb(int nb, bool vec)
{
    switch (nb) {
    case 1: return pick_vec<T, MB, 1, RC, FORM1, W, S>(vec);
    case 2: return MAXNB >= 2 ? pick_vec<T, MB, (MAXNB >= 2 ? 2 : 1), RC, FORM1, W, S>(vec) : nullptr;
    case 4: return MAXNB >= 4 ? pick_vec<T, MB, (MAXNB >= 4 ? 4 : 1), RC, FORM1, W, S>(vec) : nullptr;
    case 8: return MAXNB >= 8 ? pick_vec<T, MB, (MAXNB >= 8 ? 8 : 1), RC, FORM1, W, S>(vec) : nullptr;
    default: return nullptr;
    }
}

template <int S>
TileKernel sel(const Plan &pl)
{
    // 32-row tiles (mb = 2) with four rank blocks: short trailing row blocks,
    // where 64-row tiles would be mostly padding or need two rank tiles.
    if (pl.mb == 2) {
        if (pl.nb != 4) return nullptr;
        return pl.waves == 8   ? pick_vec<double, 2, 4, true, false, 8, S>(pl.vec)
               : pl.waves == 4 ? pick_vec<double, 2, 4, true, false, 4, S>(pl.vec)
                               : nullptr;
    }
    if (pl.mb != 4) return nullptr;
    if (pl.waves == 8) return pick_nb<double, 4, true, false, 4, 8, S>(pl.nb, pl.vec);
    return pl.waves == 4 ? pick_nb<double, 4, true, false, 4, 4, S>(pl.nb, pl.vec) : nullptr;
}
}  // namespace

TileKernel select_tile_f64_rows(const Plan &pl)
{
    if (pl.layout != 1 || pl.form != 0) return nullptr;
    const int s = tile_slots(pl);
    return s == 1 ? sel<1>(pl) : s == 2 ? sel<2>(pl) : s == 3 ? sel<3>(pl) : nullptr;
}

}  // namespace mttkrp
