// Tile-kernel instantiations: f64, layout 0, form 1 (the output index fixed
// per workgroup, tile rows reduced against their factor rows); four waves
// (mb = 2: nb <= 4; mb = 4: nb <= 2) or eight waves when two waves per
// SIMD fit the registers; no outer slots (the item reduction reads the
// outer factors).  Also the multi-mode launches of eight-wave form-1 plans.
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
    if (pl.waves == 8)
        return pl.mb == 2 ? pick_nb<double, 2, false, true, 4, 8, S>(pl.nb, pl.vec)
               : pl.mb == 4 ? pick_nb<double, 4, false, true, 2, 8, S>(pl.nb, pl.vec)
                            : nullptr;
    if (pl.waves != 4) return nullptr;
    return pl.mb == 2 ? pick_nb<double, 2, false, true, 4, 4, S>(pl.nb, pl.vec)
           : pl.mb == 4 ? pick_nb<double, 4, false, true, 2, 4, S>(pl.nb, pl.vec)
                        : nullptr;
}
template <int MB, int NB>
MultiKernel multi_vec(bool vec)
{
    if constexpr (tile_min_waves(sizeof(double), MB, NB, true, 0) != 2)
        return nullptr;
    else
        return vec ? mttkrp_tile_multi_kernel<double, MB, NB, true, 8>
                   : mttkrp_tile_multi_kernel<double, MB, NB, false, 8>;
}
}  // namespace

MultiKernel select_multi_f64(const Plan &pl)
{
    if (pl.layout != 0 || pl.form != 1 || pl.waves != 8 || tile_slots(pl) != 0) return nullptr;
    if (pl.mb == 2)
        return pl.nb == 1 ? multi_vec<2, 1>(pl.vec)
               : pl.nb == 2 ? multi_vec<2, 2>(pl.vec)
               : pl.nb == 4 ? multi_vec<2, 4>(pl.vec)
                            : nullptr;
    if (pl.mb == 4)
        return pl.nb == 1 ? multi_vec<4, 1>(pl.vec) : pl.nb == 2 ? multi_vec<4, 2>(pl.vec) : nullptr;
    return nullptr;
}

TileKernel select_tile_f64_form1(const Plan &pl)
{
    if (pl.layout != 0 || pl.form != 1) return nullptr;
    const int s = tile_slots(pl);
    return s == 0 ? sel<0>(pl) : nullptr;
}

}  // namespace mttkrp
