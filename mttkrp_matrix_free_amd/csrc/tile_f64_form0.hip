// Tile-kernel instantiations: f64, layout 0 (contraction index contiguous),
// form 0 (tile rows are the output rows); four waves, mb = 2 (nb <= 8) or
// mb = 4 (nb <= 2); one to three outer slots.
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
    if (pl.mb == 2) return pick_nb<double, 2, false, false, 8, 4, S>(pl.nb, pl.vec);
    if (pl.mb == 4) return pick_nb<double, 4, false, false, 2, 4, S>(pl.nb, pl.vec);
    return nullptr;
}
}  // namespace

TileKernel select_tile_f64_form0(const Plan &pl)
{
    if (pl.layout != 0 || pl.form != 0 || pl.waves != 4) return nullptr;
    const int s = tile_slots(pl);
    return s == 1 ? sel<1>(pl) : s == 2 ? sel<2>(pl) : s == 3 ? sel<3>(pl) : nullptr;
}

}  // namespace mttkrp
