// Selection of a tile-kernel instantiation for a plan.  The instantiations
// are spread over several translation units (tile_*.hip) that compile in
// parallel; each exposes the selector of its group.
#pragma once

#include "plan.hpp"

namespace mttkrp {

typedef void (*TileKernel)(KParams);

// layout 0, form 0 / form 1, layout 1 -- for fp64 and fp32.  Each returns
// nullptr when the plan asks for a tile its group does not instantiate.
TileKernel select_tile_f64_form0(const Plan &pl);
TileKernel select_tile_f64_form1(const Plan &pl);
TileKernel select_tile_f64_rows(const Plan &pl);
TileKernel select_tile_f32_form0(const Plan &pl);
TileKernel select_tile_f32_form1(const Plan &pl);
TileKernel select_tile_f32_rows(const Plan &pl);

// Multi-mode launches (several form-1 modes sharing a B tile, one pass each).
typedef void (*MultiKernel)(KPack);
MultiKernel select_multi_f64(const Plan &pl);
MultiKernel select_multi_f32(const Plan &pl);

inline int tile_slots(const Plan &pl) { return plan_slots(pl.form, pl.kp.nouter); }

}  // namespace mttkrp
