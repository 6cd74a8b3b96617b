// Host-side helpers shared by the HIP translation units of the forge C ABI:
// device check, per-step scalars, tile choice and launch bookkeeping.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "forge.h"
#include "wgrad_kernels.hpp"

namespace forge {

// FORGE_ERR_DEVICE unless the current device is a gfx950 (cached per device).
forge_status check_device();
// Workgroups of a persistent launch on the current device: one per compute
// unit, rounded down to whole pairs per XCD (8 XCDs), or 0 if too few.
int persistent_grid();
AdamWConsts make_adamw(const forge_adamw_params& p);
SgdmConsts make_sgdm(const forge_sgdm_params& p);

struct TileShape {
  int bm, bn;
};
TileShape shape_of(forge_tile t);
int64_t count_tiles(int64_t d_in, int64_t d_out, TileShape s);
double persistent_makespan(int64_t tiles, int grid);
forge_tile resolve_tile(forge_tile t, int64_t d_in, int64_t d_out, int64_t experts,
                        bool allow_persistent = true);
forge_status launch_status();
WgradArgs base_args(const void* X, const void* dY, float* W, float* S1, float* S2, int64_t T,
                    int64_t d_in, int64_t d_out);
// Tile counts must fit the kernels' 32-bit block indices.
bool grid_fits(int64_t d_in, int64_t d_out, forge_tile tile, int64_t experts);

// Tile configurations behind the public tile ids.
using Cfg256x256 = TileCfg<256, 256, 2, 2, 32, 1>;
using Cfg256x128 = TileCfg<256, 128, 2, 2, 32, 1>;
using Cfg128x128 = TileCfg<128, 128, 2, 2, 32, 2>;

template <class C>
void set_grid(WgradArgs& a, int64_t experts) {
  a.tiles_m = int32_t((a.d_in + C::BM - 1) / C::BM);
  a.tiles_n = int32_t((a.d_out + C::BN - 1) / C::BN);
  a.num_tiles = int32_t(a.tiles_m * a.tiles_n * experts);
  a.group_m = 4;
}

// AdamW epilogue variant: the exact square root when eps = 0.
template <template <int> class F, int BASE = EPI_ADAMW, class... Args>
forge_status with_adamw_epi(const forge_adamw_params& p, Args&&... args) {
  return p.eps > 0.0 ? F<BASE>::run(args...) : F<BASE | EPI_EXACT_SQRT>::run(args...);
}

// The fused weight-gradient launches of forge.hip, for the linear-backward
// calls (one instantiation of each kernel in the library).
forge_status launch_wgrad_adamw(const WgradArgs& a, const forge_adamw_params& p, forge_tile tile,
                                hipStream_t s);
forge_status launch_wgrad_sgdm(const WgradArgs& a, forge_tile tile, hipStream_t s);

}  // namespace forge
