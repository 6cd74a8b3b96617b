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
// The tile a call runs: `t`, or the library's choice for t = DEFAULT. Where
// the persistent schedule is not allowed (grouped calls, the input gradient),
// FORGE_TILE_PERSISTENT falls back to 256x256 tiles.
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

// Dense weight-gradient launches: a grid of tiles of configuration C, or the
// persistent schedule (full 256x256 and half 256x128 tiles).
template <class C, int EPI>
forge_status launch_dense_t(WgradArgs a, hipStream_t s) {
  set_grid<C>(a, 1);
  hipLaunchKernelGGL((wgrad_dense_kernel<C, EPI>), dim3(a.num_tiles), dim3(C::THREADS), 0, s, a);
  return launch_status();
}

template <int EPI>
forge_status launch_persistent(WgradArgs a, hipStream_t s) {
  set_grid<Cfg256x256>(a, 1);
  const int grid = persistent_grid();
  if (grid <= 0) return launch_dense_t<Cfg256x256, EPI>(a, s);
  hipLaunchKernelGGL((wgrad_persistent_kernel<Cfg256x256, Cfg256x128, EPI>), dim3(grid),
                     dim3(Cfg256x256::THREADS), 0, s, a);
  return launch_status();
}

template <int EPI>
forge_status launch_dense(const WgradArgs& a, forge_tile tile, hipStream_t s) {
  switch (tile) {
    case FORGE_TILE_128x128: return launch_dense_t<Cfg128x128, EPI>(a, s);
    case FORGE_TILE_256x128: return launch_dense_t<Cfg256x128, EPI>(a, s);
    case FORGE_TILE_256x256: return launch_dense_t<Cfg256x256, EPI>(a, s);
    case FORGE_TILE_PERSISTENT: return launch_persistent<EPI>(a, s);
    default: return FORGE_ERR_TILE;
  }
}

template <int EPI>
struct DenseLaunch {
  static forge_status run(const WgradArgs& a, forge_tile tile, hipStream_t s) {
    return launch_dense<EPI>(a, tile, s);
  }
};

// The fused weight-gradient launches of forge.hip, for the linear-backward
// calls (one instantiation of each kernel in the library).
forge_status launch_wgrad_adamw(const WgradArgs& a, const forge_adamw_params& p, forge_tile tile,
                                hipStream_t s);
forge_status launch_wgrad_sgdm(const WgradArgs& a, forge_tile tile, hipStream_t s);

}  // namespace forge
