// Input-gradient entry points of the forge C ABI: dX = dY W_b on its own,
// and the linear-layer backward that issues it before the fused optimizer
// step on the same stream.
#include "dgrad_kernels.hpp"
#include "host.hpp"
#include "validate.hpp"

namespace forge {
namespace {

template <class C, int EPI>
forge_status launch_dgrad_t(WgradArgs a, const float* W, int K, hipStream_t s) {
  set_grid<C>(a, 1);
  hipLaunchKernelGGL((dgrad_kernel<C, EPI>), dim3(a.num_tiles), dim3(C::THREADS), 0, s, a, W, K);
  return launch_status();
}

template <int EPI>
forge_status launch_dgrad(const WgradArgs& a, const float* W, int K, forge_tile tile,
                          hipStream_t s) {
  switch (tile) {
    case FORGE_TILE_128x128: return launch_dgrad_t<Cfg128x128, EPI>(a, W, K, s);
    case FORGE_TILE_256x128: return launch_dgrad_t<Cfg256x128, EPI>(a, W, K, s);
    case FORGE_TILE_256x256: return launch_dgrad_t<Cfg256x256, EPI>(a, W, K, s);
    default: return FORGE_ERR_TILE;
  }
}

// The dX contraction over [d_in, T] (M = d_in, N = tokens): its tile, or a
// shape error if the grid would not fit. Grid launches only.
forge_status plan_dgrad(forge_tile tile, int64_t T, int64_t d_in, forge_tile* out) {
  *out = resolve_tile(tile, d_in, T, 1, false);
  return grid_fits(d_in, T, *out, 1) ? FORGE_OK : FORGE_ERR_SHAPE;
}

// Launch the planned dX contraction (T > 0, d_in > 0). The epilogue sees dX
// as a [T, d_in] matrix: rows are tokens.
forge_status run_dgrad(const void* dY, const float* W, void* dX, forge_dtype dt, int64_t T,
                       int64_t d_in, int64_t d_out, forge_tile tile, hipStream_t s) {
  WgradArgs a = base_args(nullptr, dY, static_cast<float*>(dX), nullptr, nullptr, T, d_in, T);
  return dt == FORGE_BF16 ? launch_dgrad<EPI_GRAD | EPI_BF16_OUT>(a, W, int(d_out), tile, s)
                          : launch_dgrad<EPI_GRAD>(a, W, int(d_out), tile, s);
}

}  // namespace
}  // namespace forge

using namespace forge;

extern "C" {

FORGE_API forge_status forge_dgrad(const void* dY, const float* W, void* dX, forge_dtype dX_dtype,
                                   int64_t T, int64_t d_in, int64_t d_out, forge_tile tile,
                                   void* stream) {
  if (forge_status s = validate_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, tile)) return s;
  if (T == 0 || d_in == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  forge_tile dt;
  if (forge_status s = plan_dgrad(tile, T, d_in, &dt)) return s;
  (void)hipGetLastError();
  return run_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, dt, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_linear_backward_adamw(const void* X, const void* dY, float* W,
                                                   float* m, float* v, void* dX,
                                                   forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                                   int64_t d_out, const forge_adamw_params* p,
                                                   forge_tile tile, void* stream) {
  if (forge_status s = validate_linear_backward_adamw(X, dY, W, m, v, dX, dX_dtype, T, d_in,
                                                      d_out, p, tile))
    return s;
  const bool do_dx = T > 0 && d_in > 0, do_w = d_in > 0 && d_out > 0;
  if (!do_dx && !do_w) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  forge_tile dt = FORGE_TILE_DEFAULT;
  if (do_dx)
    if (forge_status s = plan_dgrad(FORGE_TILE_DEFAULT, T, d_in, &dt)) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (do_w && !grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // dX first: it reads W before the fused step overwrites it.
  if (do_dx)
    if (forge_status s = run_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, dt, st)) return s;
  if (!do_w) return FORGE_OK;
  WgradArgs a = base_args(X, dY, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  return launch_wgrad_adamw(a, *p, tile, st);
}

FORGE_API forge_status forge_linear_backward_sgdm(const void* X, const void* dY, float* W,
                                                  float* mom, void* dX, forge_dtype dX_dtype,
                                                  int64_t T, int64_t d_in, int64_t d_out,
                                                  const forge_sgdm_params* p, forge_tile tile,
                                                  void* stream) {
  if (forge_status s = validate_linear_backward_sgdm(X, dY, W, mom, dX, dX_dtype, T, d_in, d_out,
                                                     p, tile))
    return s;
  const bool do_dx = T > 0 && d_in > 0, do_w = d_in > 0 && d_out > 0;
  if (!do_dx && !do_w) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  forge_tile dt = FORGE_TILE_DEFAULT;
  if (do_dx)
    if (forge_status s = plan_dgrad(FORGE_TILE_DEFAULT, T, d_in, &dt)) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (do_w && !grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (do_dx)
    if (forge_status s = run_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, dt, st)) return s;
  if (!do_w) return FORGE_OK;
  WgradArgs a = base_args(X, dY, W, mom, nullptr, T, d_in, d_out);
  a.sgd = make_sgdm(*p);
  return launch_wgrad_sgdm(a, tile, st);
}

}  // extern "C"
