// fp8-input weight-gradient entry points of the forge C ABI.
#include "fp8_kernels.hpp"
#include "host.hpp"
#include "validate.hpp"

namespace forge {
namespace {

// fp8 inputs: formats are template parameters of the kernels.
template <class C, int EPI, int FA, int FB>
forge_status launch_fp8_dense_t(WgradArgs a, hipStream_t s) {
  set_grid<C>(a, 1);
  hipLaunchKernelGGL((wgrad_fp8_kernel<C, EPI, FA, FB>), dim3(a.num_tiles), dim3(C::THREADS), 0,
                     s, a);
  return launch_status();
}

template <int EPI, int FA, int FB>
forge_status launch_fp8_t(WgradArgs a, forge_tile tile, hipStream_t s) {
  switch (tile) {
    case FORGE_TILE_128x128: return launch_fp8_dense_t<Cfg128x128, EPI, FA, FB>(a, s);
    case FORGE_TILE_256x128: return launch_fp8_dense_t<Cfg256x128, EPI, FA, FB>(a, s);
    case FORGE_TILE_256x256: return launch_fp8_dense_t<Cfg256x256, EPI, FA, FB>(a, s);
    case FORGE_TILE_PERSISTENT: {
      set_grid<Cfg256x256>(a, 1);
      const int grid = persistent_grid();
      if (grid <= 0) return launch_fp8_dense_t<Cfg256x256, EPI, FA, FB>(a, s);
      hipLaunchKernelGGL((wgrad_fp8_persistent_kernel<Cfg256x256, Cfg256x128, EPI, FA, FB>),
                         dim3(grid), dim3(Cfg256x256::THREADS), 0, s, a);
      return launch_status();
    }
    default: return FORGE_ERR_TILE;
  }
}

template <int EPI>
struct Fp8Launch {
  static forge_status run(const WgradArgs& a, forge_dtype xf, forge_dtype yf, forge_tile tile,
                          hipStream_t s) {
    const bool x5 = xf == FORGE_FP8_E5M2, y5 = yf == FORGE_FP8_E5M2;
    if (!x5 && !y5) return launch_fp8_t<EPI, FP8_E4M3, FP8_E4M3>(a, tile, s);
    if (!x5 && y5) return launch_fp8_t<EPI, FP8_E4M3, FP8_E5M2>(a, tile, s);
    if (x5 && !y5) return launch_fp8_t<EPI, FP8_E5M2, FP8_E4M3>(a, tile, s);
    return launch_fp8_t<EPI, FP8_E5M2, FP8_E5M2>(a, tile, s);
  }
};

}  // namespace
}  // namespace forge

using namespace forge;

extern "C" {

FORGE_API forge_status forge_wgrad_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                       const void* dY8, forge_dtype dy_fmt, double dy_scale,
                                       float* grad, int64_t T, int64_t d_in, int64_t d_out,
                                       forge_tile tile, void* stream) {
  if (forge_status s = validate_wgrad_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, grad, T,
                                          d_in, d_out, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X8, dY8, grad, nullptr, nullptr, T, d_in, d_out);
  a.gscale = float(x_scale * dy_scale);
  return Fp8Launch<EPI_GRAD | EPI_SCALE>::run(a, x_fmt, dy_fmt, tile,
                                              static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad_adamw_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                             const void* dY8, forge_dtype dy_fmt,
                                             double dy_scale, float* W, float* m, float* v,
                                             int64_t T, int64_t d_in, int64_t d_out,
                                             const forge_adamw_params* p, forge_tile tile,
                                             void* stream) {
  if (forge_status s = validate_wgrad_adamw_fp8(X8, x_fmt, x_scale, dY8, dy_fmt, dy_scale, W, m,
                                                v, T, d_in, d_out, p, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X8, dY8, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  a.gscale = float(x_scale * dy_scale);
  return with_adamw_epi<Fp8Launch, EPI_ADAMW | EPI_SCALE>(*p, a, x_fmt, dy_fmt, tile,
                                                          static_cast<hipStream_t>(stream));
}

}  // extern "C"
