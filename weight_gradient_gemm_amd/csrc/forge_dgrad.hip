// Input-gradient entry points of the forge C ABI: dX = dY W_b on its own,
// and the linear-layer backward that issues it before the fused optimizer
// step on the same stream; each from the float32 weight or from a bf16 copy
// of it (which the fused step then refreshes). Also the fused steps that
// refresh such a copy without an input gradient.
#include "dgrad_kernels.hpp"
#include "host.hpp"
#include "validate.hpp"

namespace forge {
namespace {

template <class C, int EPI, bool WB>
forge_status launch_dgrad_t(WgradArgs a, const void* W, int K, hipStream_t s) {
  set_grid<C>(a, 1);
  hipLaunchKernelGGL((dgrad_kernel<C, EPI, WB>), dim3(a.num_tiles), dim3(C::THREADS), 0, s, a, W,
                     K);
  return launch_status();
}

template <int EPI, bool WB>
forge_status launch_dgrad(const WgradArgs& a, const void* W, int K, forge_tile tile,
                          hipStream_t s) {
  switch (tile) {
    case FORGE_TILE_128x128: return launch_dgrad_t<Cfg128x128, EPI, WB>(a, W, K, s);
    case FORGE_TILE_256x128: return launch_dgrad_t<Cfg256x128, EPI, WB>(a, W, K, s);
    case FORGE_TILE_256x256: return launch_dgrad_t<Cfg256x256, EPI, WB>(a, W, K, s);
    default: return FORGE_ERR_TILE;
  }
}

// The dX contraction over [d_in, T] (M = d_in, N = tokens): its tile, or a
// shape error if the grid would not fit. Grid launches only.
forge_status plan_dgrad(forge_tile tile, int64_t T, int64_t d_in, forge_tile* out) {
  *out = resolve_tile(tile, d_in, T, 1, false);
  return grid_fits(d_in, T, *out, 1) ? FORGE_OK : FORGE_ERR_SHAPE;
}

// Launch the planned dX contraction (T > 0, d_in > 0) from float32 W, or with
// wb from its bf16 copy. The epilogue sees dX as a [T, d_in] matrix: rows are
// tokens.
template <bool WB>
forge_status run_dgrad(const void* dY, const void* W, void* dX, forge_dtype dt, int64_t T,
                       int64_t d_in, int64_t d_out, forge_tile tile, hipStream_t s) {
  WgradArgs a = base_args(nullptr, dY, static_cast<float*>(dX), nullptr, nullptr, T, d_in, T);
  return dt == FORGE_BF16 ? launch_dgrad<EPI_GRAD | EPI_BF16_OUT, WB>(a, W, int(d_out), tile, s)
                          : launch_dgrad<EPI_GRAD, WB>(a, W, int(d_out), tile, s);
}

// The fused steps that also store the bf16 copy of the updated W (a.Wb).
forge_status launch_wgrad_adamw_wb(const WgradArgs& a, const forge_adamw_params& p,
                                   forge_tile tile, hipStream_t s) {
  return with_adamw_epi<DenseLaunch, EPI_ADAMW | EPI_WB_OUT>(p, a, tile, s);
}

forge_status launch_wgrad_sgdm_wb(const WgradArgs& a, forge_tile tile, hipStream_t s) {
  return launch_dense<EPI_SGDM | EPI_WB_OUT>(a, tile, s);
}

// The shared body of the linear-backward calls: dX from W (or its bf16 copy
// Wb when WB), then the fused step `step(a, tile, stream)` on the arguments
// `a` (which carry Wb for the copy's refresh).
template <bool WB, class Step>
forge_status linear_backward(const void* dY, const void* Wdx, void* dX, forge_dtype dX_dtype,
                             int64_t T, int64_t d_in, int64_t d_out, WgradArgs a,
                             forge_tile tile, void* stream, Step step) {
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
  // dX first: it reads W (or Wb) before the fused step overwrites it.
  if (do_dx)
    if (forge_status s = run_dgrad<WB>(dY, Wdx, dX, dX_dtype, T, d_in, d_out, dt, st)) return s;
  if (!do_w) return FORGE_OK;
  return step(a, tile, st);
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
  return run_dgrad<false>(dY, W, dX, dX_dtype, T, d_in, d_out, dt,
                          static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_dgrad_bf16w(const void* dY, const void* Wb, void* dX,
                                         forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                         int64_t d_out, forge_tile tile, void* stream) {
  if (forge_status s = validate_dgrad_bf16w(dY, Wb, dX, dX_dtype, T, d_in, d_out, tile)) return s;
  if (T == 0 || d_in == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  forge_tile dt;
  if (forge_status s = plan_dgrad(tile, T, d_in, &dt)) return s;
  (void)hipGetLastError();
  return run_dgrad<true>(dY, Wb, dX, dX_dtype, T, d_in, d_out, dt,
                         static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_linear_backward_adamw(const void* X, const void* dY, float* W,
                                                   float* m, float* v, void* dX,
                                                   forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                                   int64_t d_out, const forge_adamw_params* p,
                                                   forge_tile tile, void* stream) {
  if (forge_status s = validate_linear_backward_adamw(X, dY, W, m, v, dX, dX_dtype, T, d_in,
                                                      d_out, p, tile))
    return s;
  WgradArgs a = base_args(X, dY, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  return linear_backward<false>(dY, W, dX, dX_dtype, T, d_in, d_out, a, tile, stream,
                                [p](const WgradArgs& w, forge_tile t, hipStream_t s) {
                                  return launch_wgrad_adamw(w, *p, t, s);
                                });
}

FORGE_API forge_status forge_linear_backward_sgdm(const void* X, const void* dY, float* W,
                                                  float* mom, void* dX, forge_dtype dX_dtype,
                                                  int64_t T, int64_t d_in, int64_t d_out,
                                                  const forge_sgdm_params* p, forge_tile tile,
                                                  void* stream) {
  if (forge_status s = validate_linear_backward_sgdm(X, dY, W, mom, dX, dX_dtype, T, d_in, d_out,
                                                     p, tile))
    return s;
  WgradArgs a = base_args(X, dY, W, mom, nullptr, T, d_in, d_out);
  a.sgd = make_sgdm(*p);
  return linear_backward<false>(dY, W, dX, dX_dtype, T, d_in, d_out, a, tile, stream,
                                launch_wgrad_sgdm);
}

FORGE_API forge_status forge_linear_backward_adamw_bf16w(const void* X, const void* dY, float* W,
                                                         float* m, float* v, void* Wb, void* dX,
                                                         forge_dtype dX_dtype, int64_t T,
                                                         int64_t d_in, int64_t d_out,
                                                         const forge_adamw_params* p,
                                                         forge_tile tile, void* stream) {
  if (forge_status s = validate_linear_backward_adamw_bf16w(X, dY, W, m, v, Wb, dX, dX_dtype, T,
                                                            d_in, d_out, p, tile))
    return s;
  WgradArgs a = base_args(X, dY, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  a.Wb = static_cast<uint16_t*>(Wb);
  return linear_backward<true>(dY, Wb, dX, dX_dtype, T, d_in, d_out, a, tile, stream,
                               [p](const WgradArgs& w, forge_tile t, hipStream_t s) {
                                 return launch_wgrad_adamw_wb(w, *p, t, s);
                               });
}

FORGE_API forge_status forge_linear_backward_sgdm_bf16w(const void* X, const void* dY, float* W,
                                                        float* mom, void* Wb, void* dX,
                                                        forge_dtype dX_dtype, int64_t T,
                                                        int64_t d_in, int64_t d_out,
                                                        const forge_sgdm_params* p,
                                                        forge_tile tile, void* stream) {
  if (forge_status s = validate_linear_backward_sgdm_bf16w(X, dY, W, mom, Wb, dX, dX_dtype, T,
                                                           d_in, d_out, p, tile))
    return s;
  WgradArgs a = base_args(X, dY, W, mom, nullptr, T, d_in, d_out);
  a.sgd = make_sgdm(*p);
  a.Wb = static_cast<uint16_t*>(Wb);
  return linear_backward<true>(dY, Wb, dX, dX_dtype, T, d_in, d_out, a, tile, stream,
                               launch_wgrad_sgdm_wb);
}

FORGE_API forge_status forge_wgrad_adamw_bf16w(const void* X, const void* dY, float* W, float* m,
                                               float* v, void* Wb, int64_t T, int64_t d_in,
                                               int64_t d_out, const forge_adamw_params* p,
                                               forge_tile tile, void* stream) {
  if (forge_status s = validate_wgrad_adamw_bf16w(X, dY, W, m, v, Wb, T, d_in, d_out, p, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  a.Wb = static_cast<uint16_t*>(Wb);
  return launch_wgrad_adamw_wb(a, *p, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad_sgdm_bf16w(const void* X, const void* dY, float* W, float* mom,
                                              void* Wb, int64_t T, int64_t d_in, int64_t d_out,
                                              const forge_sgdm_params* p, forge_tile tile,
                                              void* stream) {
  if (forge_status s = validate_wgrad_sgdm_bf16w(X, dY, W, mom, Wb, T, d_in, d_out, p, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, W, mom, nullptr, T, d_in, d_out);
  a.sgd = make_sgdm(*p);
  a.Wb = static_cast<uint16_t*>(Wb);
  return launch_wgrad_sgdm_wb(a, tile, static_cast<hipStream_t>(stream));
}

}  // extern "C"
