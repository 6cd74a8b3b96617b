// The bf16 weight-gradient entry points of the forge C ABI (fused AdamW and
// SGD-momentum, the unfused pair, routed experts, precision variants):
// validation, tile choice and kernel launch on the caller's stream. Nothing
// here allocates device memory.
#include <algorithm>
#include <cstring>

#include "elementwise_kernels.hpp"
#include "host.hpp"
#include "validate.hpp"

namespace forge {
namespace {

template <class C, int EPI>
forge_status launch_grouped_t(WgradArgs a, const GroupTable& gt, int32_t E, hipStream_t s) {
  set_grid<C>(a, E);
  hipLaunchKernelGGL((wgrad_grouped_kernel<C, EPI>), dim3(a.num_tiles), dim3(C::THREADS), 0, s,
                     a, gt);
  return launch_status();
}

template <int EPI>
struct GroupedLaunch {
  static forge_status run(const WgradArgs& a, const GroupTable& gt, int32_t E, forge_tile tile,
                          hipStream_t s) {
    switch (tile) {
      case FORGE_TILE_128x128: return launch_grouped_t<Cfg128x128, EPI>(a, gt, E, s);
      case FORGE_TILE_256x128: return launch_grouped_t<Cfg256x128, EPI>(a, gt, E, s);
      case FORGE_TILE_256x256: return launch_grouped_t<Cfg256x256, EPI>(a, gt, E, s);
      default: return FORGE_ERR_TILE;
    }
  }
};

template <bool EXACT, bool GRAD_BF16, bool STATE_BF16>
forge_status launch_adamw_elementwise(const void* grad, float* W, void* m, void* v, int64_t n,
                                      const AdamWConsts& c, hipStream_t s) {
  const int64_t n4 = (n + 3) / 4;
  const int blocks = int(std::min<int64_t>((n4 + 255) / 256, 256 * 16));
  hipLaunchKernelGGL((adamw_elementwise_kernel<EXACT, GRAD_BF16, STATE_BF16>), dim3(blocks),
                     dim3(256), 0, s, grad, W, m, v, n, c);
  return launch_status();
}

template <int EPI>
struct ElementwiseAdamW {
  static forge_status run(const void* grad, bool grad_bf16, float* W, void* m, void* v,
                          bool state_bf16, int64_t n, const AdamWConsts& c, hipStream_t s) {
    constexpr bool X = (EPI & EPI_EXACT_SQRT) != 0;
    if (grad_bf16)
      return state_bf16 ? launch_adamw_elementwise<X, true, true>(grad, W, m, v, n, c, s)
                        : launch_adamw_elementwise<X, true, false>(grad, W, m, v, n, c, s);
    return state_bf16 ? launch_adamw_elementwise<X, false, true>(grad, W, m, v, n, c, s)
                      : launch_adamw_elementwise<X, false, false>(grad, W, m, v, n, c, s);
  }
};

}  // namespace

forge_status launch_wgrad_adamw(const WgradArgs& a, const forge_adamw_params& p, forge_tile tile,
                                hipStream_t s) {
  return with_adamw_epi<DenseLaunch>(p, a, tile, s);
}

forge_status launch_wgrad_sgdm(const WgradArgs& a, forge_tile tile, hipStream_t s) {
  return launch_dense<EPI_SGDM>(a, tile, s);
}

}  // namespace forge

using namespace forge;

extern "C" {

FORGE_API forge_status forge_wgrad_adamw(const void* X, const void* dY, float* W, float* m,
                                         float* v, int64_t T, int64_t d_in, int64_t d_out,
                                         const forge_adamw_params* p, forge_tile tile,
                                         void* stream) {
  if (forge_status s = validate_wgrad_adamw(X, dY, W, m, v, T, d_in, d_out, p, tile)) return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, W, m, v, T, d_in, d_out);
  a.adam = make_adamw(*p);
  return with_adamw_epi<DenseLaunch>(*p, a, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad_sgdm(const void* X, const void* dY, float* W, float* mom,
                                        int64_t T, int64_t d_in, int64_t d_out,
                                        const forge_sgdm_params* p, forge_tile tile,
                                        void* stream) {
  if (forge_status s = validate_wgrad_sgdm(X, dY, W, mom, T, d_in, d_out, p, tile)) return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, W, mom, nullptr, T, d_in, d_out);
  a.sgd = make_sgdm(*p);
  return launch_dense<EPI_SGDM>(a, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad(const void* X, const void* dY, float* grad, int64_t T,
                                   int64_t d_in, int64_t d_out, forge_tile tile, void* stream) {
  if (forge_status s = validate_wgrad(X, dY, grad, T, d_in, d_out, tile)) return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, grad, nullptr, nullptr, T, d_in, d_out);
  return launch_dense<EPI_GRAD>(a, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_adamw(const float* grad, float* W, float* m, float* v, int64_t n,
                                   const forge_adamw_params* p, void* stream) {
  if (forge_status s = validate_adamw(grad, W, m, v, n, p)) return s;
  if (n == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  (void)hipGetLastError();
  return with_adamw_epi<ElementwiseAdamW>(*p, grad, false, W, m, v, false, n, make_adamw(*p),
                                          static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_sgdm(const float* grad, float* W, float* mom, int64_t n,
                                  const forge_sgdm_params* p, void* stream) {
  if (forge_status s = validate_sgdm(grad, W, mom, n, p)) return s;
  if (n == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  (void)hipGetLastError();
  const int64_t n4 = (n + 3) / 4;
  const int blocks = int(std::min<int64_t>((n4 + 255) / 256, 256 * 16));
  hipLaunchKernelGGL(sgdm_elementwise_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), grad, W, mom, n, make_sgdm(*p));
  return launch_status();
}

FORGE_API forge_status forge_grouped_wgrad_adamw(const void* X_perm, const void* dY_perm,
                                                 const int64_t* offsets, int32_t E, float* W,
                                                 float* m, float* v, int64_t d_in, int64_t d_out,
                                                 const forge_adamw_params* p, forge_tile tile,
                                                 void* stream) {
  if (forge_status s = validate_grouped_adamw(X_perm, dY_perm, offsets, E, W, m, v, d_in, d_out,
                                              p, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, E, /*allow_persistent=*/false);
  if (!grid_fits(d_in, d_out, tile, E)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  GroupTable gt;
  std::memset(&gt, 0, sizeof(gt));
  for (int32_t e = 0; e <= E; ++e) gt.off[e] = offsets[e];
  // Launch order: most rows first, so the heavy experts start early and the
  // empty ones (epilogue only) fill the tail.
  for (int32_t e = 0; e < E; ++e) gt.order[e] = e;
  std::stable_sort(gt.order, gt.order + E, [&](int32_t x, int32_t y) {
    return offsets[x + 1] - offsets[x] > offsets[y + 1] - offsets[y];
  });
  WgradArgs a = base_args(X_perm, dY_perm, W, m, v, 0, d_in, d_out);
  a.adam = make_adamw(*p);
  return with_adamw_epi<GroupedLaunch>(*p, a, gt, E, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_grouped_wgrad_sgdm(const void* X_perm, const void* dY_perm,
                                                const int64_t* offsets, int32_t E, float* W,
                                                float* mom, int64_t d_in, int64_t d_out,
                                                const forge_sgdm_params* p, forge_tile tile,
                                                void* stream) {
  if (forge_status s = validate_grouped_sgdm(X_perm, dY_perm, offsets, E, W, mom, d_in, d_out, p,
                                             tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, E, /*allow_persistent=*/false);
  if (!grid_fits(d_in, d_out, tile, E)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  GroupTable gt;
  std::memset(&gt, 0, sizeof(gt));
  for (int32_t e = 0; e <= E; ++e) gt.off[e] = offsets[e];
  for (int32_t e = 0; e < E; ++e) gt.order[e] = e;
  std::stable_sort(gt.order, gt.order + E, [&](int32_t x, int32_t y) {
    return offsets[x + 1] - offsets[x] > offsets[y + 1] - offsets[y];
  });
  WgradArgs a = base_args(X_perm, dY_perm, W, mom, nullptr, 0, d_in, d_out);
  a.sgd = make_sgdm(*p);
  return GroupedLaunch<EPI_SGDM>::run(a, gt, E, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad_bf16(const void* X, const void* dY, void* grad_bf16,
                                        int64_t T, int64_t d_in, int64_t d_out, forge_tile tile,
                                        void* stream) {
  if (forge_status s = validate_wgrad_bf16(X, dY, grad_bf16, T, d_in, d_out, tile)) return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, static_cast<float*>(grad_bf16), nullptr, nullptr, T, d_in, d_out);
  return launch_dense<EPI_GRAD | EPI_BF16_OUT>(a, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_wgrad_adamw_bf16state(const void* X, const void* dY, float* W,
                                                   void* m_bf16, void* v_bf16, int64_t T,
                                                   int64_t d_in, int64_t d_out,
                                                   const forge_adamw_params* p, forge_tile tile,
                                                   void* stream) {
  if (forge_status s =
          validate_wgrad_adamw_bf16state(X, dY, W, m_bf16, v_bf16, T, d_in, d_out, p, tile))
    return s;
  if (d_in == 0 || d_out == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  tile = resolve_tile(tile, d_in, d_out, 1);
  if (!grid_fits(d_in, d_out, tile, 1)) return FORGE_ERR_SHAPE;
  (void)hipGetLastError();
  WgradArgs a = base_args(X, dY, W, static_cast<float*>(m_bf16), static_cast<float*>(v_bf16), T,
                          d_in, d_out);
  a.adam = make_adamw(*p);
  return with_adamw_epi<DenseLaunch, EPI_ADAMW | EPI_BF16_STATE>(
      *p, a, tile, static_cast<hipStream_t>(stream));
}

FORGE_API forge_status forge_adamw_mixed(const void* grad, forge_dtype grad_dtype, float* W,
                                         void* m, void* v, forge_dtype state_dtype, int64_t n,
                                         const forge_adamw_params* p, void* stream) {
  if (forge_status s = validate_adamw_mixed(grad, grad_dtype, W, m, v, state_dtype, n, p))
    return s;
  if (n == 0) return FORGE_OK;
  if (forge_status s = check_device()) return s;
  (void)hipGetLastError();
  return with_adamw_epi<ElementwiseAdamW>(*p, grad, grad_dtype == FORGE_BF16, W, m, v,
                                          state_dtype == FORGE_BF16, n, make_adamw(*p),
                                          static_cast<hipStream_t>(stream));
}

FORGE_API const char* forge_status_string(forge_status s) {
  switch (s) {
    case FORGE_OK: return "ok";
    case FORGE_ERR_NULL: return "a required pointer is NULL";
    case FORGE_ERR_SHAPE: return "invalid or unsupported size";
    case FORGE_ERR_ALIGN: return "pointer not 16-byte aligned, or d_in/d_out not a multiple of 8";
    case FORGE_ERR_ALIAS: return "output buffers overlap each other or an input";
    case FORGE_ERR_HPARAM: return "hyperparameter out of range";
    case FORGE_ERR_CLIP_NOT_FUSABLE:
      return "global-norm clipping cannot be fused into the weight-gradient epilogue";
    case FORGE_ERR_TILE: return "unknown tile id";
    case FORGE_ERR_DEVICE: return "no gfx950 device is current";
    case FORGE_ERR_LAUNCH: return "kernel launch failed";
    case FORGE_ERR_DTYPE: return "unknown element type";
    default: return "unknown status";
  }
}

}  // extern "C"
