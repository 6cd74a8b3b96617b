// Host-side argument validation for the forge C ABI. Pure C++: no HIP calls,
// so every error path can be exercised on a machine without a GPU.
//
// Order of checks (the first failing one is returned): NULL, SHAPE, ALIGN,
// ALIAS, CLIP_NOT_FUSABLE, HPARAM, TILE. The device check and the launch come
// after validation, in the HIP translation unit.
#pragma once

#include <cstdint>

#include "forge.h"

namespace forge {

struct Span {
  const void* p;
  uint64_t bytes;
};

// True if the two byte ranges overlap (empty ranges never overlap).
bool spans_overlap(const Span& a, const Span& b);

forge_status check_dense(const void* X, const void* dY, const void* const* outs, int n_outs,
                         int64_t T, int64_t d_in, int64_t d_out);
// As check_dense, with out k holding elem_bytes[k] bytes per element and X,
// dY in_bytes per element (fp8 inputs: 1, and d_in, d_out multiples of 16).
forge_status check_dense_sized(const void* X, const void* dY, const void* const* outs,
                               const int* elem_bytes, int n_outs, int64_t T, int64_t d_in,
                               int64_t d_out, int in_bytes = 2);
// Element size of a forge_dtype, or 0 if unknown.
int dtype_bytes(forge_dtype t);
forge_status check_adamw_params(const forge_adamw_params* p);
forge_status check_sgdm_params(const forge_sgdm_params* p);
forge_status check_tile(forge_tile tile);
forge_status check_elementwise(const float* grad, const float* const* outs, int n_outs, int64_t n);
forge_status check_elementwise_sized(const void* grad, int grad_bytes, const void* const* outs,
                                     const int* elem_bytes, int n_outs, int64_t n);
forge_status check_grouped(const void* X_perm, const void* dY_perm, const int64_t* offsets,
                           int32_t E, const void* const* outs, int n_outs, int64_t d_in,
                           int64_t d_out);

// Full validation of each entry point, everything except the device.
forge_status validate_wgrad_adamw(const void* X, const void* dY, const float* W, const float* m,
                                  const float* v, int64_t T, int64_t d_in, int64_t d_out,
                                  const forge_adamw_params* p, forge_tile tile);
forge_status validate_wgrad_sgdm(const void* X, const void* dY, const float* W, const float* mom,
                                 int64_t T, int64_t d_in, int64_t d_out,
                                 const forge_sgdm_params* p, forge_tile tile);
forge_status validate_wgrad(const void* X, const void* dY, const float* grad, int64_t T,
                            int64_t d_in, int64_t d_out, forge_tile tile);
forge_status validate_adamw(const float* grad, const float* W, const float* m, const float* v,
                            int64_t n, const forge_adamw_params* p);
forge_status validate_sgdm(const float* grad, const float* W, const float* mom, int64_t n,
                           const forge_sgdm_params* p);
forge_status validate_wgrad_bf16(const void* X, const void* dY, const void* grad, int64_t T,
                                 int64_t d_in, int64_t d_out, forge_tile tile);
forge_status validate_wgrad_adamw_bf16state(const void* X, const void* dY, const float* W,
                                            const void* m, const void* v, int64_t T,
                                            int64_t d_in, int64_t d_out,
                                            const forge_adamw_params* p, forge_tile tile);
forge_status validate_adamw_mixed(const void* grad, forge_dtype grad_dtype, const float* W,
                                  const void* m, const void* v, forge_dtype state_dtype,
                                  int64_t n, const forge_adamw_params* p);
forge_status validate_wgrad_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                const void* dY8, forge_dtype dy_fmt, double dy_scale,
                                const float* grad, int64_t T, int64_t d_in, int64_t d_out,
                                forge_tile tile);
forge_status validate_wgrad_adamw_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                      const void* dY8, forge_dtype dy_fmt, double dy_scale,
                                      const float* W, const float* m, const float* v, int64_t T,
                                      int64_t d_in, int64_t d_out, const forge_adamw_params* p,
                                      forge_tile tile);
forge_status validate_dgrad(const void* dY, const float* W, const void* dX, forge_dtype dX_dtype,
                            int64_t T, int64_t d_in, int64_t d_out, forge_tile tile);
forge_status validate_linear_backward_adamw(const void* X, const void* dY, const float* W,
                                            const float* m, const float* v, const void* dX,
                                            forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                            int64_t d_out, const forge_adamw_params* p,
                                            forge_tile tile);
forge_status validate_linear_backward_sgdm(const void* X, const void* dY, const float* W,
                                           const float* mom, const void* dX, forge_dtype dX_dtype,
                                           int64_t T, int64_t d_in, int64_t d_out,
                                           const forge_sgdm_params* p, forge_tile tile);
forge_status validate_dgrad_bf16w(const void* dY, const void* Wb, const void* dX,
                                  forge_dtype dX_dtype, int64_t T, int64_t d_in, int64_t d_out,
                                  forge_tile tile);
forge_status validate_wgrad_adamw_bf16w(const void* X, const void* dY, const float* W,
                                        const float* m, const float* v, const void* Wb,
                                        int64_t T, int64_t d_in, int64_t d_out,
                                        const forge_adamw_params* p, forge_tile tile);
forge_status validate_wgrad_sgdm_bf16w(const void* X, const void* dY, const float* W,
                                       const float* mom, const void* Wb, int64_t T, int64_t d_in,
                                       int64_t d_out, const forge_sgdm_params* p,
                                       forge_tile tile);
forge_status validate_linear_backward_adamw_bf16w(const void* X, const void* dY, const float* W,
                                                  const float* m, const float* v, const void* Wb,
                                                  const void* dX, forge_dtype dX_dtype, int64_t T,
                                                  int64_t d_in, int64_t d_out,
                                                  const forge_adamw_params* p, forge_tile tile);
forge_status validate_linear_backward_sgdm_bf16w(const void* X, const void* dY, const float* W,
                                                 const float* mom, const void* Wb, const void* dX,
                                                 forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                                 int64_t d_out, const forge_sgdm_params* p,
                                                 forge_tile tile);
forge_status validate_grouped_adamw(const void* X_perm, const void* dY_perm,
                                    const int64_t* offsets, int32_t E, const float* W,
                                    const float* m, const float* v, int64_t d_in, int64_t d_out,
                                    const forge_adamw_params* p, forge_tile tile);
forge_status validate_grouped_sgdm(const void* X_perm, const void* dY_perm,
                                   const int64_t* offsets, int32_t E, const float* W,
                                   const float* mom, int64_t d_in, int64_t d_out,
                                   const forge_sgdm_params* p, forge_tile tile);

// Largest d_in and d_out: one LDS stage of token rows must stay within a
// 31-bit byte window (32-bit row/column indices, 64-bit element offsets).
constexpr int64_t kMaxDim = int64_t(1) << 22;
constexpr int64_t kMaxTokens = int64_t(1) << 30;
// One buffer of the optimizer state, in elements (64-bit offsets; bounded so
// byte counts never overflow).
constexpr int64_t kMaxElems = int64_t(1) << 40;

}  // namespace forge
