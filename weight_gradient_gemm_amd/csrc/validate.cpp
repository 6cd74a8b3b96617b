// Host-side argument validation for the forge C ABI (pure C++, no HIP).
#include "validate.hpp"

#include <cmath>

namespace forge {

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

// Rejects NaN as well as anything outside [0, 1).
bool unit_interval(double x) { return x >= 0.0 && x < 1.0; }

forge_status check_clip(double max_grad_norm) {
  if (std::isnan(max_grad_norm) || max_grad_norm < 0.0) return FORGE_ERR_HPARAM;
  if (max_grad_norm > 0.0) return FORGE_ERR_CLIP_NOT_FUSABLE;
  return FORGE_OK;
}

forge_status check_outs_disjoint(const Span* spans, int n) {
  for (int a = 0; a < n; ++a)
    for (int b = a + 1; b < n; ++b)
      if (spans_overlap(spans[a], spans[b])) return FORGE_ERR_ALIAS;
  return FORGE_OK;
}

}  // namespace

bool spans_overlap(const Span& a, const Span& b) {
  if (a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

forge_status check_tile(forge_tile tile) {
  return (tile >= 0 && tile < FORGE_TILE_COUNT) ? FORGE_OK : FORGE_ERR_TILE;
}

int dtype_bytes(forge_dtype t) { return t == FORGE_F32 ? 4 : (t == FORGE_BF16 ? 2 : 0); }

forge_status check_dense(const void* X, const void* dY, const void* const* outs, int n_outs,
                         int64_t T, int64_t d_in, int64_t d_out) {
  const int four[6] = {4, 4, 4, 4, 4, 4};
  return check_dense_sized(X, dY, outs, four, n_outs, T, d_in, d_out);
}

forge_status check_dense_sized(const void* X, const void* dY, const void* const* outs,
                               const int* elem_bytes, int n_outs, int64_t T, int64_t d_in,
                               int64_t d_out, int in_bytes) {
  if (T < 0 || d_in < 0 || d_out < 0) return FORGE_ERR_SHAPE;
  const bool empty_out = d_in == 0 || d_out == 0;
  if (!empty_out) {
    for (int k = 0; k < n_outs; ++k)
      if (!outs[k]) return FORGE_ERR_NULL;
    if (T > 0 && (!X || !dY)) return FORGE_ERR_NULL;
  }
  if (T > kMaxTokens || d_in > kMaxDim || d_out > kMaxDim) return FORGE_ERR_SHAPE;
  if (d_in * d_out > kMaxElems) return FORGE_ERR_SHAPE;
  if (empty_out) return FORGE_OK;
  const int64_t mult = 16 / in_bytes;        // 16-byte chunks of a token row
  if ((d_in % mult) != 0 || (d_out % mult) != 0 || (d_in % 8) != 0 || (d_out % 8) != 0)
    return FORGE_ERR_ALIGN;
  for (int k = 0; k < n_outs; ++k)
    if (!aligned16(outs[k])) return FORGE_ERR_ALIGN;
  if (T > 0 && (!aligned16(X) || !aligned16(dY))) return FORGE_ERR_ALIGN;

  Span spans[6] = {};
  int n = 0;
  const uint64_t elems = uint64_t(d_in) * uint64_t(d_out);
  for (int k = 0; k < n_outs; ++k) spans[n++] = Span{outs[k], elems * uint64_t(elem_bytes[k])};
  if (forge_status s = check_outs_disjoint(spans, n)) return s;
  if (T > 0) {
    const Span sx{X, uint64_t(T) * uint64_t(d_in) * uint64_t(in_bytes)},
        sy{dY, uint64_t(T) * uint64_t(d_out) * uint64_t(in_bytes)};
    for (int k = 0; k < n_outs; ++k)
      if (spans_overlap(spans[k], sx) || spans_overlap(spans[k], sy)) return FORGE_ERR_ALIAS;
  }
  return FORGE_OK;
}

forge_status check_adamw_params(const forge_adamw_params* p) {
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_clip(p->max_grad_norm)) return s;
  if (!finite_nonneg(p->lr) || !unit_interval(p->beta1) || !unit_interval(p->beta2) ||
      !finite_nonneg(p->eps) || !finite_nonneg(p->weight_decay) || p->step < 1)
    return FORGE_ERR_HPARAM;
  return FORGE_OK;
}

forge_status check_sgdm_params(const forge_sgdm_params* p) {
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_clip(p->max_grad_norm)) return s;
  if (!finite_nonneg(p->lr) || !unit_interval(p->momentum) || !finite_nonneg(p->weight_decay))
    return FORGE_ERR_HPARAM;
  return FORGE_OK;
}

forge_status check_elementwise(const float* grad, const float* const* outs, int n_outs,
                               int64_t n) {
  const void* o[4] = {};
  const int four[4] = {4, 4, 4, 4};
  for (int k = 0; k < n_outs; ++k) o[k] = outs[k];
  return check_elementwise_sized(grad, 4, o, four, n_outs, n);
}

forge_status check_elementwise_sized(const void* grad, int grad_bytes, const void* const* outs,
                                     const int* elem_bytes, int n_outs, int64_t n) {
  if (n < 0) return FORGE_ERR_SHAPE;
  if (n == 0) return FORGE_OK;
  if (!grad) return FORGE_ERR_NULL;
  for (int k = 0; k < n_outs; ++k)
    if (!outs[k]) return FORGE_ERR_NULL;
  if (n > kMaxElems) return FORGE_ERR_SHAPE;
  if (!aligned16(grad)) return FORGE_ERR_ALIGN;
  for (int k = 0; k < n_outs; ++k)
    if (!aligned16(outs[k])) return FORGE_ERR_ALIGN;
  Span spans[4] = {};
  int m = 0;
  for (int k = 0; k < n_outs; ++k) spans[m++] = Span{outs[k], uint64_t(n) * uint64_t(elem_bytes[k])};
  if (forge_status s = check_outs_disjoint(spans, m)) return s;
  const Span sg{grad, uint64_t(n) * uint64_t(grad_bytes)};
  for (int k = 0; k < m; ++k)
    if (spans_overlap(spans[k], sg)) return FORGE_ERR_ALIAS;
  return FORGE_OK;
}

forge_status check_grouped(const void* X_perm, const void* dY_perm, const int64_t* offsets,
                           int32_t E, const void* const* outs, int n_outs, int64_t d_in,
                           int64_t d_out) {
  if (!offsets) return FORGE_ERR_NULL;
  if (E < 1 || E > FORGE_MAX_EXPERTS) return FORGE_ERR_SHAPE;
  if (offsets[0] != 0) return FORGE_ERR_SHAPE;
  for (int32_t e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return FORGE_ERR_SHAPE;
  const int64_t R = offsets[E];
  if (d_in < 0 || d_out < 0) return FORGE_ERR_SHAPE;
  const bool empty_out = d_in == 0 || d_out == 0;
  if (!empty_out) {
    for (int k = 0; k < n_outs; ++k)
      if (!outs[k]) return FORGE_ERR_NULL;
    if (R > 0 && (!X_perm || !dY_perm)) return FORGE_ERR_NULL;
  }
  if (R > kMaxTokens || d_in > kMaxDim || d_out > kMaxDim) return FORGE_ERR_SHAPE;
  if (d_in * d_out > kMaxElems / E) return FORGE_ERR_SHAPE;
  if (empty_out) return FORGE_OK;
  if ((d_in % 8) != 0 || (d_out % 8) != 0) return FORGE_ERR_ALIGN;
  for (int k = 0; k < n_outs; ++k)
    if (!aligned16(outs[k])) return FORGE_ERR_ALIGN;
  if (R > 0 && (!aligned16(X_perm) || !aligned16(dY_perm))) return FORGE_ERR_ALIGN;
  Span spans[4] = {};
  int n = 0;
  const uint64_t state_bytes = uint64_t(E) * uint64_t(d_in) * uint64_t(d_out) * 4u;
  for (int k = 0; k < n_outs; ++k) spans[n++] = Span{outs[k], state_bytes};
  if (forge_status s = check_outs_disjoint(spans, n)) return s;
  if (R > 0) {
    const Span sx{X_perm, uint64_t(R) * uint64_t(d_in) * 2u};
    const Span sy{dY_perm, uint64_t(R) * uint64_t(d_out) * 2u};
    for (int k = 0; k < n; ++k)
      if (spans_overlap(spans[k], sx) || spans_overlap(spans[k], sy)) return FORGE_ERR_ALIAS;
  }
  return FORGE_OK;
}

forge_status validate_wgrad_adamw(const void* X, const void* dY, const float* W, const float* m,
                                  const float* v, int64_t T, int64_t d_in, int64_t d_out,
                                  const forge_adamw_params* p, forge_tile tile) {
  const void* outs[3] = {W, m, v};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense(X, dY, outs, 3, T, d_in, d_out)) return s;
  if (forge_status s = check_adamw_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_wgrad_sgdm(const void* X, const void* dY, const float* W, const float* mom,
                                 int64_t T, int64_t d_in, int64_t d_out,
                                 const forge_sgdm_params* p, forge_tile tile) {
  const void* outs[2] = {W, mom};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense(X, dY, outs, 2, T, d_in, d_out)) return s;
  if (forge_status s = check_sgdm_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_wgrad(const void* X, const void* dY, const float* grad, int64_t T,
                            int64_t d_in, int64_t d_out, forge_tile tile) {
  const void* outs[1] = {grad};
  if (forge_status s = check_dense(X, dY, outs, 1, T, d_in, d_out)) return s;
  return check_tile(tile);
}

forge_status validate_adamw(const float* grad, const float* W, const float* m, const float* v,
                            int64_t n, const forge_adamw_params* p) {
  const float* outs[3] = {W, m, v};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_elementwise(grad, outs, 3, n)) return s;
  return check_adamw_params(p);
}

forge_status validate_sgdm(const float* grad, const float* W, const float* mom, int64_t n,
                           const forge_sgdm_params* p) {
  const float* outs[2] = {W, mom};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_elementwise(grad, outs, 2, n)) return s;
  return check_sgdm_params(p);
}

forge_status validate_wgrad_bf16(const void* X, const void* dY, const void* grad, int64_t T,
                                 int64_t d_in, int64_t d_out, forge_tile tile) {
  const void* outs[1] = {grad};
  const int bytes[1] = {2};
  if (forge_status s = check_dense_sized(X, dY, outs, bytes, 1, T, d_in, d_out)) return s;
  return check_tile(tile);
}

forge_status validate_wgrad_adamw_bf16state(const void* X, const void* dY, const float* W,
                                            const void* m, const void* v, int64_t T,
                                            int64_t d_in, int64_t d_out,
                                            const forge_adamw_params* p, forge_tile tile) {
  const void* outs[3] = {W, m, v};
  const int bytes[3] = {4, 2, 2};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense_sized(X, dY, outs, bytes, 3, T, d_in, d_out)) return s;
  if (forge_status s = check_adamw_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_adamw_mixed(const void* grad, forge_dtype grad_dtype, const float* W,
                                  const void* m, const void* v, forge_dtype state_dtype,
                                  int64_t n, const forge_adamw_params* p) {
  const int gb = dtype_bytes(grad_dtype), sb = dtype_bytes(state_dtype);
  const void* outs[3] = {W, m, v};
  const int bytes[3] = {4, sb, sb};
  if (!p) return FORGE_ERR_NULL;
  if (gb == 0 || sb == 0) return FORGE_ERR_DTYPE;
  if (forge_status s = check_elementwise_sized(grad, gb, outs, bytes, 3, n)) return s;
  return check_adamw_params(p);
}

forge_status validate_grouped_adamw(const void* X_perm, const void* dY_perm,
                                    const int64_t* offsets, int32_t E, const float* W,
                                    const float* m, const float* v, int64_t d_in, int64_t d_out,
                                    const forge_adamw_params* p, forge_tile tile) {
  const void* outs[3] = {W, m, v};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_grouped(X_perm, dY_perm, offsets, E, outs, 3, d_in, d_out)) return s;
  if (forge_status s = check_adamw_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_grouped_sgdm(const void* X_perm, const void* dY_perm,
                                   const int64_t* offsets, int32_t E, const float* W,
                                   const float* mom, int64_t d_in, int64_t d_out,
                                   const forge_sgdm_params* p, forge_tile tile) {
  const void* outs[2] = {W, mom};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_grouped(X_perm, dY_perm, offsets, E, outs, 2, d_in, d_out)) return s;
  if (forge_status s = check_sgdm_params(p)) return s;
  return check_tile(tile);
}

namespace {

bool is_fp8(forge_dtype t) { return t == FORGE_FP8_E4M3 || t == FORGE_FP8_E5M2; }

// Per-tensor scales: finite and positive, with a float32 product that is too.
forge_status check_fp8_scales(double x_scale, double dy_scale) {
  if (!(std::isfinite(x_scale) && x_scale > 0.0 && std::isfinite(dy_scale) && dy_scale > 0.0))
    return FORGE_ERR_HPARAM;
  const float g = float(x_scale * dy_scale);
  return std::isfinite(g) && g >= 1.17549435e-38f ? FORGE_OK : FORGE_ERR_HPARAM;
}

}  // namespace

forge_status validate_wgrad_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                const void* dY8, forge_dtype dy_fmt, double dy_scale,
                                const float* grad, int64_t T, int64_t d_in, int64_t d_out,
                                forge_tile tile) {
  if (!is_fp8(x_fmt) || !is_fp8(dy_fmt)) return FORGE_ERR_DTYPE;
  const void* outs[1] = {grad};
  const int bytes[1] = {4};
  if (forge_status s = check_dense_sized(X8, dY8, outs, bytes, 1, T, d_in, d_out, 1)) return s;
  if (forge_status s = check_fp8_scales(x_scale, dy_scale)) return s;
  return check_tile(tile);
}

forge_status validate_wgrad_adamw_fp8(const void* X8, forge_dtype x_fmt, double x_scale,
                                      const void* dY8, forge_dtype dy_fmt, double dy_scale,
                                      const float* W, const float* m, const float* v, int64_t T,
                                      int64_t d_in, int64_t d_out, const forge_adamw_params* p,
                                      forge_tile tile) {
  if (!is_fp8(x_fmt) || !is_fp8(dy_fmt)) return FORGE_ERR_DTYPE;
  const void* outs[3] = {W, m, v};
  const int bytes[3] = {4, 4, 4};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense_sized(X8, dY8, outs, bytes, 3, T, d_in, d_out, 1)) return s;
  if (forge_status s = check_adamw_params(p)) return s;
  if (forge_status s = check_fp8_scales(x_scale, dy_scale)) return s;
  return check_tile(tile);
}

namespace {

// dX = dY W with W of w_bytes bytes per element (float32 or its bf16 copy).
forge_status check_dgrad(const void* dY, const void* W, int w_bytes, const void* dX,
                         forge_dtype dX_dtype, int64_t T, int64_t d_in, int64_t d_out,
                         forge_tile tile) {
  const int xb = dtype_bytes(dX_dtype);
  if (xb == 0) return FORGE_ERR_DTYPE;
  if (T < 0 || d_in < 0 || d_out < 0) return FORGE_ERR_SHAPE;
  if (T == 0 || d_in == 0) return check_tile(tile);      // dX is empty
  if (!dX) return FORGE_ERR_NULL;
  if (d_out > 0 && (!dY || !W)) return FORGE_ERR_NULL;
  if (T > kMaxTokens || d_in > kMaxDim || d_out > kMaxDim) return FORGE_ERR_SHAPE;
  if ((d_in % 8) != 0 || (d_out % 8) != 0) return FORGE_ERR_ALIGN;
  if (!aligned16(dX)) return FORGE_ERR_ALIGN;
  if (d_out > 0 && (!aligned16(dY) || !aligned16(W))) return FORGE_ERR_ALIGN;
  const Span sx{dX, uint64_t(T) * uint64_t(d_in) * uint64_t(xb)};
  const Span sy{dY, uint64_t(T) * uint64_t(d_out) * 2u};
  const Span sw{W, uint64_t(d_out) * uint64_t(d_in) * uint64_t(w_bytes)};
  if (spans_overlap(sx, sy) || spans_overlap(sx, sw)) return FORGE_ERR_ALIAS;
  return check_tile(tile);
}

// The linear-backward calls: dX must also stay clear of X and the state
// the fused step writes.
forge_status check_dx_clear(const void* dX, forge_dtype dX_dtype, int64_t T, int64_t d_in,
                            int64_t d_out, const void* X, const void* const* state, int n) {
  if (T == 0 || d_in == 0) return FORGE_OK;
  const Span sx{dX, uint64_t(T) * uint64_t(d_in) * uint64_t(dtype_bytes(dX_dtype))};
  if (spans_overlap(sx, Span{X, uint64_t(T) * uint64_t(d_in) * 2u})) return FORGE_ERR_ALIAS;
  for (int k = 0; k < n; ++k)
    if (spans_overlap(sx, Span{state[k], uint64_t(d_in) * uint64_t(d_out) * 4u}))
      return FORGE_ERR_ALIAS;
  return FORGE_OK;
}

}  // namespace

forge_status validate_dgrad(const void* dY, const float* W, const void* dX, forge_dtype dX_dtype,
                            int64_t T, int64_t d_in, int64_t d_out, forge_tile tile) {
  return check_dgrad(dY, W, 4, dX, dX_dtype, T, d_in, d_out, tile);
}

forge_status validate_dgrad_bf16w(const void* dY, const void* Wb, const void* dX,
                                  forge_dtype dX_dtype, int64_t T, int64_t d_in, int64_t d_out,
                                  forge_tile tile) {
  return check_dgrad(dY, Wb, 2, dX, dX_dtype, T, d_in, d_out, tile);
}

forge_status validate_linear_backward_adamw(const void* X, const void* dY, const float* W,
                                            const float* m, const float* v, const void* dX,
                                            forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                            int64_t d_out, const forge_adamw_params* p,
                                            forge_tile tile) {
  if (forge_status s = validate_wgrad_adamw(X, dY, W, m, v, T, d_in, d_out, p, tile)) return s;
  if (forge_status s = validate_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, FORGE_TILE_DEFAULT))
    return s;
  const void* state[2] = {m, v};
  return check_dx_clear(dX, dX_dtype, T, d_in, d_out, X, state, 2);
}

forge_status validate_linear_backward_sgdm(const void* X, const void* dY, const float* W,
                                           const float* mom, const void* dX, forge_dtype dX_dtype,
                                           int64_t T, int64_t d_in, int64_t d_out,
                                           const forge_sgdm_params* p, forge_tile tile) {
  if (forge_status s = validate_wgrad_sgdm(X, dY, W, mom, T, d_in, d_out, p, tile)) return s;
  if (forge_status s = validate_dgrad(dY, W, dX, dX_dtype, T, d_in, d_out, FORGE_TILE_DEFAULT))
    return s;
  const void* state[1] = {mom};
  return check_dx_clear(dX, dX_dtype, T, d_in, d_out, X, state, 1);
}

// The bf16-copy calls: Wb is written by the fused step, so it is checked as
// one more output (disjoint from W, the state, X and dY); in the
// linear-backward calls dX is read from Wb and must stay clear of W as well.
forge_status validate_wgrad_adamw_bf16w(const void* X, const void* dY, const float* W,
                                        const float* m, const float* v, const void* Wb,
                                        int64_t T, int64_t d_in, int64_t d_out,
                                        const forge_adamw_params* p, forge_tile tile) {
  const void* outs[4] = {W, m, v, Wb};
  const int bytes[4] = {4, 4, 4, 2};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense_sized(X, dY, outs, bytes, 4, T, d_in, d_out)) return s;
  if (forge_status s = check_adamw_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_wgrad_sgdm_bf16w(const void* X, const void* dY, const float* W,
                                       const float* mom, const void* Wb, int64_t T, int64_t d_in,
                                       int64_t d_out, const forge_sgdm_params* p,
                                       forge_tile tile) {
  const void* outs[3] = {W, mom, Wb};
  const int bytes[3] = {4, 4, 2};
  if (!p) return FORGE_ERR_NULL;
  if (forge_status s = check_dense_sized(X, dY, outs, bytes, 3, T, d_in, d_out)) return s;
  if (forge_status s = check_sgdm_params(p)) return s;
  return check_tile(tile);
}

forge_status validate_linear_backward_adamw_bf16w(const void* X, const void* dY, const float* W,
                                                  const float* m, const float* v, const void* Wb,
                                                  const void* dX, forge_dtype dX_dtype, int64_t T,
                                                  int64_t d_in, int64_t d_out,
                                                  const forge_adamw_params* p, forge_tile tile) {
  if (forge_status s = validate_wgrad_adamw_bf16w(X, dY, W, m, v, Wb, T, d_in, d_out, p, tile))
    return s;
  if (forge_status s = check_dgrad(dY, Wb, 2, dX, dX_dtype, T, d_in, d_out, FORGE_TILE_DEFAULT))
    return s;
  const void* state[3] = {W, m, v};
  return check_dx_clear(dX, dX_dtype, T, d_in, d_out, X, state, 3);
}

forge_status validate_linear_backward_sgdm_bf16w(const void* X, const void* dY, const float* W,
                                                 const float* mom, const void* Wb, const void* dX,
                                                 forge_dtype dX_dtype, int64_t T, int64_t d_in,
                                                 int64_t d_out, const forge_sgdm_params* p,
                                                 forge_tile tile) {
  if (forge_status s = validate_wgrad_sgdm_bf16w(X, dY, W, mom, Wb, T, d_in, d_out, p, tile))
    return s;
  if (forge_status s = check_dgrad(dY, Wb, 2, dX, dX_dtype, T, d_in, d_out, FORGE_TILE_DEFAULT))
    return s;
  const void* state[2] = {W, mom};
  return check_dx_clear(dX, dX_dtype, T, d_in, d_out, X, state, 2);
}

}  // namespace forge
