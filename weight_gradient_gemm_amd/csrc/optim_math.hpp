// Per-element optimizer arithmetic, shared by the fused epilogues and the
// unfused elementwise kernels so both paths round identically (bitwise).
//
// Built with -ffp-contract=off, so the only fused multiply-adds are the
// explicit ones below. The square root and reciprocal are the hardware
// v_sqrt_f32 and v_rcp_f32 (1 ulp each): the update m_hat / (sqrt(v_hat) + eps)
// then carries a few float32 ulps of relative error, far inside a weight-delta
// accuracy bar of 1e-3 lr, and costs ~11 vector instructions per element
// instead of ~40 for correctly rounded division and square root.
#pragma once

#include <hip/hip_runtime.h>

namespace forge {

// Scalars of one AdamW step, formed on the host in double and rounded once.
struct AdamWConsts {
  float beta1;         // beta1
  float one_m_beta1;   // 1 - beta1
  float beta2;         // beta2
  float one_m_beta2;   // 1 - beta2
  float decay;         // 1 - lr * weight_decay            (decoupled decay)
  float step_size;     // lr / (1 - beta1^t)               (first-moment bias correction)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)            (second-moment bias correction)
  float eps;
};

struct SgdmConsts {
  float momentum;
  float weight_decay;
  float lr;
};

// AdamW with decoupled weight decay (the method's optimizer consumes the float32
// gradient as it leaves the accumulator; FORGE assessment, introduction).
//   m = beta1 m + (1 - beta1) g
//   v = beta2 v + (1 - beta2) g^2
//   w = w (1 - lr wd) - (lr / bc1) m / (sqrt(v) / sqrt(bc2) + eps)
// which is W - lr (m_hat / (sqrt(v_hat) + eps) + wd W) with the bias
// corrections folded into two host-side scalars.
// v_sqrt_f32 is not accurate on float32 denormals. With eps > 0 such a v
// cannot move the denominator by an ulp; callers with eps = 0 instantiate
// EXACT_SQRT, the correctly rounded root.
template <bool EXACT_SQRT>
__device__ __forceinline__ void adamw_elem(float g, float& w, float& m, float& v,
                                           const AdamWConsts& c) {
  m = __builtin_fmaf(c.beta1, m, c.one_m_beta1 * g);
  v = __builtin_fmaf(c.beta2, v, c.one_m_beta2 * (g * g));
  const float s = EXACT_SQRT ? sqrtf(v) : __builtin_amdgcn_sqrtf(v);
  const float denom = __builtin_fmaf(s, c.inv_sqrt_bc2, c.eps);
  const float upd = m * __builtin_amdgcn_rcpf(denom);
  w = __builtin_fmaf(-c.step_size, upd, w * c.decay);
}

// SGD with momentum, coupled weight decay, no dampening:
//   b = momentum b + (g + wd w),  w = w - lr b.
__device__ __forceinline__ void sgdm_elem(float g, float& w, float& b, const SgdmConsts& c) {
  b = __builtin_fmaf(c.momentum, b, __builtin_fmaf(c.weight_decay, w, g));
  w = __builtin_fmaf(-c.lr, b, w);
}

}  // namespace forge
