// Per-element optimizer arithmetic, shared by the fused epilogues and the
// unfused elementwise kernels so both paths round identically.
//
// Built with -ffp-contract=off and IEEE-rounded float32 division and square
// root: every operation below is one correctly rounded float32 operation, in
// the order written.
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
__device__ __forceinline__ void adamw_elem(float g, float& w, float& m, float& v,
                                           const AdamWConsts& c) {
  m = c.beta1 * m + c.one_m_beta1 * g;
  v = c.beta2 * v + c.one_m_beta2 * (g * g);
  const float denom = sqrtf(v) * c.inv_sqrt_bc2 + c.eps;
  w = w * c.decay - c.step_size * (m / denom);
}

// SGD with momentum, coupled weight decay, no dampening.
__device__ __forceinline__ void sgdm_elem(float g, float& w, float& b, const SgdmConsts& c) {
  b = c.momentum * b + (g + c.weight_decay * w);
  w = w - c.lr * b;
}

}  // namespace forge
