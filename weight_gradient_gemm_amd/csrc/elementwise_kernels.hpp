// Unfused elementwise optimizer kernels: the second half of the
// HBM-materialising comparison path (a stored gradient, then the optimizer).
// The arithmetic is the fused epilogue's (optim_math.hpp), so fused and
// unfused results are bitwise equal.
#pragma once

#include <type_traits>

#include "wgrad_kernels.hpp"

namespace forge {

// Unfused elementwise optimizers (the HBM-materialising comparison path).
// AdamW reads a float32 or bf16 gradient and keeps m, v in float32 or bf16
// (W is float32); the arithmetic is the fused epilogue's, in float32.
template <bool EXACT_SQRT, bool GRAD_BF16, bool STATE_BF16>
__global__ __launch_bounds__(256) void adamw_elementwise_kernel(const void* __restrict__ grad,
                                                                float* __restrict__ W,
                                                                void* __restrict__ m_,
                                                                void* __restrict__ v_, int64_t n,
                                                                AdamWConsts c) {
  typedef typename std::conditional<GRAD_BF16, __bf16, float>::type GT;
  typedef typename std::conditional<STATE_BF16, __bf16, float>::type ST;
  typedef GT gt4 __attribute__((ext_vector_type(4)));
  typedef ST st4 __attribute__((ext_vector_type(4)));
  const GT* g = static_cast<const GT*>(grad);
  ST* m = static_cast<ST*>(m_);
  ST* v = static_cast<ST*>(v_);
  const int64_t n4 = n >> 2;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n4; k += stride) {
    const f32x4_t gg = __builtin_convertvector(reinterpret_cast<const gt4*>(g)[k], f32x4_t);
    f32x4_t w = reinterpret_cast<const f32x4_t*>(W)[k];
    f32x4_t mm = __builtin_convertvector(reinterpret_cast<const st4*>(m)[k], f32x4_t);
    f32x4_t vv = __builtin_convertvector(reinterpret_cast<const st4*>(v)[k], f32x4_t);
    adamw_vec4<EXACT_SQRT>(gg, w, mm, vv, c);
    reinterpret_cast<f32x4_t*>(W)[k] = w;
    reinterpret_cast<st4*>(m)[k] = __builtin_convertvector(mm, st4);
    reinterpret_cast<st4*>(v)[k] = __builtin_convertvector(vv, st4);
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t k = (n4 << 2) + threadIdx.x;
    float w = W[k], mm = float(m[k]), vv = float(v[k]);
    adamw_elem<EXACT_SQRT>(float(g[k]), w, mm, vv, c);
    W[k] = w;
    m[k] = ST(mm);
    v[k] = ST(vv);
  }
}

__global__ __launch_bounds__(256) void sgdm_elementwise_kernel(const float* __restrict__ g,
                                                               float* __restrict__ W,
                                                               float* __restrict__ mom, int64_t n,
                                                               SgdmConsts c) {
  const int64_t n4 = n >> 2;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n4; k += stride) {
    const f32x4_t gg = reinterpret_cast<const f32x4_t*>(g)[k];
    f32x4_t w = reinterpret_cast<const f32x4_t*>(W)[k];
    f32x4_t b = reinterpret_cast<const f32x4_t*>(mom)[k];
    sgdm_vec4(gg, w, b, c);
    reinterpret_cast<f32x4_t*>(W)[k] = w;
    reinterpret_cast<f32x4_t*>(mom)[k] = b;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t k = (n4 << 2) + threadIdx.x;
    float w = W[k], b = mom[k];
    sgdm_elem(g[k], w, b, c);
    W[k] = w;
    mom[k] = b;
  }
}

}  // namespace forge
