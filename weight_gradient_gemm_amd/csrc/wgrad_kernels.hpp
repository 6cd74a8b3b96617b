// Weight-gradient GEMM with optimizer epilogues for gfx950 (CDNA4).
//
// Computes, per output tile of W [d_out, d_in], the float32 accumulator
//     acc[i, o] = sum_t X[t, i] * dY[t, o]        (C = X^T dY, M = d_in, N = d_out)
// over ALL tokens t (the reduction is never split: FORGE assessment, "What's
// already in tree and easy to miss", K kept whole per tile), then consumes acc
// in registers: AdamW / SGD-momentum update of W and its state, or a plain
// float32 store of the gradient for the unfused comparison path.
//
// Mainloop: bf16 MFMA v_mfma_f32_32x32x16_bf16, 4 waves per workgroup, each
// wave owning a (BM/WAVES_M) x (BN/WAVES_N) block of the tile. Both operands
// have the token axis strided (X and dY are row-major [T, d]), so tiles are
// staged through LDS in their natural [token][feature] layout with coalesced
// 16-byte loads along the feature axis, and the MFMA operands (8 consecutive
// tokens per lane) are gathered with the gfx950 LDS transpose read
// ds_read_b64_tr_b16. Stages of 32 tokens, double-buffered, one barrier per
// stage.
//
// Order of accumulation: for every element, the tokens enter in ascending
// chunks of 16 through one accumulator, whatever the tile shape. Ragged token
// tails are zero-filled, so every tile shape and the grouped variant see the
// same chunk sequence, which makes the result bitwise partition-independent.
//
// Epilogue: the MFMA 32x32 result layout gives each lane 4 consecutive rows
// (d_in indices) of one column (a d_out index): exactly 16 contiguous bytes of
// W, m, v in their [d_out, d_in] layout, so the state moves as float4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "forge.h"
#include "optim_math.hpp"

namespace forge {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

enum Epi : int { EPI_ADAMW = 0, EPI_SGDM = 1, EPI_GRAD = 2 };

constexpr int kBK = 32;          // tokens per LDS stage (same for every tile shape)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

struct WgradArgs {
  const uint16_t* X;   // [rows, d_in] bf16 bits
  const uint16_t* dY;  // [rows, d_out] bf16 bits
  float* W;            // [(E,) d_out, d_in]; the gradient for EPI_GRAD
  float* S1;           // m (AdamW) or momentum buffer (SGD)
  float* S2;           // v (AdamW)
  int64_t T;           // tokens (dense calls)
  int32_t d_in;
  int32_t d_out;
  int32_t tiles_m;     // ceil(d_in / BM)
  int32_t tiles_n;     // ceil(d_out / BN)
  int32_t num_tiles;   // tiles_m * tiles_n (* E)
  int32_t group_m;     // tile-order swizzle: tile rows per group
  AdamWConsts adam;
  SgdmConsts sgd;
};

struct GroupTable {
  int64_t off[FORGE_MAX_EXPERTS + 1];
};

// Row stride (elements) of an LDS stage holding `w` features per token: padded
// so that the four token rows read together by a 16-lane transpose read start
// 64 bytes apart modulo 256 (distinct LDS banks).
__host__ __device__ constexpr int lds_stride(int w) {
  return w + ((((w * 2) % 256) == 0) ? 32 : (64 - (w * 2) % 256 + 256) % 256 / 2);
}

// Workgroup -> tile. Workgroups are dispatched round-robin over the 8 XCDs, so
// block b runs on XCD b % 8. Remap so that each XCD gets one contiguous range
// of logical tiles (its L2 then serves neighbouring tiles), then walk the
// logical range in groups of `group_m` tile rows for operand reuse.
__device__ __forceinline__ void map_tile(int b, int num_tiles, int tiles_m, int tiles_n,
                                         int group_m, int& e, int& tm, int& tn) {
  const int xcd = b & 7, local = b >> 3;
  const int per = num_tiles >> 3, rem = num_tiles & 7;
  const int logical = xcd < rem ? xcd * (per + 1) + local
                                : rem * (per + 1) + (xcd - rem) * per + local;
  const int per_expert = tiles_m * tiles_n;
  e = logical / per_expert;
  const int t = logical - e * per_expert;
  const int group_size = group_m * tiles_n;
  const int g = t / group_size;
  const int first_m = g * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int r = t - g * group_size;
  tm = first_m + r % gm;
  tn = r / gm;
}

// The optimizer on the 4 consecutive elements one lane owns.
__device__ __forceinline__ void adamw_vec4(const f32x4_t& g, f32x4_t& w, f32x4_t& m, f32x4_t& v,
                                           const AdamWConsts& c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float wj = w[j], mj = m[j], vj = v[j];
    adamw_elem(g[j], wj, mj, vj, c);
    w[j] = wj;
    m[j] = mj;
    v[j] = vj;
  }
}

__device__ __forceinline__ void sgdm_vec4(const f32x4_t& g, f32x4_t& w, f32x4_t& b,
                                          const SgdmConsts& c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float wj = w[j], bj = b[j];
    sgdm_elem(g[j], wj, bj, c);
    w[j] = wj;
    b[j] = bj;
  }
}

// MFMA operand for a 32-wide feature block at column c0 and the 16 tokens
// starting at row k0 of an LDS stage [token][feature] with row stride LD:
// lane l gets features c0 + (l % 32), tokens k0 + 8 (l / 32) + 0..7.
// Two transpose reads, each giving 4 tokens: within a group of 16 lanes, lane
// j supplies the address of 4 consecutive features of token row j / 4 and
// receives feature j of each of the group's 4 rows.
template <int LD>
__device__ __forceinline__ bf16x8_t load_operand(const uint16_t* s, int k0, int c0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (j >> 2);
  const int col = c0 + 16 * (g & 1) + 4 * (j & 3);
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const uint16_t* p0 = s + row * LD + col;
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * LD));
  const i16x4_t both[2] = {lo, hi};
  bf16x8_t r;
  __builtin_memcpy(&r, both, sizeof(r));
  return r;
}

template <int BM, int BN, int WAVES_M, int EPI>
__device__ __forceinline__ void wgrad_tile(const WgradArgs& a, const uint16_t* __restrict__ X,
                                           const uint16_t* __restrict__ dY,
                                           float* __restrict__ W, float* __restrict__ S1,
                                           float* __restrict__ S2, int64_t T, int tile_m,
                                           int tile_n, uint16_t* smem) {
  constexpr int WAVES_N = kWaves / WAVES_M;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LDX = lds_stride(BM), LDY = lds_stride(BN);
  constexpr int STAGE = kBK * (LDX + LDY);
  constexpr int XCH = kBK * BM / 8, YCH = kBK * BN / 8;  // 16-byte chunks per stage
  constexpr int XPT = XCH / kThreads, YPT = YCH / kThreads;
  static_assert(XCH % kThreads == 0 && YCH % kThreads == 0, "stage not evenly split");
  static_assert(TM >= 1 && TN >= 1, "wave tile smaller than one MFMA block");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int d_in = a.d_in, d_out = a.d_out;
  const int i0 = tile_m * BM, o0 = tile_n * BN;

  // Per-thread global chunks: chunk c = tid + kThreads * q covers row
  // c / (W/8) of the stage and features (c % (W/8)) * 8 .. + 7.
  int x_row[XPT], x_col[XPT], y_row[YPT], y_col[YPT];
  bool x_ok[XPT], y_ok[YPT];
#pragma unroll
  for (int q = 0; q < XPT; ++q) {
    const int c = tid + kThreads * q;
    x_row[q] = c / (BM / 8);
    x_col[q] = (c % (BM / 8)) * 8;
    x_ok[q] = i0 + x_col[q] < d_in;
  }
#pragma unroll
  for (int q = 0; q < YPT; ++q) {
    const int c = tid + kThreads * q;
    y_row[q] = c / (BN / 8);
    y_col[q] = (c % (BN / 8)) * 8;
    y_ok[q] = o0 + y_col[q] < d_out;
  }

  u32x4_t xr[XPT], yr[YPT];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int64_t k = k0 + x_row[q];
      xr[q] = (u32x4_t){0u, 0u, 0u, 0u};
      if (x_ok[q] && k < T)
        xr[q] = *reinterpret_cast<const u32x4_t*>(X + k * d_in + i0 + x_col[q]);
    }
#pragma unroll
    for (int q = 0; q < YPT; ++q) {
      const int64_t k = k0 + y_row[q];
      yr[q] = (u32x4_t){0u, 0u, 0u, 0u};
      if (y_ok[q] && k < T)
        yr[q] = *reinterpret_cast<const u32x4_t*>(dY + k * d_out + o0 + y_col[q]);
    }
  };
  auto sstore = [&](int buf) {
    uint16_t* sx = smem + buf * STAGE;
    uint16_t* sy = sx + kBK * LDX;
#pragma unroll
    for (int q = 0; q < XPT; ++q)
      *reinterpret_cast<u32x4_t*>(sx + x_row[q] * LDX + x_col[q]) = xr[q];
#pragma unroll
    for (int q = 0; q < YPT; ++q)
      *reinterpret_cast<u32x4_t*>(sy + y_row[q] * LDY + y_col[q]) = yr[q];
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;

  auto compute = [&](int buf) {
    const uint16_t* sx = smem + buf * STAGE;
    const uint16_t* sy = sx + kBK * LDX;
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8_t af[TM], bfrag[TN];
#pragma unroll
      for (int m = 0; m < TM; ++m) af[m] = load_operand<LDX>(sx, kk, wm * WM + m * 32, lane);
#pragma unroll
      for (int n = 0; n < TN; ++n) bfrag[n] = load_operand<LDY>(sy, kk, wn * WN + n * 32, lane);
#pragma unroll
      for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[m], bfrag[n], acc[m][n], 0, 0, 0);
    }
  };

  const int64_t nk = (T + kBK - 1) / kBK;
  if (nk > 0) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int cur = int(kt & 1);
      const bool more = kt + 1 < nk;
      if (more) gload((kt + 1) * kBK);
      compute(cur);
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane owns rows i = .. + 8q + 4 (lane / 32) + 0..3 of column o.
  const int o_lane = lane & 31, i_lane = 4 * (lane >> 5);
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    const int o = o0 + wn * WN + n * 32 + o_lane;
    if (o >= d_out) continue;
#pragma unroll
    for (int m = 0; m < TM; ++m) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = i0 + wm * WM + m * 32 + 8 * q + i_lane;
        if (i >= d_in) continue;
        const int64_t off = int64_t(o) * d_in + i;
        const f32x4_t g = {acc[m][n][4 * q + 0], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                           acc[m][n][4 * q + 3]};
        if constexpr (EPI == EPI_GRAD) {
          *reinterpret_cast<f32x4_t*>(W + off) = g;
        } else if constexpr (EPI == EPI_ADAMW) {
          f32x4_t w = *reinterpret_cast<const f32x4_t*>(W + off);
          f32x4_t mm = *reinterpret_cast<const f32x4_t*>(S1 + off);
          f32x4_t vv = *reinterpret_cast<const f32x4_t*>(S2 + off);
          adamw_vec4(g, w, mm, vv, a.adam);
          *reinterpret_cast<f32x4_t*>(W + off) = w;
          *reinterpret_cast<f32x4_t*>(S1 + off) = mm;
          *reinterpret_cast<f32x4_t*>(S2 + off) = vv;
        } else {
          f32x4_t w = *reinterpret_cast<const f32x4_t*>(W + off);
          f32x4_t b = *reinterpret_cast<const f32x4_t*>(S1 + off);
          sgdm_vec4(g, w, b, a.sgd);
          *reinterpret_cast<f32x4_t*>(W + off) = w;
          *reinterpret_cast<f32x4_t*>(S1 + off) = b;
        }
      }
    }
  }
}

template <int BM, int BN, int WAVES_M, int EPI>
__global__ __launch_bounds__(kThreads) void wgrad_dense_kernel(WgradArgs a) {
  constexpr int STAGE = kBK * (lds_stride(BM) + lds_stride(BN));
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  int e, tm, tn;
  map_tile(blockIdx.x, a.num_tiles, a.tiles_m, a.tiles_n, a.group_m, e, tm, tn);
  wgrad_tile<BM, BN, WAVES_M, EPI>(a, a.X, a.dY, a.W, a.S1, a.S2, a.T, tm, tn, smem);
}

template <int BM, int BN, int WAVES_M, int EPI>
__global__ __launch_bounds__(kThreads) void wgrad_grouped_kernel(WgradArgs a, GroupTable gt) {
  constexpr int STAGE = kBK * (lds_stride(BM) + lds_stride(BN));
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  int e, tm, tn;
  map_tile(blockIdx.x, a.num_tiles, a.tiles_m, a.tiles_n, a.group_m, e, tm, tn);
  const int64_t r0 = gt.off[e], r1 = gt.off[e + 1];
  const int64_t state = int64_t(e) * a.d_out * a.d_in;
  wgrad_tile<BM, BN, WAVES_M, EPI>(a, a.X + r0 * a.d_in, a.dY + r0 * a.d_out, a.W + state,
                                   a.S1 + state, a.S2 + state, r1 - r0, tm, tn, smem);
}

// Unfused elementwise optimizers (the HBM-materialising comparison path).
__global__ __launch_bounds__(256) void adamw_elementwise_kernel(const float* __restrict__ g,
                                                                float* __restrict__ W,
                                                                float* __restrict__ m,
                                                                float* __restrict__ v, int64_t n,
                                                                AdamWConsts c) {
  const int64_t n4 = n >> 2;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n4; k += stride) {
    const f32x4_t gg = reinterpret_cast<const f32x4_t*>(g)[k];
    f32x4_t w = reinterpret_cast<const f32x4_t*>(W)[k];
    f32x4_t mm = reinterpret_cast<const f32x4_t*>(m)[k];
    f32x4_t vv = reinterpret_cast<const f32x4_t*>(v)[k];
    adamw_vec4(gg, w, mm, vv, c);
    reinterpret_cast<f32x4_t*>(W)[k] = w;
    reinterpret_cast<f32x4_t*>(m)[k] = mm;
    reinterpret_cast<f32x4_t*>(v)[k] = vv;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t k = (n4 << 2) + threadIdx.x;
    float w = W[k], mm = m[k], vv = v[k];
    adamw_elem(g[k], w, mm, vv, c);
    W[k] = w;
    m[k] = mm;
    v[k] = vv;
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
