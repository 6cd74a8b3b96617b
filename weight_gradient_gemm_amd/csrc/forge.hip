// Host side of the forge C ABI: validation, per-step scalars, tile choice and
// kernel launch on the caller's stream. Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

#include "forge.h"
#include "dgrad_kernels.hpp"
#include "fp8_kernels.hpp"
#include "validate.hpp"
#include "wgrad_kernels.hpp"

namespace forge {
namespace {

constexpr int kMaxDevices = 64;
// Per-device verdict of the architecture check: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_arch_ok[kMaxDevices];
// Per-device compute-unit count (0 unknown).
std::atomic<int> g_cu_count[kMaxDevices];

forge_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FORGE_ERR_DEVICE;
  }
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FORGE_ERR_DEVICE;
    }
    v = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_cu_count[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? FORGE_OK : FORGE_ERR_DEVICE;
}

// Workgroups of a persistent launch on the current device: one per compute
// unit, rounded down to whole pairs per XCD (8 XCDs), or 0 if too few.
int persistent_grid() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int cus = g_cu_count[dev].load(std::memory_order_relaxed);
  return (cus / 16) * 16;
}

AdamWConsts make_adamw(const forge_adamw_params& p) {
  const double t = double(p.step);
  const double bc1 = 1.0 - std::pow(p.beta1, t);
  const double bc2 = 1.0 - std::pow(p.beta2, t);
  AdamWConsts c;
  c.beta1 = float(p.beta1);
  c.one_m_beta1 = float(1.0 - p.beta1);
  c.beta2 = float(p.beta2);
  c.one_m_beta2 = float(1.0 - p.beta2);
  c.decay = float(1.0 - p.lr * p.weight_decay);
  c.step_size = float(p.lr / bc1);
  c.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
  c.eps = float(p.eps);
  return c;
}

SgdmConsts make_sgdm(const forge_sgdm_params& p) {
  SgdmConsts c;
  c.momentum = float(p.momentum);
  c.weight_decay = float(p.weight_decay);
  c.lr = float(p.lr);
  return c;
}

struct TileShape {
  int bm, bn;
};

TileShape shape_of(forge_tile t) {
  switch (t) {
    case FORGE_TILE_128x128: return {128, 128};
    case FORGE_TILE_256x256:
    case FORGE_TILE_PERSISTENT: return {256, 256};
    case FORGE_TILE_256x128:
    default: return {256, 128};
  }
}

int64_t count_tiles(int64_t d_in, int64_t d_out, TileShape s) {
  return ((d_in + s.bm - 1) / s.bm) * ((d_out + s.bn - 1) / s.bn);
}

// Default tile: the one with the best estimated throughput for the shape. A
// tile's share of the matrix-core rate (measured on gfx950 for the
// Llama-3-8B MLP-down contraction, relative to 256x256) is scaled by how well
// its tiles fill whole waves of workgroups over the 256 compute units.
// Makespan, in full-tile times, of the persistent schedule for `tiles` 256x256
// tiles on `grid` workgroups (odd XCDs half a tile behind). A half tile costs
// 0.6 of a full one (it runs at ~85% of the full tile's rate).
double persistent_makespan(int64_t tiles, int grid) {
  const int nw = grid / 8;
  double worst = 0.0;
  for (int xcd = 0; xcd < 8; ++xcd) {
    const int64_t per = tiles / 8, rem = tiles % 8;
    const int R = int(per + (xcd < rem ? 1 : 0));
    const int phase = schedule_phase(xcd, R, nw);
    for (int j = 0; j < nw; ++j) {
      double t = 0.0;
      int tile, half;
      for (int k = 0; schedule_item(k, j, nw, R, phase, tile, half); ++k) t += half < 0 ? 1.0 : 0.6;
      worst = std::max(worst, t);
    }
  }
  return worst;
}

forge_tile resolve_tile(forge_tile t, int64_t d_in, int64_t d_out, int64_t experts,
                        bool allow_persistent = true) {
  if ((experts > 1 || !allow_persistent) && t == FORGE_TILE_PERSISTENT) return FORGE_TILE_256x256;
  if (t != FORGE_TILE_DEFAULT) return t;
  struct Cand {
    forge_tile id;
    double rate;     // relative per-tile throughput
    int64_t slots;   // concurrent workgroups on 256 CUs
  };
  const Cand cands[] = {{FORGE_TILE_256x256, 1.00, 256},
                        {FORGE_TILE_256x128, 0.85, 256},
                        {FORGE_TILE_128x128, 0.80, 512}};
  forge_tile best = FORGE_TILE_256x128;
  double best_score = -1.0;
  for (const Cand& c : cands) {
    const int64_t tiles = experts * count_tiles(d_in, d_out, shape_of(c.id));
    const int64_t rounds = (tiles + c.slots - 1) / c.slots;
    const double fill = double(tiles) / double(rounds * c.slots);
    const double score = c.rate * fill;
    if (score > best_score + 1e-9) {
      best_score = score;
      best = c.id;
    }
  }
  // The persistent schedule: the 256x256 tile rate, balanced to half tiles.
  const int grid = persistent_grid();
  const int64_t tiles = count_tiles(d_in, d_out, shape_of(FORGE_TILE_256x256));
  if (allow_persistent && experts == 1 && grid > 0 && tiles >= grid) {
    const double score = double(tiles) / (double(grid) * persistent_makespan(tiles, grid));
    if (score > best_score + 1e-9) best = FORGE_TILE_PERSISTENT;
  }
  return best;
}

forge_status launch_status() {
  return hipGetLastError() == hipSuccess ? FORGE_OK : FORGE_ERR_LAUNCH;
}

// Tile configurations behind the public tile ids.
using Cfg256x256 = TileCfg<256, 256, 2, 2, 32, 1>;
using Cfg256x128 = TileCfg<256, 128, 2, 2, 32, 1>;
using Cfg128x128 = TileCfg<128, 128, 2, 2, 32, 2>;

template <class C>
void set_grid(WgradArgs& a, int64_t experts) {
  a.tiles_m = int32_t((a.d_in + C::BM - 1) / C::BM);
  a.tiles_n = int32_t((a.d_out + C::BN - 1) / C::BN);
  a.num_tiles = int32_t(a.tiles_m * a.tiles_n * experts);
  a.group_m = 4;
}

template <class C, int EPI>
forge_status launch_dense_t(WgradArgs a, hipStream_t s) {
  set_grid<C>(a, 1);
  hipLaunchKernelGGL((wgrad_dense_kernel<C, EPI>), dim3(a.num_tiles), dim3(C::THREADS), 0, s, a);
  return launch_status();
}

template <int EPI>
forge_status launch_persistent(WgradArgs a, hipStream_t s) {
  set_grid<Cfg256x256>(a, 1);
  const int grid = persistent_grid();
  if (grid <= 0) return launch_dense_t<Cfg256x256, EPI>(a, s);
  hipLaunchKernelGGL((wgrad_persistent_kernel<Cfg256x256, Cfg256x128, EPI>), dim3(grid),
                     dim3(Cfg256x256::THREADS), 0, s, a);
  return launch_status();
}

template <int EPI>
forge_status launch_dense(const WgradArgs& a, forge_tile tile, hipStream_t s) {
  switch (tile) {
    case FORGE_TILE_128x128: return launch_dense_t<Cfg128x128, EPI>(a, s);
    case FORGE_TILE_256x128: return launch_dense_t<Cfg256x128, EPI>(a, s);
    case FORGE_TILE_256x256: return launch_dense_t<Cfg256x256, EPI>(a, s);
    case FORGE_TILE_PERSISTENT: return launch_persistent<EPI>(a, s);
    default: return FORGE_ERR_TILE;
  }
}

// AdamW epilogue variant: the exact square root when eps = 0.
template <template <int> class F, int BASE = EPI_ADAMW, class... Args>
forge_status with_adamw_epi(const forge_adamw_params& p, Args&&... args) {
  return p.eps > 0.0 ? F<BASE>::run(args...) : F<BASE | EPI_EXACT_SQRT>::run(args...);
}

template <int EPI>
struct DenseLaunch {
  static forge_status run(const WgradArgs& a, forge_tile tile, hipStream_t s) {
    return launch_dense<EPI>(a, tile, s);
  }
};

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

WgradArgs base_args(const void* X, const void* dY, float* W, float* S1, float* S2, int64_t T,
                    int64_t d_in, int64_t d_out) {
  WgradArgs a;
  std::memset(&a, 0, sizeof(a));
  a.X = static_cast<const uint16_t*>(X);
  a.dY = static_cast<const uint16_t*>(dY);
  a.W = W;
  a.S1 = S1;
  a.S2 = S2;
  a.T = T;
  a.d_in = int32_t(d_in);
  a.d_out = int32_t(d_out);
  return a;
}

// Tile counts must fit the kernels' 32-bit block indices.
bool grid_fits(int64_t d_in, int64_t d_out, forge_tile tile, int64_t experts) {
  return experts * count_tiles(d_in, d_out, shape_of(tile)) < (int64_t(1) << 31);
}

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
  tile = resolve_tile(tile, d_in, d_out, E);
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
  return with_adamw_epi<DenseLaunch>(*p, a, tile, st);
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
  return launch_dense<EPI_SGDM>(a, tile, st);
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
