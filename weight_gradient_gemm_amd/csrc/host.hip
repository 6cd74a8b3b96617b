// Host-side helpers of the forge C ABI (no kernels): the device check, the
// per-step optimizer scalars and the tile choice. Nothing here allocates
// device memory.
#include "host.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>

namespace forge {
namespace {

constexpr int kMaxDevices = 64;
// Per-device verdict of the architecture check: 0 unknown, 1 gfx950, -1 other.
std::atomic<int> g_arch_ok[kMaxDevices];
// Per-device compute-unit count (0 unknown).
std::atomic<int> g_cu_count[kMaxDevices];

}  // namespace

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

// Default tile: the one with the best estimated throughput for the shape. A
// tile's share of the matrix-core rate (measured on gfx950 for the
// Llama-3-8B MLP-down contraction, relative to 256x256) is scaled by how well
// its tiles fill whole waves of workgroups over the 256 compute units; the
// persistent schedule is scored by its makespan.
forge_tile resolve_tile(forge_tile t, int64_t d_in, int64_t d_out, int64_t experts,
                        bool allow_persistent) {
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

}  // namespace forge
