// Weight gradient from fp8 inputs for gfx950: X and dY as OCP fp8 codes (E4M3
// or E5M2) with one float scale per tensor, g = s_x s_dy sum_t dY[t, o] X[t, i]
// accumulated in float32 by v_mfma_scale_f32_32x32x64_f8f6f4 (unit block
// scales), then the same epilogues as the bf16 kernels with the scale product
// applied to the accumulator once. FORGE assessment, "Math verified, not
// asserted", P6: the paper's fp8 row is 44x worse than its baseline; this
// path makes that trade measurable at twice the bf16 matrix rate.
//
// Mainloop: stages of 64 tokens (one MFMA k-step), [token][feature] byte rows
// in LDS, loaded straight from memory as in the bf16 kernel. An MFMA operand
// is 32 consecutive tokens of one feature per lane, gathered with four LDS
// transpose reads (ds_read_b64_tr_b8): within a group of 16 lanes, lanes 2r
// and 2r + 1 supply the two 8-byte halves of a 16-byte run of row r, and lane
// j receives byte j of each of the 8 rows. Each 32-lane half of such a read
// covers 8 token rows x 32 contiguous bytes; the 16-byte chunk c of row r is
// stored at c ^ 2 ((r >> k) & (RB / 32 - 1)), RB the row length in bytes and
// 2^k = 256 / RB, which puts those 8 runs on 8 distinct 32-byte bank slots.
//
// Ring of 4 slots, loads issued 4 stages ahead into the slot freed by the
// previous barrier; per stage: issue stage s + 4, read the operands of stage
// s + 1, MFMAs on stage s, then one barrier that also waits for stage s + 2.
// Tokens enter each element in ascending 64-token chunks, so the result is
// bitwise the same for every tiling.
#pragma once

#include "wgrad_kernels.hpp"

namespace forge {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// MFMA operand format codes (the instruction's cbsz / blgp fields).
enum Fp8Fmt : int { FP8_E4M3 = 0, FP8_E5M2 = 1 };

__device__ __forceinline__ i32x2_t lds_read_tr8(const char* p) {
  typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(p));
}

// Swizzle term of the fp8 LDS rows (see the file comment).
template <int RB>
__host__ __device__ constexpr int fp8_swz(int r) {
  return RB >= 256 ? 2 * (r & 7) : 2 * ((r >> 1) & 3);
}

template <class C, int EPI, int FA, int FB>
__device__ __forceinline__ void wgrad_tile_fp8(const WgradArgs& a, const uint8_t* __restrict__ X,
                                               const uint8_t* __restrict__ dY,
                                               float* __restrict__ W, float* __restrict__ S1,
                                               float* __restrict__ S2, int64_t T, int tile_m,
                                               int tile_n, const Slots& sl) {
  constexpr int BM = C::BM, BN = C::BN, TM = C::TM, TN = C::TN;
  constexpr int BK = 64;                                // tokens per stage
  constexpr int RBX = BM, RBY = BN;                     // bytes per token row
  static_assert(RBX == 128 || RBX == 256, "fp8 rows of 128 or 256 bytes");
  static_assert(RBY == 128 || RBY == 256, "fp8 rows of 128 or 256 bytes");
  constexpr int QX = BK * RBX / 1024, QY = BK * RBY / 1024;   // 1 KB loads per stage
  constexpr int NQW = (QX + QY) / C::WAVES;
  static_assert((QX + QY) % C::WAVES == 0, "stage loads split evenly over the waves");
  static_assert(BK * (RBX + RBY) <= C::STAGE * 2, "stage exceeds a slot");
  constexpr int L = 4;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int d_in = a.d_in, d_out = a.d_out;
  const int i0 = tile_m * BM, o0 = tile_n * BN;

  // Stage loads: instruction q covers 1024 / RB rows of X (q < QX) or dY;
  // lane t fills row q * rows + t / (RB / 16), physical chunk t % (RB / 16).
  uint32_t voff[NQW];
  int soff[NQW];
#pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = wave * NQW + i;
    const bool isx = q < QX;
    const int rb = isx ? RBX : RBY, cpr = rb / 16, rows = 1024 / rb;
    const int dim = isx ? d_in : d_out, c0 = isx ? i0 : o0;
    const int row0 = (isx ? q : q - QX) * rows;
    const int lrow = lane / cpr, p = lane % cpr;
    const int r = row0 + lrow;
    const int ch = p ^ (isx ? fp8_swz<RBX>(r) : fp8_swz<RBY>(r));
    voff[i] = c0 + 16 * ch < dim ? uint32_t(lrow * dim + 16 * ch) : kOOB;
    soff[i] = row0 * dim;
  }
  const int nfull = int(T / BK), tail = int(T - int64_t(nfull) * BK);
  int g_stage = 0;
  const uint8_t* gx = X + i0;
  const uint8_t* gy = dY + o0;
  auto stage_bytes = [&](int dim, int c0) {
    const int rows = g_stage < nfull ? BK : (g_stage == nfull ? tail : 0);
    const int n = rows * dim - c0;
    return n > 0 ? uint32_t(n) : 0u;
  };
  auto load_stage = [&](uint16_t* slot) {
    const __amdgpu_buffer_rsrc_t rx = window32(gx, stage_bytes(d_in, i0));
    const __amdgpu_buffer_rsrc_t ry = window32(gy, stage_bytes(d_out, o0));
    gx += BK * d_in;
    gy += BK * d_out;
    ++g_stage;
#pragma unroll
    for (int i = 0; i < NQW; ++i) {
      const int q = wave * NQW + i;
      load16_to_lds(q < QX ? rx : ry, slot + q * 512, voff[i], soff[i]);
    }
  };

  // Operand read addresses: lane l takes feature 32 b + 16 ((l / 16) % 2) +
  // (l % 16) of its 32-feature block b and tokens 32 (l / 32) + 8 q .. + 7 in
  // read q; as a transpose-read address it supplies row 32 (l / 32) + (l % 16) / 2
  // (+ 8 q), bytes 8 (l % 2) of chunk 2 b + (l / 16) % 2.
  const int hg = lane >> 5, G2 = (lane >> 4) & 1, jl = lane & 15;
  const int rsub = 32 * hg + (jl >> 1);
  uint32_t fa[TM], fb[TN];
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    const int c = ((wm * C::WM + m * 32) >> 4) + G2;
    fa[m] = uint32_t(rsub * RBX + ((c ^ fp8_swz<RBX>(rsub)) << 4) + 8 * (jl & 1));
  }
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    const int c = ((wn * C::WN + n * 32) >> 4) + G2;
    fb[n] = uint32_t(BK * RBX + rsub * RBY + ((c ^ fp8_swz<RBY>(rsub)) << 4) + 8 * (jl & 1));
  }
  auto operand = [](const uint16_t* slot, uint32_t off, int rb) {
    const char* b = reinterpret_cast<const char*>(slot) + off;
    const i32x2_t r0 = lds_read_tr8(b);
    const i32x2_t r1 = lds_read_tr8(b + 8 * rb);
    const i32x2_t r2 = lds_read_tr8(b + 16 * rb);
    const i32x2_t r3 = lds_read_tr8(b + 24 * rb);
    const i32x8_t v = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
    return v;
  };
  i32x8_t frag[2][TM + TN];
  auto read_frags = [&](int f, const uint16_t* slot) {
#pragma unroll
    for (int m = 0; m < TM; ++m) frag[f][m] = operand(slot, fa[m], RBX);
#pragma unroll
    for (int n = 0; n < TN; ++n) frag[f][TM + n] = operand(slot, fb[n], RBY);
  };
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int m = 0; m < TM; ++m)
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[m][n][r] = 0.0f;
  auto mfmas = [&](int f) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int n = 0; n < TN; ++n)
        acc[m][n] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            frag[f][m], frag[f][TM + n], acc[m][n], FA, FB, 0, 127, 0, 127);
  };
  // Three transpose reads per MFMA: the next stage's operands are all
  // requested within the first ~2/3 of the stage's MFMAs, so they have landed
  // when the barrier waits for them.
  constexpr int NREAD = 4 * (TM + TN);
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
      if (3 * i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);      // DS read
      if (i < NQW) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);           // VMEM read
    }
  };
  constexpr int kWaitStage = waitcnt_imm(2 * NQW, 0);
  constexpr int kWaitFirst = waitcnt_imm(2 * NQW, 15);
#define FORGE_FP8_BARRIER(IMM)                \
  do {                                        \
    __builtin_amdgcn_sched_barrier(0);        \
    __builtin_amdgcn_s_waitcnt(IMM);          \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)
  // Stage s: slot `cur` holds stage s (its operands are already in frag[f]);
  // it takes stage s + 4, while stage s + 1's operands are read from `nxt`.
  auto stage = [&](uint16_t* cur, uint16_t* nxt, int f) {
    load_stage(cur);
    read_frags(f ^ 1, nxt);
    mfmas(f);
    interleave();
    FORGE_FP8_BARRIER(kWaitStage);
  };
  const int nk = int((T + BK - 1) / BK);
  if (nk > 0) {
    load_stage(sl.s0);
    load_stage(sl.s1);
    load_stage(sl.s2);
    load_stage(sl.s3);
    FORGE_FP8_BARRIER(kWaitFirst);              // stages 0 and 1 have landed
    read_frags(0, sl.s0);
    FORGE_FP8_BARRIER(waitcnt_imm(2 * NQW, 0));   // every wave is done reading slot 0
    // Whole rounds of 4 stages (static slots); stages past T load zeros,
    // which add exactly +0 to the accumulators.
    const int rounds = (nk + L - 1) / L;
    for (int r = 0; r < rounds; ++r) {
      stage(sl.s0, sl.s1, 0);
      stage(sl.s1, sl.s2, 1);
      stage(sl.s2, sl.s3, 0);
      stage(sl.s3, sl.s0, 1);
    }
  }
#undef FORGE_FP8_BARRIER
  uint16_t* ep = wave == 0 ? sl.s0 : wave == 1 ? sl.s1 : wave == 2 ? sl.s2 : sl.s3;
  epilogue<C, EPI>(a, acc, W, S1, S2, i0, o0, wm, wn, lane, reinterpret_cast<float*>(ep));
}

template <class C, int EPI, int FA, int FB>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void wgrad_fp8_kernel(WgradArgs a) {
  FORGE_DECLARE_SLOTS(C::STAGE);
  int e, tm, tn;
  map_tile(blockIdx.x, a.num_tiles, a.tiles_m, a.tiles_n, a.group_m, e, tm, tn);
  wgrad_tile_fp8<C, EPI, FA, FB>(a, reinterpret_cast<const uint8_t*>(a.X),
                                 reinterpret_cast<const uint8_t*>(a.dY), a.W, a.S1, a.S2, a.T,
                                 tm, tn, ring);
}

// The persistent schedule of the bf16 kernel, with the fp8 mainloop.
template <class CF, class CH, int EPI, int FA, int FB>
__global__ __launch_bounds__(CF::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void wgrad_fp8_persistent_kernel(WgradArgs a) {
  static_assert(CF::THREADS == CH::THREADS && CF::BM == CH::BM && CF::BN == 2 * CH::BN,
                "half tiles must split the full tile's columns");
  FORGE_DECLARE_SLOTS(CF::STAGE);
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3, nw = gridDim.x >> 3;
  const int per = a.num_tiles >> 3, rem = a.num_tiles & 7;
  const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  const int R = per + (xcd < rem ? 1 : 0);
  const int phase = schedule_phase(xcd, R, nw);
  const uint8_t* X = reinterpret_cast<const uint8_t*>(a.X);
  const uint8_t* dY = reinterpret_cast<const uint8_t*>(a.dY);
  for (int k = 0;; ++k) {
    int tile, half;
    if (!schedule_item(k, j, nw, R, phase, tile, half)) break;
    int tm, tn;
    grouped_walk(start + tile, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    if (half < 0)
      wgrad_tile_fp8<CF, EPI, FA, FB>(a, X, dY, a.W, a.S1, a.S2, a.T, tm, tn, ring);
    else
      wgrad_tile_fp8<CH, EPI, FA, FB>(a, X, dY, a.W, a.S1, a.S2, a.T, tm, 2 * tn + half, ring);
    __syncthreads();
  }
}

}  // namespace forge
