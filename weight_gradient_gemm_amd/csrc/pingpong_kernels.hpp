// Two-group ("ping-pong") persistent weight-gradient kernel for gfx950.
//
// The fused step's optimizer epilogue streams 24 bytes of state per weight
// through the compute unit and leaves the matrix cores idle while it runs
// (FORGE assessment, introduction: the step runs per tile, in the epilogue of
// the weight-gradient GEMM). Here one workgroup per compute unit holds two
// groups of four waves. Each group walks its own list of BM x BN tiles
// (mainloop over all tokens, then the epilogue); the second group starts
// about one epilogue later than the first, so while one group streams its
// tile's W, m, v the other group's mainloop keeps the matrix cores busy.
//
// Pairing: the groups share no data, only the workgroup barrier. Every
// mainloop stage and every epilogue piece ends with one s_barrier, and both
// groups execute exactly the same number of barriers (the count is a pure
// function of the schedule; the group with less work pads with bare
// barriers). The i-th barrier of one group therefore meets the i-th barrier
// of the other, the groups advance in lockstep ticks, and no wave ever spins
// on memory. A tick in which both groups run mainloop stages issues both
// groups' MFMAs on each SIMD (two waves per SIMD); a tick in which one group
// runs an epilogue piece hands the matrix cores to the other group.
//
// Accumulation order: the same as every other kernel of the library (tokens
// in ascending 16-token chunks through one accumulator, zero-filled tails), so
// results are bitwise those of any other tiling.
#pragma once

#include "wgrad_kernels.hpp"

namespace forge {

// L ring slots of one group, each its own __shared__ array (so the compiler
// can tell the slots apart when it places waits for direct-to-LDS loads).
template <int L>
struct Ring {
  uint16_t* s[L];
};

// Workgroup barriers of the two-group kernel. With an explicit wait first
// (IMM as for s_waitcnt), or bare: a wave's own memory operations stay in
// flight across a bare barrier; only the wave itself ever waits for them.
#define FORGE_PP_BARRIER_WAIT(IMM)            \
  do {                                        \
    __builtin_amdgcn_sched_barrier(0);        \
    __builtin_amdgcn_s_waitcnt(IMM);          \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)
#define FORGE_PP_BARRIER()                    \
  do {                                        \
    __builtin_amdgcn_sched_barrier(0);        \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)

// Barriers of one mainloop over T tokens with a ring of L slots: one after
// the first L stage loads, then one per stage, in whole rounds of L stages.
__host__ __device__ constexpr int pp_mainloop_barriers(int64_t T, int BK, int L) {
  return T > 0 ? int(1 + (((T + BK - 1) / BK + L - 1) / L) * L) : 0;
}

// Mainloop of one tile: acc[i, o] = sum_t X[t, i] dY[t, o] over all T tokens.
// The same staging, swizzle, transpose reads and MFMA order as wgrad_tile,
// with a ring of L slots (loads issued L - 1 stages ahead) and exactly
// pp_mainloop_barriers(T, BK, L) workgroup barriers. `wave` is the wave's
// index within its group.
template <class C, int L>
__device__ __forceinline__ void mainloop_ring(const WgradArgs& a, const uint16_t* __restrict__ X,
                                              const uint16_t* __restrict__ dY, int64_t T,
                                              int tile_m, int tile_n, const Ring<L>& ring,
                                              int wave, int lane,
                                              f32x16_t (&acc)[C::TM][C::TN]) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TM = C::TM, TN = C::TN;
  constexpr int RBX = BM * 2, RBY = BN * 2;             // bytes per token row
  constexpr int CPX = BM / 8, CPY = BN / 8;             // 16-byte chunks per row
  constexpr int QX = BK * RBX / 1024, QY = BK * RBY / 1024;
  constexpr int NQW = (QX + QY) / C::WAVES;             // 1 KB loads per wave per stage
  static_assert(L >= 2, "at least two ring slots");
  static_assert((QX + QY) % C::WAVES == 0, "stage loads split evenly over the waves");
  static_assert((L - 1) * NQW <= 63, "loads in flight exceed the vector-memory counter");

  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int d_in = a.d_in, d_out = a.d_out;
  const int i0 = tile_m * BM, o0 = tile_n * BN;

  uint32_t voff[NQW];
  int soff[NQW];
#pragma unroll
  for (int i = 0; i < NQW; ++i) {
    const int q = wave * NQW + i;
    const bool isx = q < QX;
    const int sh = isx ? ilog2(CPX) : ilog2(CPY);
    const int dim = isx ? d_in : d_out, c0 = isx ? i0 : o0;
    const int row0 = (isx ? q : q - QX) << (6 - sh);
    const int lrow = lane >> sh, p = lane & ((1 << sh) - 1);
    const int ch = p ^ (4 * ((row0 + lrow) & 3));
    voff[i] = c0 + 8 * ch < dim ? uint32_t(lrow * dim + 8 * ch) * 2u : kOOB;
    soff[i] = row0 * dim * 2;
  }
  const int nfull = int(T / BK), tail = int(T - int64_t(nfull) * BK);
  int g_stage = 0;
  const uint16_t* gx = X + i0;
  const uint16_t* gy = dY + o0;
  auto stage_bytes = [&](int dim, int c0) {
    const int rows = g_stage < nfull ? BK : (g_stage == nfull ? tail : 0);
    const int n = rows * dim - c0;
    return n > 0 ? uint32_t(n) * 2u : 0u;
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

  const int g = lane >> 4, j = lane & 15;
  const int rsub = 8 * (g >> 1) + (j >> 2);
  uint32_t fa[TM], fb[TN];
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    const int blk = (wm * C::WM + m * 32) >> 5;
    const int ch = (4 * blk + 2 * (g & 1) + ((j & 3) >> 1)) ^ (4 * (j >> 2));
    fa[m] = uint32_t(rsub * RBX + ch * 16 + (j & 1) * 8);
  }
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    const int blk = (wn * C::WN + n * 32) >> 5;
    const int ch = (4 * blk + 2 * (g & 1) + ((j & 3) >> 1)) ^ (4 * (j >> 2));
    fb[n] = uint32_t(BK * RBX + rsub * RBY + ch * 16 + (j & 1) * 8);
  }
  auto operand = [](const uint16_t* slot, uint32_t off, int rb) {
    const char* b = reinterpret_cast<const char*>(slot) + off;
    const i16x4_t lo = lds_read_tr16(b);
    const i16x4_t hi = lds_read_tr16(b + 4 * rb);
    const i16x4_t both[2] = {lo, hi};
    bf16x8_t r;
    __builtin_memcpy(&r, both, sizeof(r));
    return r;
  };
  bf16x8_t frag[2][TM + TN];
  auto read_frags = [&](int f, const uint16_t* slot, int kk) {
#pragma unroll
    for (int m = 0; m < TM; ++m) frag[f][m] = operand(slot, fa[m] + kk * 16 * RBX, RBX);
#pragma unroll
    for (int n = 0; n < TN; ++n) frag[f][TM + n] = operand(slot, fb[n] + kk * 16 * RBY, RBY);
  };
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
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[f][m], frag[f][TM + n],
                                                            acc[m][n], 0, 0, 0);
  };
  constexpr int NREAD = 2 * (TM + TN);
  auto interleave = [&](int loads) {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
      if (i < NREAD / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // DS read
      if (i < loads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // VMEM read
    }
  };
  // Per stage s: MFMAs on chunk 0 while chunk 1's operands are read; wait for
  // this wave's reads (slot s % L is then free) and its loads of stage s + 1;
  // barrier; load stage s + L into the freed slot, MFMAs on chunk 1 while
  // stage s + 1's chunk 0 operands are read.
  constexpr int kWaitMid = waitcnt_imm((L - 2) * NQW, 0);
  constexpr int kWaitFirst = waitcnt_imm((L - 1) * NQW, 15);
  auto stage = [&](uint16_t* cur, uint16_t* nxt) {
    read_frags(1, cur, 1);
    mfmas(0);
    interleave(0);
    FORGE_PP_BARRIER_WAIT(kWaitMid);
    load_stage(cur);
    read_frags(0, nxt, 0);
    mfmas(1);
    interleave(NQW);
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nk = int((T + BK - 1) / BK);
  if (nk > 0) {
#pragma unroll
    for (int k = 0; k < L; ++k) load_stage(ring.s[k]);
    FORGE_PP_BARRIER_WAIT(kWaitFirst);
    read_frags(0, ring.s[0], 0);
    // Whole rounds of L stages (one loop exit keeps the accumulators in
    // place); the extra stages load zeros and add exact +0.
    const int rounds = (nk + L - 1) / L;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
      for (int k = 0; k < L; ++k) stage(ring.s[k], ring.s[(k + 1) % L]);
    }
  }
}

// Barriers of one paced epilogue: one that frees the ring, P per row step,
// one that releases the staging area.
template <class C, int D, int P>
__host__ __device__ constexpr int pp_epilogue_barriers() {
  return 1 + ((C::TN * (32 / (64 / (C::WM / 4)))) + D - 1) * P + 1;
}

// Optimizer epilogue paced by the workgroup barrier. The wave's accumulators
// pass through LDS (one 32-column block at a time) to a row-major layout, as
// in epilogue(); each "row instruction" then covers 64 / (WM / 4) whole rows
// of WM contiguous floats. Row step p issues the state loads of row
// instruction p and finishes row instruction p - (D - 1) (optimizer
// arithmetic and stores), so D row instructions of loads are in flight and a
// step never waits for a load issued in the same step; each step is followed
// by P bare barriers, which spreads the state traffic over P ticks of the
// other group. Exactly pp_epilogue_barriers<C, D, P>() barriers.
template <class C, int EPI, int D, int P>
__device__ __forceinline__ void epilogue_paced(const WgradArgs& a,
                                               f32x16_t (&acc)[C::TM][C::TN],
                                               float* __restrict__ W, float* __restrict__ S1,
                                               float* __restrict__ S2, int i0, int o0, int wm,
                                               int wn, int lane, float* ep) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM;
  constexpr int LD = WM + 4;                 // floats per LDS row
  constexpr int LPR = WM / 4;                // lanes per row (4 elements each)
  constexpr int RPI = 64 / LPR;              // rows per instruction
  constexpr int NI = 32 / RPI;               // row instructions per 32-column block
  constexpr int R = TN * NI;                 // row instructions of the wave
  constexpr int OP = epi_op(EPI);
  constexpr int NS = OP == EPI_ADAMW ? 3 : (OP == EPI_SGDM ? 2 : 0);
  constexpr int ESW = epi_w_bytes(EPI), ESS = epi_state_bytes(EPI);
  constexpr int ES[4] = {ESW, ESS, ESS, 2};
  constexpr bool WB = (EPI & EPI_WB_OUT) != 0;
  static_assert(D >= 1, "at least one row instruction in flight");
  static_assert((EPI & EPI_BF16_STATE) == 0, "bf16 optimizer state uses epilogue_wide");
  static_assert(!WB || (OP != EPI_GRAD && ESW == 4), "the bf16 copy is of an updated W");
  static_assert(pp_epilogue_barriers<C, D, P>() == (R + D - 1) * P + 2, "barrier count");

  const int d_in = a.d_in, d_out = a.d_out;
  // Every wave of the group is done with the ring and its last (zero-stage)
  // loads have landed before any wave overwrites a slot with accumulators.
  FORGE_PP_BARRIER_WAIT(waitcnt_imm(0, 0));
  const int r_lane = lane / LPR, c_lane = (lane % LPR) * 4;
  const int iw0 = i0 + wm * WM;
  const bool lane_ok = iw0 + c_lane < d_in;
  const uint32_t elem = uint32_t(r_lane * d_in + c_lane);
  char* const arr[4] = {reinterpret_cast<char*>(W), reinterpret_cast<char*>(S1),
                        reinterpret_cast<char*>(S2), reinterpret_cast<char*>(a.Wb)};
  auto voff = [&](int k) { return lane_ok ? elem * uint32_t(ES[k]) : kOOB; };
  auto inst_bytes = [&](int k) { return uint32_t(RPI) * uint32_t(d_in) * uint32_t(ES[k]); };
  auto block_window = [&](int k, int n) {
    const int64_t ob = int64_t(o0) + wn * C::WN + n * 32;
    return window(arr[k] + (ob * d_in + iw0) * ES[k], ((int64_t(d_out) - ob) * d_in - iw0) * ES[k]);
  };
  // The staging area through an explicit LDS pointer, so its accesses are LDS
  // instructions (a generic access would also count on the vector-memory
  // counter and make every wait cover the state loads in flight).
  typedef __attribute__((address_space(3))) f32x4_t lds_f32x4;
  typedef __attribute__((address_space(3))) float lds_float;
  lds_float* const eps = (lds_float*)(ep);
  auto dump = [&](int n) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t g = {acc[m][n][4 * q + 0], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                           acc[m][n][4 * q + 3]};
        *(lds_f32x4*)(eps + (lane & 31) * LD + m * 32 + 8 * q + 4 * (lane >> 5)) = g;
      }
  };
  f32x4_t st[D][NS > 0 ? NS : 1];
  auto issue = [&](int r) {
    const int n = r / NI, jr = r % NI;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const __amdgpu_buffer_rsrc_t rs = block_window(k, n);
      st[r % D][k] = k == 0 ? load4<ESW>(rs, voff(k), jr * inst_bytes(k))
                            : load4<ESS>(rs, voff(k), jr * inst_bytes(k));
    }
  };
  auto finish = [&](int r) {
    const int n = r / NI, jr = r % NI;
    if (jr == 0) dump(n);   // in order after the previous block's LDS reads
    f32x4_t g = *(const lds_f32x4*)(eps + (jr * RPI + r_lane) * LD + c_lane);
    const __amdgpu_buffer_rsrc_t rw = block_window(0, n);
    const uint32_t so = jr * inst_bytes(0);
    if constexpr (OP == EPI_GRAD) {
      store4<ESW>(rw, voff(0), so, g);
    } else if constexpr (OP == EPI_ADAMW) {
      f32x4_t& w = st[r % D][0];
      adamw_vec4<(EPI & EPI_EXACT_SQRT) != 0>(g, w, st[r % D][1], st[r % D][2], a.adam);
      store4<ESW>(rw, voff(0), so, w);
      store4<ESS>(block_window(1, n), voff(1), jr * inst_bytes(1), st[r % D][1]);
      store4<ESS>(block_window(2, n), voff(2), jr * inst_bytes(2), st[r % D][2]);
      if constexpr (WB) store4<2>(block_window(3, n), voff(3), jr * inst_bytes(3), w);
    } else {
      sgdm_vec4(g, st[r % D][0], st[r % D][1], a.sgd);
      store4<ESW>(rw, voff(0), so, st[r % D][0]);
      store4<ESS>(block_window(1, n), voff(1), jr * inst_bytes(1), st[r % D][1]);
      if constexpr (WB) store4<2>(block_window(3, n), voff(3), jr * inst_bytes(3), st[r % D][0]);
    }
  };
#pragma unroll
  for (int p = 0; p < R + D - 1; ++p) {
    if (p < R) issue(p);
    if (p >= D - 1) finish(p - (D - 1));
#pragma unroll
    for (int q = 0; q < P; ++q) FORGE_PP_BARRIER();
  }
  // Every LDS read of the staging area is done before the ring is reused.
  FORGE_PP_BARRIER_WAIT(waitcnt_imm(63, 0));
}

// Schedule of the two-group kernel for one worker (compute unit). Its items
// are items j, j + nw, j + 2 nw, ... of its XCD's contiguous range of the
// grouped tile walk (CF tiles); items 2k and 2k + 1 go to groups 0 and 1. If
// the count n is odd, the last item is split along d_in into two CQ tiles,
// one per group, so both groups carry the same work. Group 1 trails group 0
// by `offset` bare barriers: one epilogue (at most one mainloop), so the
// groups' epilogues do not overlap when the mainloop is at least as long.
// Both groups derive the same barrier total from (n, per-item barriers).
struct PPSchedule {
  int n;        // items of this worker
  int offset;   // bare barriers group 1 runs before its first item
  int total;    // barriers every wave executes
};

__host__ __device__ inline PPSchedule pp_schedule(int R_xcd, int j, int nw, int main_bars,
                                                  int epi_bars, int epi_bars_split, bool split) {
  PPSchedule s;
  s.n = j < R_xcd ? (R_xcd - j + nw - 1) / nw : 0;
  const int item = main_bars + epi_bars;
  s.offset = s.n > 1 ? (main_bars < epi_bars ? main_bars : epi_bars) : 0;
  if (split) {
    s.total = s.offset + (s.n >> 1) * item + ((s.n & 1) ? main_bars + epi_bars_split : 0);
  } else {
    const int t0 = ((s.n + 1) >> 1) * item, t1 = s.offset + (s.n >> 1) * item;
    s.total = t0 > t1 ? t0 : t1;
  }
  return s;
}

// One group of the two-group persistent dense kernel. The grid is 8 * nw
// workgroups (nw per XCD); each XCD owns a contiguous range of the grouped
// walk over CF tiles.
template <class CF, class CQ, int EPI, int D, int P, bool SPLIT, int L, int G>
__device__ __forceinline__ void pingpong_group(const WgradArgs& a, const Ring<L>& ring,
                                               int wave, int lane) {
  static_assert(CF::BN == CQ::BN && CF::BM == 2 * CQ::BM, "split tiles halve d_in");
  constexpr int EB = pp_epilogue_barriers<CF, D, P>(), EQ = pp_epilogue_barriers<CQ, D, P>();
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3, nw = gridDim.x >> 3;
  const int per = a.num_tiles >> 3, rem = a.num_tiles & 7;
  const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  const int R = per + (xcd < rem ? 1 : 0);
  const int MB = pp_mainloop_barriers(a.T, CF::BK, L);
  const PPSchedule s = pp_schedule(R, j, nw, MB, EB, EQ, SPLIT);
  int bars = 0;
  if (G == 1) {
    for (int i = 0; i < s.offset; ++i) FORGE_PP_BARRIER();
    bars = s.offset;
  }
  // Staging area of this wave's epilogue: two waves per ring slot.
  char* const stage_slot = reinterpret_cast<char*>(wave < 2 ? ring.s[0] : ring.s[1]);
  const int wm = wave % CF::WAVES_M, wn = wave / CF::WAVES_M;
  const int nfull = SPLIT ? (s.n & ~1) : s.n;
  for (int k = G; k < nfull; k += 2) {
    int tm, tn;
    grouped_walk(start + j + k * nw, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    f32x16_t acc[CF::TM][CF::TN];
    mainloop_ring<CF, L>(a, a.X, a.dY, a.T, tm, tn, ring, wave, lane, acc);
    float* const ep = reinterpret_cast<float*>(stage_slot) + (wave & 1) * 32 * (CF::WM + 4);
    epilogue_paced<CF, EPI, D, P>(a, acc, a.W, a.S1, a.S2, tm * CF::BM, tn * CF::BN, wm, wn,
                                  lane, ep);
    bars += MB + EB;
  }
  if (SPLIT && (s.n & 1)) {
    int tm, tn;
    grouped_walk(start + j + (s.n - 1) * nw, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    const int tq = 2 * tm + G;   // this group's d_in half
    f32x16_t acc[CQ::TM][CQ::TN];
    mainloop_ring<CQ, L>(a, a.X, a.dY, a.T, tq, tn, ring, wave, lane, acc);
    float* const ep = reinterpret_cast<float*>(stage_slot) + (wave & 1) * 32 * (CQ::WM + 4);
    epilogue_paced<CQ, EPI, D, P>(a, acc, a.W, a.S1, a.S2, tq * CQ::BM, tn * CQ::BN,
                               wave % CQ::WAVES_M, wave / CQ::WAVES_M, lane, ep);
    bars += MB + EQ;
  }
  for (; bars < s.total; ++bars) FORGE_PP_BARRIER();
}

template <class CF, class CQ, int EPI, int D, int P, bool SPLIT>
__global__ __launch_bounds__(2 * CF::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void wgrad_pingpong_kernel(WgradArgs a) {
  constexpr int L = 3;
  static_assert(CF::THREADS == CQ::THREADS && CQ::STAGE <= CF::STAGE, "split tiles fit the ring");
  static_assert(2 * 32 * (CF::WM + 4) * 4 <= CF::STAGE * 2, "two waves' staging per slot");
  __shared__ __attribute__((aligned(1024))) uint16_t g0s0[CF::STAGE], g0s1[CF::STAGE],
      g0s2[CF::STAGE], g1s0[CF::STAGE], g1s1[CF::STAGE], g1s2[CF::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (Filled member by member: an aggregate initializer of LDS addresses would
  // become a constant in global memory.)
  Ring<L> ring;
  if (wave < 4) {
    ring.s[0] = g0s0;
    ring.s[1] = g0s1;
    ring.s[2] = g0s2;
    pingpong_group<CF, CQ, EPI, D, P, SPLIT, L, 0>(a, ring, wave, lane);
  } else {
    ring.s[0] = g1s0;
    ring.s[1] = g1s1;
    ring.s[2] = g1s2;
    pingpong_group<CF, CQ, EPI, D, P, SPLIT, L, 1>(a, ring, wave - 4, lane);
  }
}

}  // namespace forge
