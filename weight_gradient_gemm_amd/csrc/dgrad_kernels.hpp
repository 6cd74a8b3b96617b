// Input-gradient GEMM of the same linear layer for gfx950: dX = dY W_b, with
// W_b the float32 weight rounded to bf16 (the operand precision of the
// layer's bf16 matmuls) and a float32 accumulator, stored as bf16 or float32.
//
// It exists to be ordered before the fused optimizer step: that step
// overwrites W in place, so dX must read W first (FORGE assessment, "Math
// verified, not asserted", P1, the in-place dX-before-update hazard). The
// linear-backward entry points launch this kernel, then the fused weight
// gradient kernel, on one stream.
//
// The tile computes C = dX^T: rows i (d_in, the MFMA M side) and columns t
// (tokens, the N side), reducing over the layer's d_out outputs o (K) in
// ascending chunks of 16, so like the weight gradient the result is bitwise
// the same for every tile shape.
//
//   A operand, W [o][i] (i contiguous): each stage of 32 rows of o is loaded
//   as float32 into registers, rounded to bf16 and written to LDS in the
//   weight-gradient kernel's operand layout ([k][feature] rows, 16-byte chunk
//   c of row r at c ^ 4 (r mod 4)), then gathered with LDS transpose reads.
//   Given a bf16 copy of W instead (WB), the stage's rows go straight into
//   that layout with direct-to-LDS loads, like the weight gradient's
//   operands: half the bytes, and no register pass or LDS store instructions.
//   B operand, dY [t][o] (o contiguous): 8 consecutive o of one token are
//   already contiguous, so each stage goes straight into LDS as [token][o]
//   rows of 64 bytes, chunk c of row r at c ^ ((r / 4) mod 4) so that the
//   16-byte reads of 16 consecutive tokens fall on distinct banks.
//   Epilogue: the weight-gradient kernel's gradient store, with dX's token
//   rows in place of W's rows.
#pragma once

#include "wgrad_kernels.hpp"

namespace forge {

// One dX^T tile. `a` is set up for the epilogue: a.W = dX, a.d_in = d_in (dX
// row length), a.d_out = T (dX rows). K = the layer's d_out.
//
// Per stage s (32 outputs o): loads for stage s + 2 are issued (float32 W
// into the register set stage s used, bf16 W and dY straight into LDS slot
// (s + 2) % 4), so each load has about a stage and a half of MFMA work to land.
// Wsrc: float32 W, or with WB its bf16 copy.
template <class C, int EPI, bool WB>
__device__ __forceinline__ void dgrad_tile(const WgradArgs& a, const uint16_t* __restrict__ dY,
                                           const void* __restrict__ Wsrc, int K, int tile_m,
                                           int tile_n, const Slots& sl) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TM = C::TM, TN = C::TN;
  constexpr int RBA = BM * 2;                       // bytes per LDS row of the A region
  constexpr int BOFF = BK * RBA;                    // byte offset of the B region
  constexpr int LPR_A = BM / 4;                     // lanes per float32 row of W (16 B each)
  constexpr int RPI_A = 64 / LPR_A;                 // W rows per load instruction
  constexpr int NA = BK / RPI_A / C::WAVES;         // W loads per wave per stage
  constexpr int NB = BN / 16 / C::WAVES;            // dY loads (16 token rows each) per wave
  static_assert(NA >= 1 && NB >= 1 && (BK / RPI_A) % C::WAVES == 0 && (BN / 16) % C::WAVES == 0,
                "stage loads split evenly over the waves");
  static_assert(BOFF + BN * 64 <= C::STAGE * 2, "stage exceeds a slot");
  // bf16 W: 1 KB direct-to-LDS loads of RPQ rows (CPA 16-byte chunks each).
  constexpr int CPA = BM / 8;
  constexpr int RPQ = 64 / CPA;
  constexpr int NQA = BK / RPQ / C::WAVES;          // bf16 W loads per wave per stage
  static_assert(!WB || (NQA >= 1 && (BK / RPQ) % C::WAVES == 0), "bf16 W loads split evenly");
  constexpr int NAL = WB ? NQA : NA;                // W load instructions per wave per stage
  const float* __restrict__ W = static_cast<const float*>(Wsrc);
  const uint16_t* __restrict__ Wh = static_cast<const uint16_t*>(Wsrc);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int d_in = a.d_in;
  const int64_t T = a.d_out;
  const int i0 = tile_m * BM;
  const int64_t t0 = int64_t(tile_n) * BN;

  // W loads: instruction j of this wave covers W rows r = RPI_A (NA wave + j)
  // + lane / LPR_A of the stage; the lane's 4 floats are columns
  // i0 + 4 (lane % LPR_A). Columns past d_in read 0.
  const int a_row = lane / LPR_A, a_col = 4 * (lane % LPR_A);
  const uint32_t a_voff = i0 + a_col < d_in ? uint32_t(a_row * d_in + a_col) * 4u : kOOB;
  // LDS byte offsets of the rounded values: 8 bytes in chunk a_col / 8 (swizzled).
  uint32_t a_lds[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    const int r = RPI_A * (NA * wave + j) + a_row;
    a_lds[j] = uint32_t(r * RBA + (((a_col >> 3) ^ (4 * (r & 3))) << 4) + (a_col & 4) * 2);
  }
  // bf16 W loads: instruction q = NQA wave + j writes LDS rows RPQ q ..
  // RPQ q + RPQ - 1; lane l fills physical chunk l % CPA of row RPQ q + l / CPA,
  // which holds logical chunk (l % CPA) ^ 4 (row mod 4). Columns past d_in read 0.
  uint32_t h_voff[WB ? NQA : 1];
#pragma unroll
  for (int j = 0; j < (WB ? NQA : 1); ++j) {
    const int lrow = lane / CPA, r = RPQ * (NQA * wave + j) + lrow;
    const int ch = (lane % CPA) ^ (4 * (r & 3));
    h_voff[j] = i0 + 8 * ch < d_in ? uint32_t(lrow * d_in + 8 * ch) * 2u : kOOB;
  }
  // dY loads: instruction q = NB wave + j writes LDS rows 16 q .. 16 q + 15;
  // lane l fills row 16 q + l / 4, physical chunk l % 4, which holds logical
  // chunk c = (l % 4) ^ ((l / 16) % 4), i.e. outputs k0 + 8 c .. + 7.
  const int b_row = lane >> 2, b_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t b_voff = uint32_t(b_row * K + 8 * b_chunk) * 2u;

  int g_stage = 0;
  const int nk = (K + BK - 1) / BK;
  const int64_t rows_t = T - t0 < BN ? T - t0 : BN;
  f32x4_t wreg[2][NA];
  auto issue = [&](uint16_t* slot, f32x4_t (&wr)[NA]) {
    const int k0 = g_stage * BK;
    const int rows_k = K - k0 < BK ? (K - k0 > 0 ? K - k0 : 0) : BK;
    const __amdgpu_buffer_rsrc_t ry =
        window32(dY + t0 * K + k0, k0 < K ? uint32_t(rows_t * K - k0) * 2u : 0u);
    ++g_stage;
    if constexpr (WB) {
      const __amdgpu_buffer_rsrc_t rh =
          window32(Wh + int64_t(k0) * d_in + i0,
                   rows_k > 0 ? uint32_t(rows_k * d_in - i0) * 2u : 0u);
#pragma unroll
      for (int j = 0; j < NQA; ++j) {
        const int q = NQA * wave + j;
        load16_to_lds(rh, slot + q * 512, h_voff[j], q * RPQ * d_in * 2);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rw =
          window32(W + int64_t(k0) * d_in + i0,
                   rows_k > 0 ? uint32_t(rows_k * d_in - i0) * 4u : 0u);
#pragma unroll
      for (int j = 0; j < NA; ++j)
        wr[j] = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                         rw, (int)a_voff, (int)(RPI_A * (NA * wave + j) * d_in * 4), 0));
    }
    const uint32_t bv = k0 + 8 * b_chunk < K ? b_voff : kOOB;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int q = NB * wave + j;
      load16_to_lds(ry, slot + BOFF / 2 + q * 512, bv, q * 16 * K * 2);
    }
  };
  auto convert_write = [&](uint16_t* slot, const f32x4_t (&wr)[NA]) {
    if constexpr (!WB) {
      char* base = reinterpret_cast<char*>(slot);
#pragma unroll
      for (int j = 0; j < NA; ++j)
        *reinterpret_cast<u32x2_t*>(base + a_lds[j]) = pack_bf16x4(wr[j]);
    }
  };

  // Operand addresses. A: the transpose-read pattern of the weight-gradient
  // kernel. B: token row = the wave's 32-token block + lane % 32; logical
  // chunk 2 kk + lane / 32 for MFMA chunk kk.
  const int g = lane >> 4, jl = lane & 15;
  const int rsub = 8 * (g >> 1) + (jl >> 2);
  uint32_t fa[TM], fb[TN][2];
#pragma unroll
  for (int m = 0; m < TM; ++m) {
    const int blk = (wm * C::WM + m * 32) >> 5;
    const int ch = (4 * blk + 2 * (g & 1) + ((jl & 3) >> 1)) ^ (4 * (jl >> 2));
    fa[m] = uint32_t(rsub * RBA + ch * 16 + (jl & 1) * 8);
  }
#pragma unroll
  for (int n = 0; n < TN; ++n) {
    const int row = wn * C::WN + n * 32 + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
      fb[n][kk] = uint32_t(BOFF + row * 64 + (((2 * kk + (lane >> 5)) ^ ((row >> 2) & 3)) << 4));
  }
  auto operand_a = [](const uint16_t* slot, uint32_t off) {
    const char* b = reinterpret_cast<const char*>(slot) + off;
    const i16x4_t lo = lds_read_tr16(b);
    const i16x4_t hi = lds_read_tr16(b + 4 * RBA);
    const i16x4_t both[2] = {lo, hi};
    bf16x8_t r;
    __builtin_memcpy(&r, both, sizeof(r));
    return r;
  };
  bf16x8_t frag[2][TM + TN];
  auto read_frags = [&](int f, const uint16_t* slot, int kk) {
#pragma unroll
    for (int m = 0; m < TM; ++m) frag[f][m] = operand_a(slot, fa[m] + kk * 16 * RBA);
#pragma unroll
    for (int n = 0; n < TN; ++n)
      frag[f][TM + n] =
          *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const char*>(slot) + fb[n][kk]);
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
        acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag[f][m], frag[f][TM + n],
                                                            acc[m][n], 0, 0, 0);
  };
  constexpr int NREAD = 2 * TM + TN;
  auto interleave = [&](int loads) {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
      if (i < (NREAD + 1) / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
      if (i < loads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // VMEM read
    }
  };
  // After this wave's loads of stage s + 2 (NAL + NB) are issued, the stage
  // s + 1 loads are complete when at most that many remain.
  constexpr int kWait = waitcnt_imm(NAL + NB, 0);
#define FORGE_DGRAD_BARRIER(IMM)              \
  do {                                        \
    __builtin_amdgcn_sched_barrier(0);        \
    __builtin_amdgcn_s_waitcnt(IMM);          \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)
  // Chunk 0: loads of stage s + 2, chunk 1's operand reads, MFMAs on chunk 0.
  // Stage s + 1's W is rounded into its slot; once its dY loads have landed
  // the barrier publishes the slot. Chunk 1: MFMAs while stage s + 1's chunk 0
  // operands are read.
  auto stage = [&](uint16_t* cur, uint16_t* nxt, uint16_t* fut, f32x4_t (&w_fut)[NA],
                   f32x4_t (&w_nxt)[NA]) {
    issue(fut, w_fut);
    read_frags(1, cur, 1);
    mfmas(0);
    interleave(NAL + NB);
    __builtin_amdgcn_sched_barrier(0);
    convert_write(nxt, w_nxt);
    FORGE_DGRAD_BARRIER(kWait);
    read_frags(0, nxt, 0);
    mfmas(1);
    interleave(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  if (nk > 0) {
    issue(sl.s0, wreg[0]);
    issue(sl.s1, wreg[1]);
    convert_write(sl.s0, wreg[0]);
    FORGE_DGRAD_BARRIER(kWait);
    read_frags(0, sl.s0, 0);
    // Whole rounds of 4 stages (static slots); stages past K load zeros,
    // which add exactly +0 to every accumulator.
    const int rounds = (nk + 3) / 4;
    for (int r = 0; r < rounds; ++r) {
      stage(sl.s0, sl.s1, sl.s2, wreg[0], wreg[1]);
      stage(sl.s1, sl.s2, sl.s3, wreg[1], wreg[0]);
      stage(sl.s2, sl.s3, sl.s0, wreg[0], wreg[1]);
      stage(sl.s3, sl.s0, sl.s1, wreg[1], wreg[0]);
    }
  }
#undef FORGE_DGRAD_BARRIER
  // The epilogue starts with a full barrier, which also drains the loads of
  // the zero stages still in flight.
  uint16_t* ep = wave == 0 ? sl.s0 : wave == 1 ? sl.s1 : wave == 2 ? sl.s2 : sl.s3;
  epilogue<C, EPI>(a, acc, a.W, nullptr, nullptr, i0, int(t0), wm, wn, lane,
                   reinterpret_cast<float*>(ep));
}

// Grid launch, one workgroup per dX^T tile in the XCD-aware walk. W: float32
// weights, or with WB their bf16 copy.
template <class C, int EPI, bool WB>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void dgrad_kernel(WgradArgs a, const void* W, int K) {
  FORGE_DECLARE_SLOTS(C::STAGE);
  int e, tm, tn;
  map_tile(blockIdx.x, a.num_tiles, a.tiles_m, a.tiles_n, a.group_m, e, tm, tn);
  dgrad_tile<C, EPI, WB>(a, a.dY, W, K, tm, tn, ring);
}

}  // namespace forge
