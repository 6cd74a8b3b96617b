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
// have the token axis strided (X and dY are row-major [T, d]) while an MFMA
// operand needs 8 consecutive tokens per lane: stages of 32 tokens go from
// global memory straight into LDS as [token][feature] rows, and the operands
// are gathered with the gfx950 LDS transpose read (see wgrad_tile).
//
// Order of accumulation: for every element, the tokens enter in ascending
// chunks of 16 through one accumulator, whatever the tile shape or schedule.
// Ragged token tails are zero-filled, so every tile shape, the persistent
// schedule and the grouped variant see the same chunk sequence, which makes
// the result bitwise partition-independent.
//
// Epilogue: accumulators pass through LDS to a row-major layout, then the
// optimizer updates W and its state with whole-row 16-byte accesses,
// software-pipelined so state loads overlap the arithmetic.
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

// What the epilogue does with the accumulator: an optimizer or a gradient
// store (low two bits), plus modifiers.
enum Epi : int {
  EPI_ADAMW = 0,
  EPI_SGDM = 1,
  EPI_GRAD = 2,
  EPI_EXACT_SQRT = 4,   // AdamW with eps = 0: the square root must be exact on denormals
  EPI_BF16_STATE = 8,   // AdamW m and v stored as bf16 (W stays float32)
  EPI_BF16_OUT = 16,    // gradient store rounded to bf16
  EPI_SCALE = 32,       // the accumulator times WgradArgs::gscale (scaled fp8 inputs)
  EPI_WB_OUT = 64,      // AdamW / SGD: the updated W also stored as bf16 into WgradArgs::Wb
};

__host__ __device__ constexpr int epi_op(int epi) { return epi & 3; }
__host__ __device__ constexpr bool is_adamw(int epi) { return epi_op(epi) == EPI_ADAMW; }
// Bytes per element of the epilogue's arrays: W (or the stored gradient), then
// the first and second optimizer state.
__host__ __device__ constexpr int epi_w_bytes(int epi) {
  return epi_op(epi) == EPI_GRAD && (epi & EPI_BF16_OUT) ? 2 : 4;
}
__host__ __device__ constexpr int epi_state_bytes(int epi) {
  return is_adamw(epi) && (epi & EPI_BF16_STATE) ? 2 : 4;
}

struct WgradArgs {
  const uint16_t* X;   // [rows, d_in] bf16 bits
  const uint16_t* dY;  // [rows, d_out] bf16 bits
  float* W;            // [(E,) d_out, d_in]; the gradient for EPI_GRAD (bf16 with EPI_BF16_OUT)
  float* S1;           // m (AdamW) or momentum buffer (SGD); bf16 with EPI_BF16_STATE
  float* S2;           // v (AdamW); bf16 with EPI_BF16_STATE
  int64_t T;           // tokens (dense calls)
  int32_t d_in;
  int32_t d_out;
  int32_t tiles_m;     // ceil(d_in / BM)
  int32_t tiles_n;     // ceil(d_out / BN)
  int32_t num_tiles;   // tiles_m * tiles_n (* E)
  int32_t group_m;     // tile-order swizzle: tile rows per group
  AdamWConsts adam;
  SgdmConsts sgd;
  float gscale;        // EPI_SCALE: factor applied to the accumulator once
  uint16_t* Wb;        // EPI_WB_OUT: [d_out, d_in] bf16 copy of the updated W (dense only)
};

struct GroupTable {
  int64_t off[FORGE_MAX_EXPERTS + 1];
  int32_t order[FORGE_MAX_EXPERTS];   // experts in launch order
};

// Compile-time shape of one workgroup's tile.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int OCC_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;            // tile extent along d_in, d_out
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int BK = BK_;                      // tokens per LDS stage
  static constexpr int OCC = OCC_;                    // workgroups per CU the resources allow
  static constexpr int WAVES = WAVES_M * WAVES_N;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 32, TN = WN / 32;    // 32x32 MFMA blocks per wave
  static constexpr int STAGE = BK * (BM + BN);        // bf16 elements of one LDS stage
  static_assert(WAVES == 4 && BK == 32, "4 waves, stages of two 16-token MFMA chunks");
  static_assert(TM >= 1 && TN >= 1, "wave tile smaller than one MFMA block");
  static_assert(BM % 128 == 0 && BN % 128 == 0 && BM <= 512 && BN <= 512,
                "rows of 16 to 64 chunks of 16 bytes");
};

// Tile grid position of logical tile t of the grouped walk (see map_tile).
__host__ __device__ inline void grouped_walk(int t, int tiles_m, int tiles_n, int group_m, int& tm,
                                             int& tn) {
  const int group_size = group_m * tiles_n;
  const int g = t / group_size;
  const int first_m = g * group_m;
  const int gm = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
  const int r = t - g * group_size;
  tm = first_m + r % gm;
  tn = r / gm;
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
  grouped_walk(logical - e * per_expert, tiles_m, tiles_n, group_m, tm, tn);
}

// The optimizer on the 4 consecutive elements one lane owns.
template <bool EXACT_SQRT>
__device__ __forceinline__ void adamw_vec4(const f32x4_t& g, f32x4_t& w, f32x4_t& m, f32x4_t& v,
                                           const AdamWConsts& c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float wj = w[j], mj = m[j], vj = v[j];
    adamw_elem<EXACT_SQRT>(g[j], wj, mj, vj, c);
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

// Byte offset that lies beyond every buffer window: the hardware returns zeros.
constexpr uint32_t kOOB = 0x80000000u;

// Raw buffer window over `bytes` bytes from `base` (reads at or past the end
// return 0, writes there are dropped). Word 3 is the gfx9-family raw-buffer
// format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > int64_t(kOOB) ? int64_t(kOOB) : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n,
                                           0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t window32(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// float32 <-> bf16 for 4 elements (round to nearest even, as the hardware
// conversion does).
__device__ __forceinline__ u32x2_t pack_bf16x4(const f32x4_t& v) {
  return __builtin_bit_cast(u32x2_t, __builtin_convertvector(v, bf16x4_t));
}
__device__ __forceinline__ f32x4_t unpack_bf16x4(const u32x2_t& u) {
  return __builtin_convertvector(__builtin_bit_cast(bf16x4_t, u), f32x4_t);
}

// Optimizer state is streamed once per step: non-temporal cache policy.
constexpr int kStatePolicy = 2;

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                        const f32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)voff, (int)soff,
                                         kStatePolicy);
}

__device__ __forceinline__ f32x4_t load16f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(
      f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kStatePolicy));
}

// Four consecutive elements of a float32 (ES = 4) or bf16 (ES = 2) array.
template <int ES>
__device__ __forceinline__ f32x4_t load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (ES == 4) {
    return load16f(r, voff, soff);
  } else {
    return unpack_bf16x4(__builtin_bit_cast(
        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, kStatePolicy)));
  }
}
template <int ES>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                       const f32x4_t& v) {
  if constexpr (ES == 4) {
    store16(r, voff, soff, v);
  } else {
    __builtin_amdgcn_raw_buffer_store_b64(pack_bf16x4(v), r, (int)voff, (int)soff, kStatePolicy);
  }
}

// s_waitcnt immediate (gfx9 family): vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4 (left at its maximum), lgkmcnt in 11:8.
__host__ __device__ constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

__host__ __device__ constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// 16 bytes per lane from a buffer window straight into LDS: lane t writes at
// dst + 16 t (dst is wave-uniform; it becomes M0).
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint16_t* dst,
                                              uint32_t voff, int soff) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, soff, 0, 0);
}

// LDS transpose read of 4 x 16-bit values (see wgrad_tile).
__device__ __forceinline__ i16x4_t lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// The four LDS ring slots of a workgroup. Each is its own __shared__ array,
// which lets the compiler tell the slots apart when it places waits for the
// direct-to-LDS loads.
struct Slots {
  uint16_t *s0, *s1, *s2, *s3;
};

// Row-major epilogue through LDS. Each wave owns a region of 32 rows x
// (WM + 4) floats (in one of the ring slots); the 4-float pad keeps both the
// column-major dump and the row-major read conflict-free. A direct store from
// the MFMA result layout would touch 32 rows of W per instruction; after the
// pass through LDS every state access covers 256 / WM whole rows of WM
// contiguous floats.
//
// The wave's 32-column blocks are cut into units of 4 row instructions and
// software-pipelined: the next unit's state loads are issued before a unit's
// optimizer math and stores, so memory latency overlaps the arithmetic. (On
// this chip family the vector-memory counter covers stores as well as loads
// and drains in issue order, so loads issued after a unit's stores would also
// wait for those stores; issuing them first keeps the stores in flight.)
// State is addressed through buffer windows of one 32-row block: rows past
// d_out lie beyond the window (loads read 0, stores are dropped) and columns
// past d_in get an out-of-window lane offset, so no lane needs a branch.
template <class C, int EPI>
__device__ __forceinline__ void epilogue(const WgradArgs& a, f32x16_t (&acc)[C::TM][C::TN],
                                         float* __restrict__ W, float* __restrict__ S1,
                                         float* __restrict__ S2, int i0, int o0, int wm, int wn,
                                         int lane, float* ep) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM;
  constexpr int LD = WM + 4;                 // floats per LDS row
  constexpr int LPR = WM / 4;                // lanes per row (4 elements each)
  constexpr int RPI = 64 / LPR;              // rows per instruction
  constexpr int NI = 32 / RPI;               // instructions per 32-column block
  constexpr int B = NI < 4 ? NI : 4;         // instructions per unit
  constexpr int UPB = NI / B;                // units per block
  constexpr int U = TN * UPB;
  constexpr int D = 2;                       // units in flight
  constexpr int OP = epi_op(EPI);
  constexpr int NS = OP == EPI_ADAMW ? 3 : (OP == EPI_SGDM ? 2 : 0);   // state arrays read
  // Bytes per element of W (or the gradient), S1, S2 and the bf16 copy of W.
  constexpr int ESW = epi_w_bytes(EPI), ESS = epi_state_bytes(EPI);
  constexpr int ES[4] = {ESW, ESS, ESS, 2};
  constexpr bool WB = (EPI & EPI_WB_OUT) != 0;
  static_assert(!WB || (OP != EPI_GRAD && ESW == 4), "the bf16 copy is of an updated W");
  static_assert(NI % B == 0, "epilogue units must tile a block");
  static_assert(32 * LD * 4 <= C::STAGE * 2, "a wave's epilogue staging exceeds a slot");

  const int d_in = a.d_in, d_out = a.d_out;
  __syncthreads();                           // every wave is done with the operand ring
  const int r_lane = lane / LPR, c_lane = (lane % LPR) * 4;
  const int iw0 = i0 + wm * WM;
  const bool lane_ok = iw0 + c_lane < d_in;
  const uint32_t elem = uint32_t(r_lane * d_in + c_lane);   // lane's first element in a block
  char* const arr[4] = {reinterpret_cast<char*>(W), reinterpret_cast<char*>(S1),
                        reinterpret_cast<char*>(S2), reinterpret_cast<char*>(a.Wb)};
  // Array k: the lane's byte offset, the bytes between row instructions, and
  // the window from the wave's first column of block n's first row.
  auto voff = [&](int k) { return lane_ok ? elem * uint32_t(ES[k]) : kOOB; };
  auto inst_bytes = [&](int k) { return uint32_t(RPI) * uint32_t(d_in) * uint32_t(ES[k]); };
  auto block_window = [&](int k, int n) {
    const int64_t ob = int64_t(o0) + wn * C::WN + n * 32;
    return window(arr[k] + (ob * d_in + iw0) * ES[k], ((int64_t(d_out) - ob) * d_in - iw0) * ES[k]);
  };
  auto dump = [&](int n) {
    // Column-major: lane (o = lane % 32) writes rows 4 (lane / 32) + 8 q .. + 3.
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t g = {acc[m][n][4 * q + 0], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                           acc[m][n][4 * q + 3]};
        *reinterpret_cast<f32x4_t*>(ep + (lane & 31) * LD + m * 32 + 8 * q + 4 * (lane >> 5)) = g;
      }
  };
  f32x4_t st[D][B][NS > 0 ? NS : 1];
  auto issue = [&](int u) {
    const int n = u / UPB, j0 = (u % UPB) * B;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      const __amdgpu_buffer_rsrc_t r = block_window(k, n);
#pragma unroll
      for (int j = 0; j < B; ++j)
        st[u % D][j][k] = k == 0 ? load4<ESW>(r, voff(k), (j0 + j) * inst_bytes(k))
                                 : load4<ESS>(r, voff(k), (j0 + j) * inst_bytes(k));
    }
  };
#pragma unroll
  for (int u = 0; u < D - 1 && u < U; ++u) issue(u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u + D - 1 < U) issue(u + D - 1);
    const int n = u / UPB, j0 = (u % UPB) * B;
    // LDS operations of one wave complete in order: the reads below see the
    // dump, and the dump follows the previous block's reads.
    if (u % UPB == 0) dump(n);
    f32x4_t g[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      g[j] = *reinterpret_cast<const f32x4_t*>(ep + ((j0 + j) * RPI + r_lane) * LD + c_lane);
      if constexpr ((EPI & EPI_SCALE) != 0) g[j] = g[j] * a.gscale;
    }
    const __amdgpu_buffer_rsrc_t rw = block_window(0, n);
    if constexpr (OP == EPI_GRAD) {
#pragma unroll
      for (int j = 0; j < B; ++j) store4<ESW>(rw, voff(0), (j0 + j) * inst_bytes(0), g[j]);
    } else if constexpr (OP == EPI_ADAMW) {
      const __amdgpu_buffer_rsrc_t r1 = block_window(1, n), r2 = block_window(2, n);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        f32x4_t& s = st[u % D][j][0];
        adamw_vec4<(EPI & EPI_EXACT_SQRT) != 0>(g[j], s, st[u % D][j][1], st[u % D][j][2],
                                                 a.adam);
        store4<ESW>(rw, voff(0), (j0 + j) * inst_bytes(0), s);
        store4<ESS>(r1, voff(1), (j0 + j) * inst_bytes(1), st[u % D][j][1]);
        store4<ESS>(r2, voff(2), (j0 + j) * inst_bytes(2), st[u % D][j][2]);
        if constexpr (WB) store4<2>(block_window(3, n), voff(3), (j0 + j) * inst_bytes(3), s);
      }
    } else {
      const __amdgpu_buffer_rsrc_t r1 = block_window(1, n);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        sgdm_vec4(g[j], st[u % D][j][0], st[u % D][j][1], a.sgd);
        store4<ESW>(rw, voff(0), (j0 + j) * inst_bytes(0), st[u % D][j][0]);
        store4<ESS>(r1, voff(1), (j0 + j) * inst_bytes(1), st[u % D][j][1]);
        if constexpr (WB)
          store4<2>(block_window(3, n), voff(3), (j0 + j) * inst_bytes(3), st[u % D][j][0]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// AdamW epilogue for bf16 optimizer state. As epilogue(), but each lane owns
// 8 consecutive columns of a row instead of 4, so m and v (8 bf16 = 16 bytes)
// move in whole 16-byte accesses, like W (two per lane): 8 memory
// instructions per 8 elements instead of 12, for a third fewer bytes.
template <class C, int EPI>
__device__ __forceinline__ void epilogue_wide(const WgradArgs& a, f32x16_t (&acc)[C::TM][C::TN],
                                              float* __restrict__ W, float* __restrict__ S1,
                                              float* __restrict__ S2, int i0, int o0, int wm,
                                              int wn, int lane, float* ep) {
  constexpr int TM = C::TM, TN = C::TN, WM = C::WM;
  constexpr int LD = WM + 4;                 // floats per LDS row
  constexpr int LPR = WM / 8;                // lanes per row (8 elements each)
  constexpr int RPI = 64 / LPR;              // rows per instruction
  constexpr int NI = 32 / RPI;               // instructions per 32-row block
  constexpr int B = NI < 4 ? NI : 4;         // instructions per unit
  constexpr int UPB = NI / B;
  constexpr int U = TN * UPB;
  constexpr int D = 2;                       // units in flight
  static_assert(is_adamw(EPI) && (EPI & EPI_BF16_STATE), "bf16-state AdamW only");
  static_assert((EPI & EPI_WB_OUT) == 0, "no bf16 weight copy with bf16 state");
  static_assert(NI % B == 0, "epilogue units must tile a block");
  static_assert(32 * LD * 4 <= C::STAGE * 2, "a wave's epilogue staging exceeds a slot");

  const int d_in = a.d_in, d_out = a.d_out;
  __syncthreads();                           // every wave is done with the operand ring
  const int r_lane = lane / LPR, c_lane = (lane % LPR) * 8;
  const int iw0 = i0 + wm * WM;
  const bool lane_ok = iw0 + c_lane < d_in;  // d_in is a multiple of 8: all 8 or none
  const uint32_t elem = uint32_t(r_lane * d_in + c_lane);
  const uint32_t vw = lane_ok ? elem * 4u : kOOB, vs = lane_ok ? elem * 2u : kOOB;
  const uint32_t iw = uint32_t(RPI) * uint32_t(d_in) * 4u, is = uint32_t(RPI) * uint32_t(d_in) * 2u;
  auto block_window = [&](char* arr, int es, int n) {
    const int64_t ob = int64_t(o0) + wn * C::WN + n * 32;
    return window(arr + (ob * d_in + iw0) * es, ((int64_t(d_out) - ob) * d_in - iw0) * es);
  };
  char* const cw = reinterpret_cast<char*>(W);
  char* const c1 = reinterpret_cast<char*>(S1);
  char* const c2 = reinterpret_cast<char*>(S2);
  auto dump = [&](int n) {
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4_t g = {acc[m][n][4 * q + 0], acc[m][n][4 * q + 1], acc[m][n][4 * q + 2],
                           acc[m][n][4 * q + 3]};
        *reinterpret_cast<f32x4_t*>(ep + (lane & 31) * LD + m * 32 + 8 * q + 4 * (lane >> 5)) = g;
      }
  };
  f32x4_t w[D][B][2];
  u32x4_t mv[D][B][2];
  auto issue = [&](int u) {
    const int n = u / UPB, j0 = (u % UPB) * B;
    const __amdgpu_buffer_rsrc_t rw = block_window(cw, 4, n), r1 = block_window(c1, 2, n),
                                 r2 = block_window(c2, 2, n);
#pragma unroll
    for (int j = 0; j < B; ++j) {
      w[u % D][j][0] = load16f(rw, vw, (j0 + j) * iw);
      w[u % D][j][1] = load16f(rw, vw + 16u, (j0 + j) * iw);
      mv[u % D][j][0] = __builtin_amdgcn_raw_buffer_load_b128(r1, (int)vs, (int)((j0 + j) * is),
                                                              kStatePolicy);
      mv[u % D][j][1] = __builtin_amdgcn_raw_buffer_load_b128(r2, (int)vs, (int)((j0 + j) * is),
                                                              kStatePolicy);
    }
  };
#pragma unroll
  for (int u = 0; u < D - 1 && u < U; ++u) issue(u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (u + D - 1 < U) issue(u + D - 1);
    const int n = u / UPB, j0 = (u % UPB) * B;
    if (u % UPB == 0) dump(n);
    f32x4_t g[B][2];
#pragma unroll
    for (int j = 0; j < B; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        g[j][h] = *reinterpret_cast<const f32x4_t*>(ep + ((j0 + j) * RPI + r_lane) * LD + c_lane +
                                                    4 * h);
        if constexpr ((EPI & EPI_SCALE) != 0) g[j][h] = g[j][h] * a.gscale;
      }
    const __amdgpu_buffer_rsrc_t rw = block_window(cw, 4, n), r1 = block_window(c1, 2, n),
                                 r2 = block_window(c2, 2, n);
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const u32x4_t mb = mv[u % D][j][0], vb = mv[u % D][j][1];
      f32x4_t m0 = unpack_bf16x4(u32x2_t{mb[0], mb[1]}), m1 = unpack_bf16x4(u32x2_t{mb[2], mb[3]});
      f32x4_t v0 = unpack_bf16x4(u32x2_t{vb[0], vb[1]}), v1 = unpack_bf16x4(u32x2_t{vb[2], vb[3]});
      adamw_vec4<(EPI & EPI_EXACT_SQRT) != 0>(g[j][0], w[u % D][j][0], m0, v0, a.adam);
      adamw_vec4<(EPI & EPI_EXACT_SQRT) != 0>(g[j][1], w[u % D][j][1], m1, v1, a.adam);
      store16(rw, vw, (j0 + j) * iw, w[u % D][j][0]);
      store16(rw, vw + 16u, (j0 + j) * iw, w[u % D][j][1]);
      const u32x2_t pm0 = pack_bf16x4(m0), pm1 = pack_bf16x4(m1);
      const u32x2_t pv0 = pack_bf16x4(v0), pv1 = pack_bf16x4(v1);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pm0[0], pm0[1], pm1[0], pm1[1]}, r1, (int)vs,
                                             (int)((j0 + j) * is), kStatePolicy);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{pv0[0], pv0[1], pv1[0], pv1[1]}, r2, (int)vs,
                                             (int)((j0 + j) * is), kStatePolicy);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One output tile: mainloop over all tokens, then the epilogue.
//
// Staging: a buffer load with the LDS flag writes lane t's 16 bytes at
// M0 + 16 t (lanes whose offset falls outside the buffer window write zeros),
// so the operands reach LDS without passing through registers, permutes or
// LDS store instructions. A stage holds [token][feature] rows of X, then of
// dY; the 16-byte chunk c of token row r is stored at chunk c ^ 4 (r mod 4).
// An MFMA operand (8 consecutive tokens of one feature per lane) is gathered
// with two LDS transpose reads (ds_read_b64_tr_b16): within a group of 16
// lanes, lane j supplies the address of 4 consecutive features of token row
// j / 4 and receives feature j of each of the group's 4 rows. Each 32-lane
// half of such a read touches 4 rows x 64 contiguous bytes; the swizzle puts
// the 4 rows on disjoint banks.
//
// Ring of 4 slots. Per stage s (two 16-token chunks):
//   chunk 0: MFMAs on chunk 0; read chunk 1's operands from slot s % 4.
//   wait for this wave's LDS reads (slot s % 4 is then free) and for its
//   loads of stage s + 1; barrier (no fence: the waits are explicit).
//   chunk 1: load stage s + 4 into slot s % 4; MFMAs on chunk 1; read stage
//   s + 1's chunk 0 operands from slot (s + 1) % 4.
// Each load has about two and a half stages of MFMA work to land.
template <class C, int EPI>
__device__ __forceinline__ void wgrad_tile(const WgradArgs& a, const uint16_t* __restrict__ X,
                                           const uint16_t* __restrict__ dY,
                                           float* __restrict__ W, float* __restrict__ S1,
                                           float* __restrict__ S2, int64_t T, int tile_m,
                                           int tile_n, const Slots& sl) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, TM = C::TM, TN = C::TN;
  constexpr int RBX = BM * 2, RBY = BN * 2;             // bytes per token row
  constexpr int CPX = BM / 8, CPY = BN / 8;             // 16-byte chunks per row
  constexpr int QX = BK * RBX / 1024, QY = BK * RBY / 1024;
  constexpr int NQW = (QX + QY) / C::WAVES;             // 1 KB loads per wave per stage
  constexpr int L = 4;                                  // ring slots
  static_assert((QX + QY) % C::WAVES == 0, "stage loads split evenly over the waves");

  // The wave index is uniform; readfirstlane lets the compiler keep what
  // derives from it (buffer windows, LDS bases, tile offsets) scalar.
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int d_in = a.d_in, d_out = a.d_out;
  const int i0 = tile_m * BM, o0 = tile_n * BN;

  // This wave's loads of a stage: instruction i is q = NQW wave + i over the
  // stage's X rows then dY rows, 64 / (chunks per row) rows each.
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
  // Stage loads walk the token axis in order with running pointers. The
  // window of stage s covers only its own token rows (BK, the tail, or none),
  // so rows past T read as zero; its size fits 32 bits.
  const int nfull = int(T / BK), tail = int(T - int64_t(nfull) * BK);
  int g_stage = 0;
  const uint16_t* gx = X + i0;
  const uint16_t* gy = dY + o0;
  auto stage_bytes = [&](int dim, int c0) {
    const int rows = g_stage < nfull ? BK : (g_stage == nfull ? tail : 0);
    const int n = rows * dim - c0;               // c0 >= dim: a tile past the edge
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

  // Transpose-read addresses (bytes within a slot) of this lane's operands:
  // lane j of 16-lane group g reads 4 features of token row 8 (g / 2) + j / 4
  // (+ 16 for chunk 1, + 4 for the second read of an operand) at chunk
  // 4 blk + 2 (g % 2) + (j % 4) / 2 of the operand's 32-feature block blk.
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
  // Operand registers: two sets, alternating between consecutive 16-token
  // chunks. Set f holds TM operands of X^T then TN operands of dY.
  bf16x8_t frag[2][TM + TN];
  auto read_frags = [&](int f, const uint16_t* slot, int kk) {
#pragma unroll
    for (int m = 0; m < TM; ++m) frag[f][m] = operand(slot, fa[m] + kk * 16 * RBX, RBX);
#pragma unroll
    for (int n = 0; n < TN; ++n) frag[f][TM + n] = operand(slot, fb[n] + kk * 16 * RBY, RBY);
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
  // Interleave each MFMA with up to two transpose reads and one stage load so
  // the matrix core keeps issuing while LDS and memory work proceed.
  constexpr int NREAD = 2 * (TM + TN);
  auto interleave = [&](int loads) {
#pragma unroll
    for (int i = 0; i < TM * TN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                       // MFMA
      if (i < NREAD / 2) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);    // DS read
      if (i < loads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // VMEM read
    }
  };
  // The barrier orders LDS traffic between waves; the waits before it are
  // explicit, so neither the compiler nor the scheduler may move memory
  // operations across it.
  constexpr int kWaitMid = waitcnt_imm((L - 2) * NQW, 0);
  constexpr int kWaitFirst = waitcnt_imm((L - 1) * NQW, 15);
#define FORGE_STAGE_BARRIER(IMM)              \
  do {                                        \
    __builtin_amdgcn_sched_barrier(0);        \
    __builtin_amdgcn_s_waitcnt(IMM);          \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_s_barrier();             \
    asm volatile("" ::: "memory");            \
    __builtin_amdgcn_sched_barrier(0);        \
  } while (0)
  auto stage = [&](uint16_t* cur, uint16_t* nxt) {
    read_frags(1, cur, 1);
    mfmas(0);
    interleave(0);
    FORGE_STAGE_BARRIER(kWaitMid);
    load_stage(cur);                             // stage s + 4 into the freed slot
    read_frags(0, nxt, 0);
    mfmas(1);
    interleave(NQW);
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nk = int((T + BK - 1) / BK);
  if (nk > 0) {
    load_stage(sl.s0);
    load_stage(sl.s1);
    load_stage(sl.s2);
    load_stage(sl.s3);
    FORGE_STAGE_BARRIER(kWaitFirst);
    read_frags(0, sl.s0, 0);
    // Whole rounds of 4 stages keep one loop exit (so the accumulators keep
    // their registers). Up to three extra stages load zeros: a chunk of zero
    // products adds exactly +0 to an accumulator that is never -0 (it starts
    // at +0 and an exact-zero sum rounds to +0), so they change no bit.
    const int rounds = (nk + L - 1) / L;
    for (int r = 0; r < rounds; ++r) {
      stage(sl.s0, sl.s1);
      stage(sl.s1, sl.s2);
      stage(sl.s2, sl.s3);
      stage(sl.s3, sl.s0);
    }
  }
#undef FORGE_STAGE_BARRIER
  // The epilogue starts with a full barrier, which also waits for the loads
  // of the zero stages still in flight.
  uint16_t* ep = wave == 0 ? sl.s0 : wave == 1 ? sl.s1 : wave == 2 ? sl.s2 : sl.s3;
  if constexpr (is_adamw(EPI) && (EPI & EPI_BF16_STATE) != 0)
    epilogue_wide<C, EPI>(a, acc, W, S1, S2, i0, o0, wm, wn, lane, reinterpret_cast<float*>(ep));
  else
    epilogue<C, EPI>(a, acc, W, S1, S2, i0, o0, wm, wn, lane, reinterpret_cast<float*>(ep));
}

// The ring slots of a kernel, sized for its largest tile.
#define FORGE_DECLARE_SLOTS(ELEMS)                                                         \
  __shared__ __attribute__((aligned(1024))) uint16_t forge_s0[ELEMS], forge_s1[ELEMS],     \
      forge_s2[ELEMS], forge_s3[ELEMS];                                                    \
  const Slots ring{forge_s0, forge_s1, forge_s2, forge_s3}

template <class C, int EPI>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void wgrad_dense_kernel(WgradArgs a) {
  FORGE_DECLARE_SLOTS(C::STAGE);
  int e, tm, tn;
  map_tile(blockIdx.x, a.num_tiles, a.tiles_m, a.tiles_n, a.group_m, e, tm, tn);
  wgrad_tile<C, EPI>(a, a.X, a.dY, a.W, a.S1, a.S2, a.T, tm, tn, ring);
}

// Routed experts: the grid is laid out expert-major in the order of
// GroupTable::order (largest experts first); within an expert the usual tile
// walk applies. An expert with no rows still runs its epilogue (zero gradient).
template <class C, int EPI>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(C::OCC, C::OCC)))
void wgrad_grouped_kernel(WgradArgs a, GroupTable gt) {
  static_assert((EPI & EPI_WB_OUT) == 0, "the bf16 weight copy is a dense-call output");
  FORGE_DECLARE_SLOTS(C::STAGE);
  const int per_expert = a.tiles_m * a.tiles_n;
  const int slot = blockIdx.x / per_expert;
  const int e = gt.order[slot];
  int unused, tm, tn;
  map_tile(blockIdx.x - slot * per_expert, per_expert, a.tiles_m, a.tiles_n, a.group_m, unused,
           tm, tn);
  const int64_t r0 = gt.off[e], r1 = gt.off[e + 1];
  const int64_t state = int64_t(e) * a.d_out * a.d_in;
  float* const s2 = is_adamw(EPI) ? a.S2 + state : nullptr;   // SGD-m has no second buffer
  wgrad_tile<C, EPI>(a, a.X + r0 * a.d_in, a.dY + r0 * a.d_out, a.W + state, a.S1 + state, s2,
                     r1 - r0, tm, tn, ring);
}

// Persistent schedule. One workgroup per CU walks a list of items, each a full
// tile (BM x BN) or a half tile (BM x BN/2, the column halves of a full tile).
// The workers of a group share a contiguous range of R full tiles of the
// grouped tile order; round k of the group covers consecutive tiles, so the
// tiles running together share operand rows and columns in L2.
//   phase 0: rounds of ng full tiles, then the remainder r: as 2r half tiles
//            when 2r <= ng (the round takes half a tile's time), else as r
//            full tiles.
//   phase 1: the same after a first round of ng half tiles (ng/2 full tiles).
// Groups in phase 1 run half a tile out of step with groups in phase 0, so
// only half the chip is in the HBM-bound optimizer epilogue at any time, and
// a remainder of half a round per worker (3.5 tiles per CU, say) is balanced
// exactly. Returns false when worker j has no item k.
__host__ __device__ inline bool schedule_item(int k, int j, int ng, int R, int phase, int& tile,
                                              int& half) {
  int pos = 0;
  if (phase) {
    if (k == 0) {
      tile = j >> 1;
      half = j & 1;
      return true;
    }
    --k;
    pos = ng >> 1;
  }
  const int F = R - pos, nf = F / ng, r = F - nf * ng;
  if (k < nf) {
    tile = pos + k * ng + j;
    half = -1;
    return true;
  }
  if (k > nf) return false;
  pos += nf * ng;
  if (2 * r <= ng) {
    if (j >= 2 * r) return false;
    tile = pos + (j >> 1);
    half = j & 1;
    return true;
  }
  if (j >= r) return false;
  tile = pos + j;
  half = -1;
  return true;
}

// The phase of XCD `xcd` holding R tiles for ng workers: odd XCDs run half a
// tile behind when every worker has at least one full tile.
__host__ __device__ inline int schedule_phase(int xcd, int R, int ng) {
  return (xcd & 1) && R >= ng ? 1 : 0;
}

// Persistent dense kernel over the schedule above. The grid is 8 * nw
// workgroups (nw per XCD, even); each XCD is one group of nw workers over its
// contiguous range of the grouped tile order. Full tiles use CF, half tiles
// CH (same BM and threads, half the BN); each element still takes its tokens
// in ascending 16-token chunks through one accumulator, so the result is
// bitwise that of any other tiling.
template <class CF, class CH, int EPI>
__global__ __launch_bounds__(CF::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void wgrad_persistent_kernel(WgradArgs a) {
  static_assert(CF::THREADS == CH::THREADS && CF::BM == CH::BM && CF::BN == 2 * CH::BN,
                "half tiles must split the full tile's columns");
  FORGE_DECLARE_SLOTS(CF::STAGE);
  const int b = blockIdx.x, xcd = b & 7, j = b >> 3, nw = gridDim.x >> 3;
  // This XCD's contiguous range of the grouped tile order.
  const int per = a.num_tiles >> 3, rem = a.num_tiles & 7;
  const int start = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  const int R = per + (xcd < rem ? 1 : 0);
  const int phase = schedule_phase(xcd, R, nw);
  for (int k = 0;; ++k) {
    int tile, half;
    if (!schedule_item(k, j, nw, R, phase, tile, half)) break;
    int tm, tn;
    grouped_walk(start + tile, a.tiles_m, a.tiles_n, a.group_m, tm, tn);
    if (half < 0)
      wgrad_tile<CF, EPI>(a, a.X, a.dY, a.W, a.S1, a.S2, a.T, tm, tn, ring);
    else
      wgrad_tile<CH, EPI>(a, a.X, a.dY, a.W, a.S1, a.S2, a.T, tm, 2 * tn + half, ring);
    __syncthreads();                 // the next tile's loads reuse the slots
  }
}

}  // namespace forge
