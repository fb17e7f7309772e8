#pragma once
// The GEMM kernel template (bf16 and E4M3 MFMA) for gfx950 with fused tensor-parallel epilogues.
//
// Every linear of the layer is C = A . B^T with both operands K-contiguous:
// A = activations [M x K], B = weights stored [out x in] = [N x K] (the
// F.linear layout of the pages' ColumnParallelLinear / RowParallelLinear
// pseudo-code, "ai阅读megatron").  One kernel template covers
//   MODE_COL    : column-parallel output, bf16(act(acc + bias)), act in {none, erf-GeLU}
//   MODE_SWIGLU : column-parallel gate+up, bf16(silu(gate + bg) * (up + bu))
//   MODE_ROW    : row-parallel partial in fp32 (Yacc = P or Yacc += P), and on the
//                 last shard bf16(Yacc + bias): the local form of Y = sum_i Y_i
// and a grouped variant (MoE experts, SWIGLU fc1 and ROW fc2 with fp32 row
// outputs) whose row tiles are laid over the ragged per-expert row ranges read
// from device memory.
//
// Design (gfx950, CDNA4):
//  * A tile configuration (Cfg) fixes the block tile BM x BN, the wave grid, the
//    K step BK and the number NS of LDS stages.  Each wave owns a
//    (BM/WAVES_M) x (BN/WAVES_N) tile of v_mfma_f32_32x32x16_bf16 fragments
//    accumulated in fp32 (the 32x32x16 form sustains ~97% of the dense bf16
//    rate on gfx950; the 16x16x32 form measured ~85%).  The large tile is
//    256 x 256 with 8 waves (two per SIMD, 128 accumulators each).
//  * Operands are swapped in the MFMA (weights as the first operand) so a
//    lane's accumulators hold runs of 4 consecutive output columns of one row.
//  * Global -> LDS: buffer_load_dwordx4 ... lds (direct to LDS, no VGPR round
//    trip, no ds_write) into an NS-deep ring of LDS stages, NS - 1 K steps
//    ahead of the MFMAs, one barrier per K step.  Each stage is its own LDS
//    variable so the compiler sees that a DMA into one stage does not alias
//    the fragment reads of another.  Buffer resources make out-of-range rows
//    read as zero without faulting, and the K position is a scalar offset, so
//    the loop has no vector address arithmetic.  (With one step of lead the
//    DMA latency, ~2-3K cycles under load, was exposed on every step.)
//  * LDS rows are BK * 2 bytes; 16-byte chunks are XOR-swizzled per row so the
//    fragment reads (16 lanes read one chunk of 16 consecutive rows) hit
//    distinct banks of the 64-bank (256 B per cycle) LDS.
//  * bf16 epilogues stage each wave's tile through LDS and store whole rows.
//  * Tile order is XCD-aware: consecutive workgroup ids land on different XCDs
//    (8 L2 slices), so ids are remapped to give each XCD a contiguous band of
//    tiles, grouped GROUP_M rows at a time for A/B panel reuse in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "gemm.h"

namespace mtp {

// CU count of the current device (gemm.hip)
int cu_count();

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
// (the epilogue's output stores are nontemporal: the launch never reads its output back, and the hint keeps
// the output from settling in the L2; 1-5% faster at the shard shapes, most with fp32 partials)
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int NS_, bool EARLY_, int NSB_ = 0>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, BK = BK_, NS = NS_;
  // Split ring (NSB = NS + 1 with NS = 2, without EARLY): the B operand's tiles get a ring of NSB stages of
  // their own, the A operand's keep NS, where the LDS cannot hold NS + 1 stages of both (256 x 192: 3 x 56 KB
  // does not fit, 2 x 32 + 3 x 24 KB does).  Each B tile is loaded two steps ahead of its use, and so is each
  // A tile, into its own stage right after a barrier inside the step that reads it (see step_spread_ab).
  // (A fourth B stage would add no lead: loads retire in issue order, so the wait for the A tile of step
  // kt + 1 also waits for every B tile issued before it.)
  static constexpr int NSB = NSB_ ? NSB_ : NS;
  static constexpr bool AB = NSB != NS;
  static constexpr int RING = AB ? NS * NSB : NS;  // K steps per loop iteration (each stage a compile-time choice)
  // EARLY: the first fragments of step k + 1 are read during the last MFMAs of step k (the barrier ending a
  // step then makes the stage two steps ahead visible, so the ring needs one more stage for the same lead)
  static constexpr bool EARLY = EARLY_;
  static constexpr int LEAD = EARLY ? 2 : 1;
  static constexpr int NWAVES = WAVES_M * WAVES_N, NT = 64 * NWAVES;
  static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;             // 32 x 32 MFMA tiles per wave
  static constexpr int CPR = BK / 8;                           // 16-byte chunks per LDS row
  static constexpr int RPL = 256 / (2 * BK);                   // LDS rows per 256-byte bank line
  static constexpr int ROWS_PER_DMA = 64 / CPR;                // rows one 64-lane DMA instruction fills
  static constexpr int GA = BM / ROWS_PER_DMA, GB = BN / ROWS_PER_DMA;  // DMA groups per stage (A, B)
  // DMA instructions per wave per stage: group g goes to wave g % NWAVES; when the groups do not divide
  // evenly, the spare slots load nothing (out of range) into a scratch LDS block, so every wave issues the
  // same number of DMAs and the wait counts stay uniform.
  static constexpr int D = (GA + GB + NWAVES - 1) / NWAVES;
  static constexpr bool SPARE = (GA + GB) % NWAVES != 0;
  static constexpr int STAGE = (BM + BN) * BK;                 // elements per LDS stage
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(NS >= 2 + LEAD - 1 && NS <= 5, "LDS stages");
  static_assert(NWAVES % 4 == 0, "whole waves per SIMD");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32 x 32 fragments");
  static_assert(BM % ROWS_PER_DMA == 0 && BN % ROWS_PER_DMA == 0, "DMA groups");
  static_assert((AB ? (NS * BM + NSB * BN) * BK * 2 : NS * STAGE * 2) + (SPARE ? 1024 : 0) <= 160 * 1024,
                "LDS capacity");
  static_assert(!AB || (!EARLY && NS == 2 && NSB == 3 && GA % NWAVES == 0 && GB % NWAVES == 0),
                "split ring: two A stages, three B stages, whole A and B slots per wave");
};

// Element offset of (row, 16-byte chunk) in an LDS stage: rows of BK elements, chunks permuted by XOR with
// (row / RPL) & (CPR - 1).  A fragment read has 16 lanes read one chunk of 16 consecutive rows; the RPL rows
// that share a 256-byte bank line differ in their permutation, so those 16 reads hit 16 distinct bank groups.
template <class C>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * C::BK + ((chunk ^ ((row / C::RPL) & (C::CPR - 1))) << 3);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats to packed bf16 (one v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Exact-erf GeLU, gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)).  erf is evaluated with Abramowitz &
// Stegun 7.1.26 (|error| <= 1.5e-7 absolute, far below bf16 resolution): for z >= 0,
// 1 - erf(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2), t = 1 / (1 + p z).  With z = |x| / sqrt 2
// and P = (a1 t + .. + a5 t^5) / 2 this gives Phi(x) = 1 - P e (x >= 0) and P e (x < 0), e = exp(-x^2 / 2),
// so gelu(x) = max(x, 0) - |x| P e for both signs, with no cancellation for negative x.  The constants
// below are p / sqrt 2, a_i / 2 and -log2(e) / 2 (e via exp2); this is an epilogue that runs once per
// output element, so every operation counts: 12 VALU operations and 2 transcendentals.
__device__ __forceinline__ float gelu_erf(float x) {
  const float e = __builtin_amdgcn_exp2f(x * x * -0.72134752044448170368f);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164188773f, fabsf(x), 1.0f));
  const float P = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 0.5307027145f, -0.7265760135f), 0.7107068705f),
                                     -0.142248368f), 0.127414796f);
  return fmaf(-e, fabsf(x) * P, x > 0.0f ? x : 0.0f);
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Workgroup ids alternate over the 8 XCDs (each with its own L2); remapped so that each XCD gets a
// contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  return (total & 7) == 0 ? (id & 7) * (total >> 3) + (id >> 3) : id;
}
// Tile of logical id `id`: GROUP_M tile rows at a time, column-major inside the group, so consecutive ids
// share A and B panels.
__device__ __forceinline__ void tile_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  const int per_group = GROUP_M * tiles_n;
  const int g = id / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int r = id - g * per_group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// Buffer resource (raw, stride 0) over `bytes` bytes at `base`.  The fields are made explicitly uniform:
// a resource the compiler cannot prove uniform is wrapped in a per-lane "waterfall" loop at every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// Store 4 consecutive bf16 outputs (8 bytes) or the in-range part of them.
__device__ __forceinline__ void store4_bf16(uint16_t* dst, const float v[4], int valid) {
  if (valid >= 4) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < valid) dst[r] = to_bf16(v[r]);
  }
}

// AT / BT: the operand is stored with the contraction index along its rows ([K x M] for A, [K x N] for B;
// the backward GEMMs: dX = dY W reads W that way, dW = dY^T X reads both).  Such a tile is kept in LDS as
// [BK rows][BM or BN columns] and its MFMA fragments are read with ds_read_b64_tr_b16, the gfx950 LDS
// transpose load: 16 lanes each name 4 consecutive columns of one row, and lane i receives column i of
// four consecutive rows.
// LDS slot of global 16-byte chunk c in row r of a row-major-K tile [BK x BX]: rows r and r + 1 .. r + 3
// place their chunks 4 slots apart (XOR for a power-of-two number of chunks per row, rotation otherwise),
// so the 32 lanes of a half-wave of transpose reads (four rows, 64 contiguous bytes each) hit 64 distinct
// banks for row pitches of 256, 384 and 512 bytes.
template <int BX>
__device__ __forceinline__ int t_slot(int c, int r) {
  constexpr int cpr = BX / 8;
  if constexpr ((cpr & (cpr - 1)) == 0) return c ^ (4 * r);
  else return (c + 4 * r) % cpr;
}

template <class C, int MODE, bool GROUPED, bool KFULL, bool SPLIT, bool AT = false, bool BT = false, int EPI = EPI_PLAIN,
          bool F8 = false>
__global__ __launch_bounds__(C::NT) void gemm_kernel(GemmParams p_arg) {
  // A private copy of the parameters: read once into scalar registers, rather than reloaded from the
  // kernel argument segment (each reload waits on the LDS/scalar counter) wherever a field is used.
  GemmParams p = p_arg;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, NS = C::NS, WAVES_N = C::WAVES_N, NWAVES = C::NWAVES;
  constexpr int TM = C::TM, TN = C::TN, FM = C::FM, FN = C::FN, CPR = C::CPR, RPL = C::RPL;
  constexpr int D = C::D, GA = C::GA, ROWS_PER_DMA = C::ROWS_PER_DMA;
  static_assert(MODE != MODE_SWIGLU || TN % 64 == 0, "gate/up fragment pairs");
  static_assert(!(AT || BT) || ((BK == 32 || C::AB) && !GROUPED && (MODE == MODE_COL || MODE == MODE_ROW)),
                "row-major-K operands: K step 32 or the split ring, plain column/row epilogues");
  static_assert(!AT || BM == 128 || BM == 256, "A rows of 256 or 512 bytes");
  static_assert(!BT || BN == 128 || BN == 192 || BN == 256, "B rows of 256, 384 or 512 bytes");
  static_assert(EPI == EPI_PLAIN || (!GROUPED && (EPI == EPI_NORM ? (MODE == MODE_COL || MODE == MODE_SWIGLU)
                                                                    : MODE == MODE_ROW)),
                "norm epilogue on column products, bias-dropout-add on row products");
  // E4M3 operands: the same bytes per LDS row (BK = 32 two-byte units = 64 one-byte codes), one
  // 32 x 32 x 64 MFMA per K step instead of two 32 x 32 x 16 ones
  static_assert(!F8 || ((BK == 32 || C::AB) && !AT && !BT && !GROUPED && EPI == EPI_PLAIN), "E4M3: plain K-major tiles");
  constexpr int NB_OUT = MODE == MODE_SWIGLU ? BN / 2 : BN;  // output columns per tile

  // one LDS variable per stage (see the design notes); unused ones are a token 16 bytes.  In the split ring
  // lds0 / lds1 hold the A tiles and ldsb0 .. ldsb2 the B tiles.
  constexpr int SA = C::AB ? BM * BK : C::STAGE;
  constexpr int SB = C::AB ? BN * BK : 8;
  __shared__ __attribute__((aligned(16))) uint16_t lds0[SA];
  __shared__ __attribute__((aligned(16))) uint16_t lds1[SA];
  __shared__ __attribute__((aligned(16))) uint16_t lds2[NS > 2 ? SA : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds3[NS > 3 ? SA : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds4[NS > 4 ? SA : 8];
  __shared__ __attribute__((aligned(16))) uint16_t ldsb0[SB];
  __shared__ __attribute__((aligned(16))) uint16_t ldsb1[SB];
  __shared__ __attribute__((aligned(16))) uint16_t ldsb2[C::NSB > 2 ? SB : 8];
  __shared__ __attribute__((aligned(16))) uint16_t lds_spare[C::SPARE ? 512 : 8];  // dropped unless used
  auto stage_buf = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return lds0;
    else if constexpr (i == 1) return lds1;
    else if constexpr (i == 2) return lds2;
    else if constexpr (i == 3) return lds3;
    else return lds4;
  };
  auto bstage_buf = [&](auto I) -> uint16_t* {
    constexpr int i = decltype(I)::value;
    if constexpr (i == 0) return ldsb0;
    else if constexpr (i == 1) return ldsb1;
    else return ldsb2;
  };
  // Wave w's private epilogue staging region of R elements, carved from the stage buffers in order (the
  // main loop has drained by then).
  auto stage_region = [&](auto RC) -> uint16_t* {
    constexpr int R = decltype(RC)::value;
    const int w = threadIdx.x >> 6;
    if constexpr (!C::AB) {
      constexpr int WPS = C::STAGE / R;
      static_assert(WPS >= 1 && (NWAVES + WPS - 1) / WPS <= NS, "staging fits");
      const int si = w / WPS;
      return (si == 0 ? lds0 : si == 1 ? lds1 : si == 2 ? lds2 : si == 3 ? lds3 : lds4) + (w % WPS) * R;
    } else {
      constexpr int PA = SA / R, PB = SB / R;  // regions per A / B buffer
      static_assert(PA >= 1 && PB >= 1 && NS * PA + C::NSB * PB >= NWAVES, "staging fits");
      if (w < NS * PA) return (w / PA == 0 ? lds0 : lds1) + (w % PA) * R;
      const int w2 = w - NS * PA, si = w2 / PB;
      return (si == 0 ? ldsb0 : si == 1 ? ldsb1 : ldsb2) + (w2 % PB) * R;
    }
  };

  __shared__ int sk_flag;
  // K steps, rounded up to a multiple of NS: the loop body covers NS steps (one per LDS stage, each stage a
  // compile-time choice) and has no branches, so the compiler's wait counts stay exact.  With KFULL the
  // step count is a multiple of NS and every chunk is in range; otherwise chunks at or past K read as zero,
  // so padding steps multiply zeros.  (The split ring's loop covers RING = 6 steps; the split schedule counts
  // in such passes and KTS rounds up to one; the steps of a last partial pass run after the loop, each behind
  // a uniform branch, and none past step KT - 1.)
  const int KT = (p.K + BK - 1) / BK;
  constexpr int RING = C::RING;
  const int KTS = (KT + RING - 1) / RING * RING;
  const int tiles_m = (p.M + BM - 1) / BM, tiles_n = (p.Nout + NB_OUT - 1) / NB_OUT;
  // split schedule (SPLIT only): each tile's RI ring passes in S chunks, partial sums of tile t in slots
  // t * S .. t * S + S - 1
  const int RI = KTS / RING;
  const int G = gridDim.x;
  const int S = p.sk_chunks;
  auto slot_of = [&](int c, int t) { return t * S + c; };

  // ---- one tile: rows m0 .. m0 + BM - 1 of the row group at row_base, K steps kt0 .. kt1 - 1.  With
  // SPLIT and sk_partial, the K range is chunk sk_which_chunk of the tile's and the partial sums of all
  // workgroups on the tile are added before the epilogue (see the split schedule below): sk_tile indexes
  // the tile's arrival counter, sk_wtile its slots in the workspace (split tiles only).
  auto run_tile = [&](int tm, int tn, int row_base, int rows, const uint16_t* __restrict__ B, int kt0, int kt1,
                      int sk_tile, int sk_wtile, int sk_which_chunk, int sk_first, int sk_last, bool sk_partial) {
  const int m0 = tm * BM;  // relative to row_base
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * TM, wn0 = (wave % WAVES_N) * TN;

  // ---- global sources: raw buffer loads.  Each operand gets a buffer resource whose base is this tile's
  // first row (the whole gather source for gathered rows) and whose size ends at the operand's last row:
  // a load past it returns zero and cannot fault.  Per-lane byte offsets are fixed across K; the K position
  // is a scalar offset, so the loop issues loads with no vector address arithmetic.  Rows past the end of
  // a tile only feed outputs that are never stored, so they need no masking; only K chunks at or past K
  // must read as zero (the KFULL = false variant redirects them out of range).
  constexpr uint32_t kOOB = 0x7FFFFFF0u;
  const uint16_t* a_base;
  int64_t a_extent;
  if constexpr (AT) {  // [K x M]: the tile's columns m0 .. m0 + BM - 1 of every row
    a_base = p.A + m0;
    a_extent = (int64_t)p.K * p.lda - m0;
  } else if (p.a_rows) {
    a_base = p.A;
    a_extent = p.a_src_rows * p.lda;
  } else {
    a_base = p.A + (int64_t)(row_base + m0) * p.lda;
    a_extent = (p.a_src_rows - (row_base + m0)) * p.lda;
  }
  const int nbase = tn * NB_OUT;
  const uint16_t* b_base = BT ? B + nbase : B + (int64_t)nbase * p.ldb;
  const int64_t b_extent = BT ? (int64_t)p.K * p.ldb - nbase
                              : ((MODE == MODE_SWIGLU ? p.up_offset : 0) + p.Nout - nbase) * p.ldb;
  // (integer clamps written out: the device min() overload for 64-bit integers goes through double, and a
  // converted value lands in a vector register, which turns every buffer load into a waterfall loop)
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_base, 2 * a_extent < (int64_t)kOOB ? 2 * a_extent : (int64_t)kOOB);
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(b_base, 2 * b_extent < (int64_t)kOOB ? 2 * b_extent : (int64_t)kOOB);
  // Direct-to-LDS loads: one buffer_load_dwordx4 ... lds moves 64 lanes x 16 B = ROWS_PER_DMA LDS rows,
  // lane l filling row (l / CPR), chunk (l % CPR) of its group.  The LDS layout is swizzled (see swz), so
  // each lane loads the global chunk that lands at its slot.  Groups 0 .. GA-1 are rows of A, the next GB
  // are rows of B (stored right after A in the stage); slot j of a wave carries group j * NWAVES + wave.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = lane / CPR;
  uint32_t d_off[D];
  int d_kc[D];  // K element offset of each lane's chunk
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const int g = j * NWAVES + wave_u;
    const int r = ROWS_PER_DMA * g + lrow - (g < GA ? 0 : BM);  // row within A or within B
    const int c = (lane % CPR) ^ ((r / RPL) & (CPR - 1));
    d_kc[j] = 8 * c;
    // a row-major-K operand: instruction g fills elements 512 g .. 512 g + 511 of the row-major [BK x BX] tile,
    // lane l the 16-byte slot at element 512 g + 8 l: row rk, slot s, holding global chunk t_chunk(s, rk) (see
    // t_slot); its K position is the row, and chunks that start past the matrix width load nothing
    auto t_off = [&](int gg, auto BXC, int64_t ld, int x0, int width) {
      constexpr int BX = decltype(BXC)::value, cpr = BX / 8;
      const int e = 512 * gg + 8 * lane;
      const int rk = e / BX, slot = (e % BX) / 8;
      const int cc = (cpr & (cpr - 1)) == 0 ? slot ^ (4 * (rk & 3)) : (slot + cpr - 4 * (rk & 3)) % cpr;
      d_kc[j] = rk;
      return x0 + 8 * cc < width ? 2u * (uint32_t)(rk * ld + 8 * cc) : kOOB;
    };
    if (g < GA && AT) {
      d_off[j] = t_off(g, std::integral_constant<int, BM>{}, p.lda, m0, p.M);
    } else if (g >= GA && g < GA + C::GB && BT) {
      d_off[j] = t_off(g - GA, std::integral_constant<int, BN>{}, p.ldb, nbase, p.Nout);
    } else if (g < GA) {
      if (p.a_rows) {
        const int m = m0 + r;
        d_off[j] = m < rows ? 2u * (uint32_t)((int64_t)p.a_rows[row_base + m] * p.lda + 8 * c) : kOOB;
      } else {
        d_off[j] = 2u * (uint32_t)(r * p.lda + 8 * c);
      }
    } else if (g < GA + C::GB) {
      int n = r;
      if constexpr (MODE == MODE_SWIGLU) {
        const int g32 = r >> 5;
        n = 32 * (g32 >> 1) + (r & 31) + ((g32 & 1) ? (int)p.up_offset : 0);
      }
      d_off[j] = 2u * (uint32_t)(n * p.ldb + 8 * c);
    } else {
      d_off[j] = kOOB;  // spare slot
    }
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // The scalar offset is not part of the hardware range check (only the per-lane offset is), so it stays
  // inside the rows: a prefetch past the last K step re-reads step 0 into a stage that is never consumed
  // (KFULL) or is redirected out of range per lane (!KFULL, reading zeros).
  auto dma_stage = [&](int k0, uint16_t* sbuf) {
    // the K position: a column offset for K-major operands, a row offset for row-major-K ones
    const int soff_a = k0 < p.K ? (AT ? 2 * k0 * (int)p.lda : 2 * k0) : 0;
    const int soff_b = k0 < p.K ? (BT ? 2 * k0 * (int)p.ldb : 2 * k0) : 0;
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int g = j * NWAVES + wave_u;  // uniform
      uint32_t vo = d_off[j];
      if constexpr (!KFULL) vo = k0 + d_kc[j] < p.K ? vo : kOOB;
      uint16_t* dst = sbuf + g * ROWS_PER_DMA * BK;
      if constexpr (C::SPARE) dst = g < GA + C::GB ? dst : lds_spare;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(g < GA ? a_rsrc : b_rsrc, (lds_ptr)dst, 16, vo, g < GA ? soff_a : soff_b,
                                               0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // 32 x 32 x 16 fragments: lane holds row (lane & 31), k = 8 * (lane >> 5) .. +7 of a 16-wide k step.
  // Two fragment sets alternate: the set of the next k step is read while the MFMAs of this one run.
  const int fr = lane & 31, fk = lane >> 5;
  using frag_t = std::conditional_t<F8, i32x8, bf16x8>;
  frag_t fa[2][FM], fb[2][FN];
  // Fragment of a [BK x BX] row-major-K tile: lane l (16-lane group g = l / 16, i = l % 16) names row
  // 16 ks + 8 (l / 32) + 4 r + i / 4 and columns x0 + 16 (g % 2) + 4 (i % 4) .. + 3; the transpose load then
  // gives it column x0 + (l % 32) of rows 16 ks + 8 (l / 32) + 4 r .. + 3, i.e. k = 8 (l / 32) + 4 r .. + 3 of
  // its MFMA operand row.  Two loads (r = 0, 1) make the 8 k values.  Rows r and r + 1 .. r + 3 use chunks
  // XOR 4 (row % 4), so the 32 lanes of a half-wave hit 64 distinct banks.
  typedef short short4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) short4_t* lds_s4;
  auto read_t = [&](const uint16_t* s, auto BXC, int x0, int ks) -> bf16x8 {
    constexpr int BX = decltype(BXC)::value;
    const int i = lane & 15, h = lane >> 5;
    const int x = x0 + 16 * ((lane >> 4) & 1) + 4 * (i & 3);
    short4_t v[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int k = 16 * ks + 8 * h + 4 * r + (i >> 2);
      const int off = k * BX + (t_slot<BX>(x >> 3, i >> 2) << 3) + (x & 7);
      v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(s + off));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // E4M3 fragment of MFMA k step ks: lane holds row (lane & 31) and the 32 codes of 16-byte chunks
  // 4 ks + 2 (lane / 32) and 4 ks + 2 (lane / 32) + 1 (a 64-code MFMA step per 4 chunks of the LDS row).  Both
  // operands use the same k assignment, so the MFMA's sum over k is the product's whatever order the hardware
  // pairs the codes in.
  auto read_f8 = [&](const uint16_t* s, int row, int ks) -> i32x8 {
    const bf16x8 lo = *reinterpret_cast<const bf16x8*>(s + swz<C>(row, 4 * ks + 2 * fk));
    const bf16x8 hi = *reinterpret_cast<const bf16x8*>(s + swz<C>(row, 4 * ks + 2 * fk + 1));
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13,
                                                             14, 15));
  };
  auto read_frags2 = [&](const uint16_t* sA, const uint16_t* sB, int ks, auto SET) {
    constexpr int q = decltype(SET)::value;
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[q][i] = read_f8(sA, wm0 + 32 * i + fr, ks);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[q][j] = read_f8(sB, wn0 + 32 * j + fr, ks);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (AT) fa[q][i] = read_t(sA, std::integral_constant<int, BM>{}, wm0 + 32 * i, ks);
        else fa[q][i] = *reinterpret_cast<const bf16x8*>(sA + swz<C>(wm0 + 32 * i + fr, 2 * ks + fk));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (BT) fb[q][j] = read_t(sB, std::integral_constant<int, BN>{}, wn0 + 32 * j, ks);
        else fb[q][j] = *reinterpret_cast<const bf16x8*>(sB + swz<C>(wn0 + 32 * j + fr, 2 * ks + fk));
      }
    }
  };
  auto read_frags = [&](const uint16_t* sbuf, int ks, auto SET) { read_frags2(sbuf, sbuf + BM * BK, ks, SET); };
  auto mma = [&](auto SET) {
    constexpr int q = decltype(SET)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        if constexpr (F8)  // formats 0 / 0: E4M3 x E4M3, no block scales
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[q][j], fa[q][i], acc[i][j], 0, 0, 0, 0, 0, 0);
        else
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[q][j], fa[q][i], acc[i][j], 0, 0, 0);
  };
  constexpr int KS = F8 ? BK / 32 : BK / 16;  // MFMA k steps per K step (32 x 32 x 64 codes, 32 x 32 x 16 bf16)
  static_assert(!C::EARLY || (NS * KS) % 2 == 0, "fragment sets alternate consistently across the ring");
  // vmcnt(n): wait until at most n of this wave's DMA instructions are outstanding (expcnt, lgkmcnt free).
  // The barrier ending step kt makes stage kt + LEAD visible: the DMAs newer than that stage may stay out.
  constexpr int kNewer = (NS - 1 - C::LEAD) * D;
  static_assert(kNewer >= 0 && kNewer < 64, "vmcnt range");
  constexpr int kWaitNext = 0x0F70 | (kNewer & 15) | ((kNewer >> 4) << 14);
  // The barrier between steps: this wave's DMA of stage kt + LEAD has landed (vmcnt), every fragment read
  // of the stage about to be overwritten has been consumed by an MFMA, and the waves meet.  A
  // __syncthreads() would add a release fence, which waits for every outstanding DMA (vmcnt(0)) and so
  // drains the whole ring; the raw s_barrier between compiler-level memory fences keeps later DMAs in flight.
  auto ring_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitNext);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // One K step on stage I: start the DMA of step kt + NS - 1 into the stage consumed last step (every wave
  // passed the barrier after reading it), run this step's MFMAs (with EARLY, the last k step reads the first
  // fragments of stage kt + 1, visible since the previous barrier), then the barrier.
  auto step = [&](auto I, int kt) {
    constexpr int i = decltype(I)::value;
    uint16_t* cur = stage_buf(std::integral_constant<int, i>{});
    dma_stage((kt + NS - 1) * BK, stage_buf(std::integral_constant<int, (i + NS - 1) % NS>{}));
    __builtin_amdgcn_sched_barrier(0);  // keep the DMA issue at the top: the scheduler would sink it
    [&]<int... S>(std::integer_sequence<int, S...>) {
      ([&] {
        constexpr int ks = S;
        constexpr int g = i * KS + ks;  // k step index within the ring pass: fixes the fragment set
        if constexpr (C::EARLY) {
          if constexpr (ks + 1 < KS)
            read_frags(cur, ks + 1, std::integral_constant<int, (g + 1) & 1>{});
          else
            read_frags(stage_buf(std::integral_constant<int, (i + 1) % NS>{}), 0,
                       std::integral_constant<int, (g + 1) & 1>{});
          mma(std::integral_constant<int, g & 1>{});
          // issue order: one fragment read, then its share of the MFMAs, and so on, so the reads of the next
          // set are spread over this set's MFMAs instead of being bunched (or sunk next to their first use)
          [&]<int... R>(std::integer_sequence<int, R...>) {
            constexpr int NR = FM + FN, NM = FM * FN;
            ((__builtin_amdgcn_sched_group_barrier(0x100, F8 ? 2 : 1, 0),  // one fragment's LDS reads
              __builtin_amdgcn_sched_group_barrier(0x008, (NM * (R + 1)) / NR - (NM * R) / NR, 0)), ...);  // MFMAs
          }(std::make_integer_sequence<int, FM + FN>{});
          __builtin_amdgcn_sched_barrier(0);
        } else {
          read_frags(cur, ks, std::integral_constant<int, 0>{});
          mma(std::integral_constant<int, 0>{});
        }
      }(), ...);
    }(std::make_integer_sequence<int, KS>{});
    ring_barrier();
  };
  // ---- split ring (C::AB): A tiles in NS = 2 stages, B tiles in NSB = 3, with a barrier inside each step.
  // Step kt reads A stage kt % 2 and B stage kt % 3.  Its B slots (the B tile of step kt + 2, into the B stage
  // consumed in step kt - 1) are spread over the first half of its MFMAs.  Its fragment reads of the last k
  // step are issued during the MFMAs of the one before; once every wave's reads have returned (lgkmcnt(0)) and
  // the waves meet at the mid-step barrier, no wave reads A stage kt % 2 again, and the A slots reload it with
  // the A tile of step kt + 2 during the MFMAs of the last k step.  Both operands thus load two steps ahead:
  // the A tile lands within ~1.25 steps (instead of within the rest of a step, had it waited for the stage
  // consumed in step kt - 1), enough for an activation read from HBM rather than from cache.  At the end of
  // step kt everything issued in step kt - 1 (the tiles of step kt + 1) has landed, while the D loads of step
  // kt may stay in flight (loads complete in issue order).  The MFMA order per accumulator is unchanged.
  // One barrier per step (ONEBAR): the mid-step barrier also waits for the tiles of step kt + 1 (everything
  // older than this step's B slots, vmcnt(JB)); no wave then reads A stage kt % 2 or B stage kt % 3 again, and
  // step kt + 1's stages are visible, so the end-of-step barrier has nothing left to order: it goes, and the
  // fragments of step kt + 1's first k step are read during the MFMAs of step kt's last one.  The A tile then
  // has about one step to land instead of ~1.25, which the 256 x 256 tile's longer step covers; with the
  // 256 x 192 tile (three quarters of the MFMA time per step) and with split-K pieces the loads arriving later
  // cost more than the barrier, cold.
  constexpr bool ONEBAR = C::AB && C::BM == 256 && C::BN == 256 && !SPLIT;
  constexpr int JA = C::AB ? GA / NWAVES : D, JB = D - JA;
  constexpr int kWaitAB = 0x0F70 | (D & 15) | ((D >> 4) << 14);  // vmcnt(D)
  // lgkmcnt(0), and with ONEBAR vmcnt(JB)
  constexpr int kWaitMid = ONEBAR ? 0x0070 | (JB & 15) | ((JB >> 4) << 14) : 0xC07F;
  auto ring_barrier_ab = [&]() {
    __builtin_amdgcn_s_waitcnt(kWaitAB);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto mid_barrier_ab = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitMid);  // lgkmcnt(0): this wave's fragment reads have returned
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  auto dma_slot_ab = [&](auto J, int k0, uint16_t* sA, uint16_t* sB) {
    constexpr int j = decltype(J)::value;
    constexpr bool is_a = j < JA;
    // the K position: a column offset for K-major operands, a row offset for row-major-K ones
    constexpr bool tr = is_a ? AT : BT;
    const int soff = k0 < p.K ? (tr ? 2 * k0 * (int)(is_a ? p.lda : p.ldb) : 2 * k0) : 0;
    const int g = j * NWAVES + wave_u;  // uniform
    uint32_t vo = d_off[j];
    if constexpr (!KFULL) vo = k0 + d_kc[j] < p.K ? vo : kOOB;
    uint16_t* dst = is_a ? sA + g * ROWS_PER_DMA * BK : sB + (g - GA) * ROWS_PER_DMA * BK;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_rsrc : b_rsrc, (lds_ptr)dst, 16, vo, soff, 0, 0);
  };
  // One K step of the split ring on A stage IA and B stage IB.  Issue order: an MFMA, then (while this k
  // step's reads remain) one fragment read, then (after odd MFMAs of the first k steps) one B slot; in the last
  // k step, after the mid-step barrier, one A slot after each of its first MFMAs (and with ONEBAR one of the
  // next step's first fragment reads after each of its MFMAs).
  auto step_spread_ab = [&](auto IA, auto IB, int kt) {
    constexpr int ia = decltype(IA)::value, ib = decltype(IB)::value;
    uint16_t* curA = stage_buf(std::integral_constant<int, ia>{});
    const uint16_t* curB = bstage_buf(std::integral_constant<int, ib>{});
    uint16_t* nxtB = bstage_buf(std::integral_constant<int, (ib + C::NSB - 1) % C::NSB>{});
    const int k2 = (kt + 2) * BK;
    constexpr int NM = FM * FN;
    static_assert(C::NSB == 3, "the B tile of step kt + 2 goes to the stage consumed in step kt - 1");
    static_assert(2 * JB <= (KS - 1) * NM && JA <= NM, "every DMA slot finds an MFMA");
    static_assert(!ONEBAR || KS % 2 == 0, "the last k step uses fragment set 1, the next step's first one set 0");
    if constexpr (!ONEBAR) read_frags2(curA, curB, 0, std::integral_constant<int, 0>{});
    [&]<int... S>(std::integer_sequence<int, S...>) {
      ([&] {
        constexpr int ks = S;
        constexpr bool last = ks + 1 == KS;
        if constexpr (!last) read_frags2(curA, curB, ks + 1, std::integral_constant<int, (ks + 1) & 1>{});
        if constexpr (last) mid_barrier_ab();
        if constexpr (last && ONEBAR)
          read_frags2(stage_buf(std::integral_constant<int, (ia + 1) % NS>{}),
                      bstage_buf(std::integral_constant<int, (ib + 1) % C::NSB>{}), 0, std::integral_constant<int, 0>{});
        [&]<int... MI>(std::integer_sequence<int, MI...>) {
          ([&] {
            constexpr int mi = MI, gm = ks * NM + mi, a = mi / FN, b = mi % FN;
            if constexpr (F8)
              acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[ks & 1][b], fa[ks & 1][a], acc[a][b], 0, 0, 0,
                                                                         0, 0, 0);
            else
              acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks & 1][b], fa[ks & 1][a], acc[a][b], 0, 0, 0);
            if constexpr (!last && gm % 2 == 1 && gm / 2 < JB)
              dma_slot_ab(std::integral_constant<int, JA + gm / 2>{}, k2, curA, nxtB);
            if constexpr (last && mi < JA) dma_slot_ab(std::integral_constant<int, mi>{}, k2, curA, nxtB);
          }(), ...);
        }(std::make_integer_sequence<int, NM>{});
        constexpr int NR = last && !ONEBAR ? 0 : FM + FN;
        [&]<int... MI>(std::integer_sequence<int, MI...>) {
          ([&] {
            constexpr int mi = MI, gm = ks * NM + mi;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (mi < NR) __builtin_amdgcn_sched_group_barrier(0x100, F8 ? 2 : 1, 0);  // one fragment's reads
            if constexpr ((!last && gm % 2 == 1 && gm / 2 < JB) || (last && mi < JA))
              __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
          }(), ...);
        }(std::make_integer_sequence<int, NM>{});
        __builtin_amdgcn_sched_barrier(0);
      }(), ...);
    }(std::make_integer_sequence<int, KS>{});
    if constexpr (!ONEBAR) ring_barrier_ab();
  };

  if constexpr (SPLIT) __syncthreads();  // the previous tile's epilogue may still read the LDS stages
  if constexpr (C::AB) {
    // prologue: the A and B tiles of steps kt0 and kt0 + 1
    [&]<int... J>(std::integer_sequence<int, J...>) {
      (dma_slot_ab(std::integral_constant<int, J>{}, kt0 * BK, stage_buf(std::integral_constant<int, 0>{}),
                   bstage_buf(std::integral_constant<int, 0>{})), ...);
      (dma_slot_ab(std::integral_constant<int, J>{}, (kt0 + 1) * BK, stage_buf(std::integral_constant<int, 1>{}),
                   bstage_buf(std::integral_constant<int, 1>{})), ...);
    }(std::make_integer_sequence<int, D>{});
    ring_barrier_ab();  // the tiles of step kt0 have landed; those of step kt0 + 1 land within step kt0
    // Grouped products: a group's last row tile often holds few rows.  When it holds at most BM / 2, the waves
    // of the lower half of the tile (wave rows WAVES_M / 2 ..) have no row to compute: they issue their share
    // of the loads and meet every barrier, but read no fragments and issue no MFMAs.  Waves w and w + 4 share
    // a SIMD and lie in different halves, so every SIMD keeps one computing wave and the tile takes about half
    // the MFMA time.  (The choice is uniform per wave and made once, around two straight-line loops.)
    bool idle_half = false;
    if constexpr (GROUPED && C::WAVES_M == 4 && NWAVES == 8) idle_half = rows - m0 <= BM / 2 && wm0 >= BM / 2;
    auto step_idle_ab = [&](auto IA, auto IB, int kt) {
      constexpr int ia = decltype(IA)::value, ib = decltype(IB)::value;
      uint16_t* curA = stage_buf(std::integral_constant<int, ia>{});
      uint16_t* nxtB = bstage_buf(std::integral_constant<int, (ib + C::NSB - 1) % C::NSB>{});
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (dma_slot_ab(std::integral_constant<int, JA + J>{}, (kt + 2) * BK, curA, nxtB), ...);
      }(std::make_integer_sequence<int, JB>{});
      mid_barrier_ab();
      [&]<int... J>(std::integer_sequence<int, J...>) {
        (dma_slot_ab(std::integral_constant<int, J>{}, (kt + 2) * BK, curA, nxtB), ...);
      }(std::make_integer_sequence<int, JA>{});
      if constexpr (!ONEBAR) ring_barrier_ab();
    };
    // Whole ring passes in the loop, then the K steps left of a last partial pass one by one (the same
    // stages); steps past the last K step are not run.
    auto run_ab = [&](auto STEP) {
      const int kend = kt1 < KT ? kt1 : KT;
      const int kpass_end = kt0 + (kend - kt0) / RING * RING;
      int kt = kt0;
      for (; kt < kpass_end; kt += RING) {
        [&]<int... U>(std::integer_sequence<int, U...>) {
          (STEP(std::integral_constant<int, U % NS>{}, std::integral_constant<int, U % C::NSB>{}, kt + U), ...);
        }(std::make_integer_sequence<int, RING>{});
      }
      if (kt < kend) {
        [&]<int... U>(std::integer_sequence<int, U...>) {
          (void)((kt + U < kend ? (STEP(std::integral_constant<int, U % NS>{},
                                       std::integral_constant<int, U % C::NSB>{}, kt + U), true)
                                : false) && ...);
        }(std::make_integer_sequence<int, RING - 1>{});
      }
    };
    if (idle_half) run_ab(step_idle_ab);
    else {
      if constexpr (ONEBAR)  // the first k step's fragments of step kt0 (the loop reads the others ahead)
        read_frags2(stage_buf(std::integral_constant<int, 0>{}), bstage_buf(std::integral_constant<int, 0>{}), 0,
                    std::integral_constant<int, 0>{});
      run_ab(step_spread_ab);
    }
  } else {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (dma_stage((kt0 + I) * BK, stage_buf(std::integral_constant<int, I>{})), ...);
  }(std::make_integer_sequence<int, NS - 1>{});
  ring_barrier();
  if constexpr (C::EARLY) read_frags(lds0, 0, std::integral_constant<int, 0>{});
  for (int kt = kt0; kt < kt1; kt += NS) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (step(std::integral_constant<int, I>{}, kt + I), ...);
    }(std::make_integer_sequence<int, NS>{});
  }
  }
  // The last steps prefetched stages past K (never consumed); drain them before the epilogue reuses LDS.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();

  if constexpr (SPLIT) {
    if (sk_partial) {
      // Every workgroup on the tile stores its partial accumulators to its own workspace slot (float4s in
      // register order, thread-linear, so the stores and the loads below are contiguous per wave), then
      // counts itself in on the tile's counter.  The last to arrive adds the slots in workgroup order (a
      // fixed order, so the sum does not depend on arrival order), resets the counter for the next launch
      // and runs the epilogue; the others are done with the tile.  Nobody waits on anybody.
      // The slots and the counter are accessed with device-scope coherent operations (sc1: written through
      // to, and read from, the point where the XCDs' L2s are coherent) and ordered by waiting for the slot
      // stores to complete before counting in, so no fence has to write back or invalidate whole L2s
      // (which would evict the operand panels the other workgroups on the XCD are streaming).
      constexpr int Q = FM * FN * 4;   // float4 per thread
      constexpr int kSc1 = 16;         // cache policy: device scope
      const int64_t slot_bytes = (int64_t)Q * C::NT * 16;
      // (the workspace holds the slots of the split tiles only: sk_slot_tiles of them)
      const __amdgpu_buffer_rsrc_t ws = make_rsrc(p.sk_ws, (int64_t)p.sk_slot_tiles * S * slot_bytes);
      typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
      const int mine = (int)(slot_of(sk_which_chunk, sk_wtile) * slot_bytes) + 16 * tid;
      // (the split ring of the 256 x 256 tile fills the LDS exactly: its flag is the first word of the last
      // B stage, free once the main loop has drained; every wave reads it before any can go on to overwrite
      // it with epilogue staging)
      int* const flag = C::AB ? reinterpret_cast<int*>(ldsb2) : &sk_flag;
      // A tile of two pieces whose other piece has already counted in: this one is last, and its partial
      // stays in registers (no store, no count, no reload).  The other piece counted in only once its slot
      // stores had completed, as below.
      bool early = false;
      if (sk_last - sk_first == 1) {
        if (tid == 0)
          *flag = __hip_atomic_load(p.sk_cnt + sk_tile, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
        __syncthreads();
        early = *flag != 0;
        __syncthreads();
      }
      if (!early) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float4 v = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                           acc[i][j][4 * q + 3]);
              __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ws,
                                                     mine + ((i * FN + j) * 4 + q) * C::NT * 16, 0, kSc1);
            }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's slot stores have completed
        __syncthreads();
        if (tid == 0)
          *flag = __hip_atomic_fetch_add(p.sk_cnt + sk_tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  sk_last - sk_first;
        __syncthreads();
        const bool last = *flag != 0;
        __syncthreads();
        if (!last) return;
      }
      if (tid == 0) __hip_atomic_store(p.sk_cnt + sk_tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The S slots are added in chunk order, in batches of up to 16 float4 per thread (half the partial tile
      // at most, so the batch's registers fit beside the accumulators): all loads of one slot's batch are
      // issued together and then added, so the reduction waits for 2 memory round trips per slot read, not
      // one per fragment and slot.  This piece's own partial is still in the accumulators: when it is the
      // first or second chunk of the tile it is used from there (a + b = b + a exactly, so the sums are those
      // of the plain chunk-order reduction); otherwise the first chunk's slot replaces it and its own slot is
      // read back in turn.  Element e of a thread's slot is fragment e / 4 (i * FN + j), quarter e % 4.
      constexpr int NE = FM * FN * 4, NB = 16, NBATCH = (NE + NB - 1) / NB;
      const int me = sk_which_chunk;
      auto load_batch = [&](int c, int bb, float4* v) {
        const int sc = (int)(slot_of(c, sk_wtile) * slot_bytes) + 16 * tid;
#pragma unroll
        for (int e = 0; e < NB; ++e)
          if (NB * bb + e < NE)
            v[e] = __builtin_bit_cast(
                float4, __builtin_amdgcn_raw_buffer_load_b128(ws, sc + (NB * bb + e) * C::NT * 16, 0, kSc1));
      };
      auto add_batch = [&](int bb, const float4* v, bool assign) {
#pragma unroll
        for (int e = 0; e < NB; ++e) {
          const int ee = NB * bb + e;
          if (ee < NE) {
            const int i = ee / (FN * 4), j = (ee / 4) % FN, q = ee % 4;
            if (assign) {
              acc[i][j][4 * q] = v[e].x; acc[i][j][4 * q + 1] = v[e].y;
              acc[i][j][4 * q + 2] = v[e].z; acc[i][j][4 * q + 3] = v[e].w;
            } else {
              acc[i][j][4 * q] = v[e].x + acc[i][j][4 * q]; acc[i][j][4 * q + 1] = v[e].y + acc[i][j][4 * q + 1];
              acc[i][j][4 * q + 2] = v[e].z + acc[i][j][4 * q + 2];
              acc[i][j][4 * q + 3] = v[e].w + acc[i][j][4 * q + 3];
            }
          }
        }
      };
      const bool own_in_acc = me <= sk_first + 1;
#pragma unroll
      for (int bb = 0; bb < NBATCH; ++bb) {
        float4 v[NB];
        if (me != sk_first) {  // the first chunk's slot: added to this piece's (second) partial, or in its place
          load_batch(sk_first, bb, v);
          add_batch(bb, v, !own_in_acc);
        }
        for (int c = sk_first + 1; c <= sk_last; ++c) {
          if (own_in_acc && c == me) continue;
          load_batch(c, bb, v);
          add_batch(bb, v, false);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  if constexpr (F8) {
    // dequantize: the product of the codes times both tensors' scale factors
    const float s = p.f8_scale_a[0] * p.f8_scale_b[0];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] *= s;
  }

  // ---- epilogue.  Weights were the MFMA's first operand, so lane holds output row (lane & 31) of its
  // 32-row fragment and, in register 4*jj + r, column 8*jj + 4*(lane >> 5) + r of its 32-column fragment.
  const int col4 = 4 * (lane >> 5);
  constexpr int TNO = MODE == MODE_SWIGLU ? TN / 2 : TN;        // output columns per wave
  constexpr int FNO = TNO / 32;                                  // output fragments per wave
  const int ncol0 = tn * NB_OUT + (wave % WAVES_N) * TNO;        // first output column of the wave tile
  // Bias of this lane's output columns, read once with clamped indices (columns past Nout are computed but
  // never stored): per-element loads under branches would each wait a full memory latency.
  constexpr bool kBias = true;
  constexpr bool kNorm = EPI == EPI_NORM;
  float bias_g[kBias ? FNO : 1][4][4], bias_u[MODE == MODE_SWIGLU ? FNO : 1][4][4];
  // norm epilogue: column sums of the folded weight (gate and up parts) and each fragment row's statistics
  float cs_g[kNorm ? FNO : 1][4][4], cs_u[kNorm && MODE == MODE_SWIGLU ? FNO : 1][4][4];
  float st_mean[kNorm ? FM : 1], st_rstd[kNorm ? FM : 1];
  if constexpr (kNorm) {
    const int64_t blen = MODE == MODE_SWIGLU ? p.up_offset + p.Nout : p.Nout;
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.bias_f32, p.bias_f32 ? 4 * blen : 0);
    const __amdgpu_buffer_rsrc_t crs = make_rsrc(p.norm_colsum, p.norm_colsum ? 4 * blen : 0);
#pragma unroll
    for (int jo = 0; jo < FNO; ++jo)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = ncol0 + 32 * jo + 8 * jj + col4 + r;
          bias_g[jo][jj][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(brs, 4 * c, 0, 0));
          cs_g[jo][jj][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(crs, 4 * c, 0, 0));
          if constexpr (MODE == MODE_SWIGLU) {
            const int cu = (int)p.up_offset + c;
            bias_u[jo][jj][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(brs, 4 * cu, 0, 0));
            cs_u[jo][jj][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(crs, 4 * cu, 0, 0));
          }
        }
    const __amdgpu_buffer_rsrc_t srs = make_rsrc(p.norm_stats + 2 * (int64_t)(row_base + m0), 8 * (int64_t)(rows - m0));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rr = wm0 + 32 * i + fr;
      st_mean[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 8 * rr, 0, 0));
      st_rstd[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, 8 * rr + 4, 0, 0));
    }
  } else if constexpr (kBias) {
    // Through a buffer resource that is empty without a bias and ends at the bias's last element: absent
    // and out-of-range elements read as zero, with no branch per element.
    const bool has_bias = p.bias != nullptr && (MODE != MODE_ROW || p.Y != nullptr);
    const int64_t blen = MODE == MODE_SWIGLU ? p.up_offset + p.Nout : p.Nout;
    const __amdgpu_buffer_rsrc_t brs = make_rsrc(p.bias, has_bias ? 2 * blen : 0);
#pragma unroll
    for (int jo = 0; jo < FNO; ++jo)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int c = ncol0 + 32 * jo + 8 * jj + col4 + r;
          bias_g[jo][jj][r] = from_bf16(__builtin_amdgcn_raw_buffer_load_b16(brs, 2 * c, 0, 0));
          if constexpr (MODE == MODE_SWIGLU)
            bias_u[jo][jj][r] = from_bf16(__builtin_amdgcn_raw_buffer_load_b16(brs, 2 * ((int)p.up_offset + c), 0, 0));
        }
  }
  // output value of (fragment row block i, output fragment jo, run jj, element r)
  auto pre = [&](int i, int j, float a, float b, float cs) -> float {
    if constexpr (kNorm) return fmaf(st_rstd[i], fmaf(-st_mean[i], cs, a), b);
    else return a + b;
  };
  auto out_val = [&](int i, int jo, int jj, int r, auto gelu) -> float {
    if constexpr (MODE == MODE_SWIGLU) {
      const float g = pre(i, jo, acc[i][2 * jo][4 * jj + r], bias_g[jo][jj][r], cs_g[kNorm ? jo : 0][jj][r]);
      const float u = pre(i, jo, acc[i][2 * jo + 1][4 * jj + r], bias_u[jo][jj][r],
                          cs_u[kNorm ? jo : 0][jj][r]);
      return silu(g) * u;
    } else {
      const float x = pre(i, jo, acc[i][jo][4 * jj + r], bias_g[jo][jj][r], cs_g[kNorm ? jo : 0][jj][r]);
      if constexpr (decltype(gelu)::value) return gelu_erf(x);
      else return x;
    }
  };
  // bias-dropout-add on the bf16 output of a row product: v = resid + (kept ? v * scale : 0) for the four
  // columns n .. n + 3 of output row orow (n a multiple of 4, so their keep bits share one byte).  Reads go
  // through buffer resources ending at the last row: rows past it read zeros and are never stored.
  constexpr bool kBda = EPI == EPI_BDA;
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t r_rs =
      make_rsrc(kBda ? p.resid : nullptr, kBda ? 2 * (int64_t)(row_base + rows) * p.ldr : 0);
  [[maybe_unused]] const __amdgpu_buffer_rsrc_t k_rs =
      make_rsrc(kBda ? p.keep : nullptr, kBda && p.keep ? (int64_t)(row_base + rows) * p.ldk : 0);
  auto bda4 = [&](int64_t orow, int n, float* v) {
    if constexpr (EPI == EPI_BDA) {
      const uint32_t roff = 2u * (uint32_t)(orow * p.ldr + n);
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(r_rs, roff, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b32(r_rs, roff + 4, 0, 0);
      const float res[4] = {__builtin_bit_cast(float, lo << 16), __builtin_bit_cast(float, lo & 0xFFFF0000u),
                            __builtin_bit_cast(float, hi << 16), __builtin_bit_cast(float, hi & 0xFFFF0000u)};
      if (p.keep) {
        const uint32_t kb = __builtin_amdgcn_raw_buffer_load_b8(k_rs, (uint32_t)(orow * p.ldk + (n >> 3)), 0, 0) >>
                            (n & 7);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = res[r] + (((kb >> r) & 1u) ? v[r] * p.drop_scale : 0.f);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = res[r] + v[r];
      }
    }
  };
  constexpr bool kStaged = MODE == MODE_COL || MODE == MODE_SWIGLU || MODE == MODE_ROW;
  if (kStaged && (MODE != MODE_ROW || p.Yacc == nullptr)) {
    // bf16 outputs go through LDS so that the global stores are whole rows: each wave writes its own
    // TM x TNO tile into a private region (the drain above retired every LDS access of the main loop),
    // then reads it back row-contiguously; no cross-wave synchronisation is needed.  Regions are row-major
    // with 8-byte units permuted per row so the 32 lanes of a write (32 rows, one unit) and of a read (2-4
    // whole rows) hit distinct banks.
    // UPR 8-byte units per row (a multiple of 8).  A write has 32 lanes store one unit of 32 consecutive
    // rows; rows whose starts fall on the same bank offset (RP apart) get distinct XOR permutations of the
    // unit index within blocks of W units, W the largest power of two dividing UPR (at most 32).
    constexpr int UPR = TNO / 4;
    constexpr int W = (UPR & -UPR) < 32 ? (UPR & -UPR) : 32;
    constexpr int RP = 32 / W;
    static_assert(UPR % 8 == 0 && (TM * UPR) % 64 == 0, "unit layout");
    uint16_t* reg = stage_region(std::integral_constant<int, TM * TNO>{});
    auto unit_at = [&](int row, int u) { return row * TNO + 4 * (u ^ ((row / RP) & (W - 1))); };
    auto stage_tile = [&](auto gelu) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jo = 0; jo < FNO; ++jo)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            float v[4] = {out_val(i, jo, jj, 0, gelu), out_val(i, jo, jj, 1, gelu), out_val(i, jo, jj, 2, gelu),
                          out_val(i, jo, jj, 3, gelu)};
            if constexpr (EPI == EPI_BDA)
              bda4((int64_t)row_base + m0 + wm0 + 32 * i + fr, ncol0 + 32 * jo + 8 * jj + col4, v);
            *reinterpret_cast<uint2*>(reg + unit_at(32 * i + fr, 8 * jo + 2 * jj + (lane >> 5))) =
                make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
          }
    };
    if (MODE == MODE_COL && p.act == 1) stage_tile(std::true_type{});
    else stage_tile(std::false_type{});
    // read back row-contiguously: pass q covers units 64 q .. 64 q + 63 of the row-major tile
#pragma unroll 4
    for (int q = 0; q < TM * UPR / 64; ++q) {
      const int id = 64 * q + lane;
      const int row = id / UPR, u = id % UPR;
      const int n = ncol0 + 4 * u;
      const int valid = p.Nout - n;
      const int m = m0 + wm0 + row;
      const uint2 d = *reinterpret_cast<const uint2*>(reg + unit_at(row, u));
      if (m < rows && valid > 0) {
        uint16_t* dst = p.Y + ((int64_t)row_base + m) * p.ldy + n;
        if (valid >= 4) {
          __builtin_nontemporal_store(u32x2{d.x, d.y}, reinterpret_cast<u32x2*>(dst));
        } else {
          // (constant indices: a runtime-indexed local array would be placed in LDS)
          dst[0] = (uint16_t)d.x;
          if (valid > 1) dst[1] = (uint16_t)(d.x >> 16);
          if (valid > 2) dst[2] = (uint16_t)d.y;
        }
      }
    }
    return;
  }
  // Direct stores: ROW with an fp32 target (the uniform choices are made once, outside the element loops).
  auto direct = [&](auto ACCUM, auto WITH_Y) {
    constexpr bool accum = decltype(ACCUM)::value, with_y = decltype(WITH_Y)::value;
    float* const yacc = p.Yacc;
    const int64_t ldacc = p.ldacc, ldy = p.ldy;
    uint16_t* const y = p.Y;
    const int nout = p.Nout;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = m0 + wm0 + 32 * i + fr;
      if (m >= rows) continue;
      const int64_t orow = (int64_t)row_base + m;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = tn * BN + wn0 + 32 * j + 8 * jj + col4;
          if (n >= nout) continue;
          const int valid = nout - n;
          float v[4] = {acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]};
          if constexpr (MODE == MODE_ROW) {
            // fp32 partial of a row-parallel shard (and, on the last shard, the bf16 result)
            float* dst = yacc + orow * ldacc + n;
            if (valid >= 4) {
              if constexpr (accum) {
                const float4 o = *reinterpret_cast<const float4*>(dst);
                v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
              }
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (r < valid) {
                  if constexpr (accum) v[r] += dst[r];
                  dst[r] = v[r];
                }
            }
            if constexpr (with_y) {
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] += bias_g[j][jj][r];
              bda4(orow, n, v);
              store4_bf16(y + orow * ldy + n, v, valid);
            }
          }
        }
      }
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  // fp32 partial alone (no bf16 output): staged through LDS like the bf16 outputs, one 32-row fragment row of
  // the wave tile at a time (32 x TN fp32, the size of a bf16 wave region), so that each store instruction
  // writes whole 16-byte units of 2-3 consecutive rows instead of 32 bytes of each of 32 rows (the
  // accumulator layout).  16-byte units are permuted per row (XOR with row mod 8), so the 8 lanes an LDS
  // access serves together hit distinct banks on the write (8 rows, one unit) and on the read (one row, 8
  // consecutive units).  Each wave's region is its own: no cross-wave synchronisation.
  auto staged_f32 = [&](auto ACCUM) {
    constexpr bool accum = decltype(ACCUM)::value;
    constexpr int UPR = TN / 4;        // 16-byte units per row
    constexpr int REG = 32 * TN * 2;   // region per wave, in uint16
    static_assert(UPR % 8 == 0 && (32 * UPR) % 64 == 0, "unit layout");
    float* const reg = reinterpret_cast<float*>(stage_region(std::integral_constant<int, REG>{}));
    auto unit_at = [&](int row, int u) { return row * TN + 4 * (u ^ (row & 7)); };
    float* const yacc = p.Yacc;
    const int64_t ldacc = p.ldacc;
    const int n0 = tn * BN + wn0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<float4*>(reg + unit_at(fr, 8 * j + 2 * jj + (lane >> 5))) =
              make_float4(acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]);
#pragma unroll 4
      for (int q = 0; q < 32 * UPR / 64; ++q) {
        const int id = 64 * q + lane;
        const int row = id / UPR, u = id % UPR;
        float4 v = *reinterpret_cast<const float4*>(reg + unit_at(row, u));
        const int m = m0 + wm0 + 32 * i + row;
        const int n = n0 + 4 * u;
        const int valid = p.Nout - n;
        if (m < rows && valid > 0) {
          float* dst = yacc + ((int64_t)row_base + m) * ldacc + n;
          if (valid >= 4) {
            if constexpr (accum) {
              const float4 o = *reinterpret_cast<const float4*>(dst);
              v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
            }
            __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(dst));
          } else {
            const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int r = 0; r < 3; ++r)
              if (r < valid) dst[r] = accum ? dst[r] + e[r] : e[r];
          }
        }
      }
    }
  };
  if constexpr (MODE == MODE_ROW) {
    if (!p.Y) {
      if (p.accumulate) staged_f32(T_{});
      else staged_f32(F_{});
      return;
    }
    if (p.accumulate) {
      if (p.Y) direct(T_{}, T_{});
      else direct(T_{}, F_{});
    } else {
      if (p.Y) direct(F_{}, T_{});
      else direct(F_{}, F_{});
    }
  }
  };

  if constexpr (SPLIT && !GROUPED) {
    // Split schedule: every tile's K range is cut into S chunks of whole ring passes, and the units
    // (tile, chunk) are dealt out chunk-major, unit u to logical workgroup u mod G, so the units that run at
    // the same time are the same K chunk of neighbouring tiles: they stream the same K slices of the shared
    // operand panels, as one-tile-per-workgroup tiles do.  (Contiguous per-workgroup K ranges, as in
    // stream-K, put concurrent workgroups at unrelated K positions and defeat the L2.)  Logical ids are
    // XCD-contiguous.
    // Hybrid form (sk_dp_tiles > 0, a multiple of the grid): the first sk_dp_tiles tiles are whole units,
    // one workgroup each, G at a time; only the remaining tiles are cut into chunks, so a ragged last wave
    // of tiles is spread over every CU while the full waves pay no partial-sum traffic.
    const int T = tiles_m * tiles_n;
    if (p.sk_share > 0) {
      // Shared tails (fewer tiles than CUs: the 175B-shard QKV has 192 tiles of 256 x 192 on 256 CUs): every
      // workgroup runs about the same K work.  Block b lands on XCD b mod 8; per XCD the first T / 8 blocks run
      // the first sk_cut ring passes of the XCD's T / 8 tiles (in the usual XCD-contiguous tile order), the
      // others the remaining passes of sk_share tiles each, one after another.  Each tile has two partial
      // sums, added by the later finisher in piece order (the split protocol below).
      const int per = T / 8, xcd = (int)blockIdx.x & 7, r = (int)blockIdx.x >> 3;
      int tm, tn;
      if (r < per) {
        const int t = xcd * per + r;
        tile_coords(t, tiles_m, tiles_n, tm, tn);
        run_tile(tm, tn, 0, p.M, p.B, 0, p.sk_cut * RING, t, t, 0, 0, 1, true);
      } else {
        for (int q = 0; q < p.sk_share; ++q) {
          const int t = xcd * per + (r - per) * p.sk_share + q;
          tile_coords(t, tiles_m, tiles_n, tm, tn);
          run_tile(tm, tn, 0, p.M, p.B, p.sk_cut * RING, KTS, t, t, 1, 0, 1, true);
        }
      }
      return;
    }
    const int TD = p.sk_dp_tiles, TR = T - TD;
    const int U = TD + TR * S;
    for (int u = xcd_remap(blockIdx.x, G); u < U; u += G) {
      int tm, tn;
      if (u < TD) {
        tile_coords(u, tiles_m, tiles_n, tm, tn);
        run_tile(tm, tn, 0, p.M, p.B, 0, KTS, 0, 0, 0, 0, 0, false);
        continue;
      }
      const int v = u - TD;
      const int c = v / TR, tr = v - c * TR;
      const int r0 = (int)((int64_t)c * RI / S), r1 = (int)((int64_t)(c + 1) * RI / S);
      tile_coords(TD + tr, tiles_m, tiles_n, tm, tn);
      run_tile(tm, tn, 0, p.M, p.B, r0 * RING, r1 * RING, TD + tr, tr, c, 0, S - 1, true);
    }
  } else {
    // ---- tile placement
      int tm, tn;
    int row_base = 0, rows = p.M;  // rows of this tile's group (all rows when ungrouped)
    const uint16_t* __restrict__ B = p.B;
    if constexpr (GROUPED) {
      // blockIdx.x = row-tile slot * tiles_n + tn; slots are laid over the groups in order.  Split-tail form
      // (SPLIT): the first sk_full_slots workgroups run each group's whole BM-row tiles only; after them come
      // the tail units, (chunk c, group g, column tile tn) chunk-major: K chunk c of the group's last, partial
      // row tile, whose S chunks are added by the last to finish (as in the split schedule above).  The tail
      // tiles are the ones that make a last, mostly idle wave; cut in S, they fill the CUs the whole tiles
      // leave free.
      const int tiles_n = (p.Nout + NB_OUT - 1) / NB_OUT;
      if (SPLIT && (int)blockIdx.x >= p.sk_full_slots) {
        const int u = (int)blockIdx.x - p.sk_full_slots;
        const int per_c = p.groups * tiles_n;
        const int c = u / per_c, r = u - c * per_c, g = r / tiles_n;
        tn = r - g * tiles_n;
        const int lo = p.group_offsets[g], hi = p.group_offsets[g + 1];
        if ((hi - lo) % BM == 0) return;  // no partial tile in this group
        const int r0 = (int)((int64_t)c * RI / S), r1 = (int)((int64_t)(c + 1) * RI / S);
        run_tile((hi - lo) / BM, tn, lo, hi - lo, B + (int64_t)g * p.group_stride_B, r0 * RING, r1 * RING, r, r, c, 0,
                 S - 1, true);
        return;
      }
      int slot = blockIdx.x / tiles_n;
      tn = blockIdx.x - slot * tiles_n;
      int g = 0;
      for (; g < p.groups; ++g) {
        const int lo = p.group_offsets[g], hi = p.group_offsets[g + 1];
        const int nt = SPLIT ? (hi - lo) / BM : (hi - lo + BM - 1) / BM;
        if (slot < nt) { row_base = lo; rows = hi - lo; break; }
        slot -= nt;
      }
      if (g == p.groups) return;  // spare slot of the upper-bound grid
      tm = slot;
      B += (int64_t)g * p.group_stride_B;
    } else {
      tile_coords(xcd_remap(blockIdx.x, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
    }
    run_tile(tm, tn, row_base, rows, B, 0, KTS, 0, 0, 0, 0, 0, false);
  }
}


template <class C, int MODE, bool GROUPED, bool AT = false, bool BT = false, int EPI = EPI_PLAIN, bool F8 = false>
static hipError_t launch_cfg(const GemmParams& p0, int grid_rows_upper, hipStream_t st, int split_groups = 0,
                             int split_chunks = 0, int dp_tiles = 0, int share = 0) {
  GemmParams p = p0;
  const int nb = MODE == MODE_SWIGLU ? C::BN / 2 : C::BN;
  const int tiles_n = (p.Nout + nb - 1) / nb;
  int64_t tiles;
  if (GROUPED)
    tiles = (int64_t)((grid_rows_upper + C::BM - 1) / C::BM + p.groups) * tiles_n;
  else
    tiles = (int64_t)((p.M + C::BM - 1) / C::BM) * tiles_n;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  // KFULL: no chunk of a K step lies past K.  The 32-deep rings also pad the step count to a multiple of
  // their ring with zero steps, which must read as zero; the split ring runs no step past K.
  const bool kfull = C::AB ? p.K % C::BK == 0 : p.K % (C::BK * C::RING) == 0;
  if constexpr (!GROUPED) {
    if (split_groups > 0 && split_chunks > 1) {
      const size_t slot = (size_t)C::FM * C::FN * 16 * sizeof(float) * C::NT;
      // whole tiles first: whole waves of the grid, leaving at least one tile to split
      if (dp_tiles < 0 || dp_tiles % split_groups != 0 || dp_tiles >= tiles) return hipErrorInvalidValue;
      if (share > 0) {
        // shared tails: per XCD, tiles / 8 first pieces and tiles / 8 / share tail workgroups; the first piece
        // of each tile gets the share of the K passes that balances the two kinds of workgroup
        if (split_chunks != 2 || dp_tiles != 0 || tiles % 8 != 0 || (tiles / 8) % share != 0 ||
            split_groups != tiles + tiles / share)
          return hipErrorInvalidValue;
        const int64_t ri = (((int64_t)p.K + C::BK - 1) / C::BK + C::RING - 1) / C::RING;
        int64_t cut = (ri * share + (share + 1) / 2) / (share + 1);
        cut = cut < 1 ? 1 : (cut > ri - 1 ? ri - 1 : cut);
        if (ri < 2) return hipErrorInvalidValue;
        p.sk_share = share;
        p.sk_cut = (int)cut;
      }
      // the caller's workspace: the counter block, then the slots of the split tiles (the plan was chosen to fit)
      if (tiles > kSplitMaxTiles || !p.ws ||
          p.ws_bytes < kSplitCounterBytes + (size_t)(tiles - dp_tiles) * split_chunks * slot)
        return hipErrorInvalidValue;
      p.sk_chunks = split_chunks;
      p.sk_dp_tiles = dp_tiles;
      p.sk_slot_tiles = (int)(tiles - dp_tiles);
      p.sk_cnt = static_cast<int*>(p.ws);
      p.sk_ws = reinterpret_cast<float*>(static_cast<char*>(p.ws) + kSplitCounterBytes);
      if (kfull)
        hipLaunchKernelGGL((gemm_kernel<C, MODE, false, true, true, AT, BT, EPI, F8>), dim3(split_groups), dim3(C::NT), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_kernel<C, MODE, false, false, true, AT, BT, EPI, F8>), dim3(split_groups), dim3(C::NT), 0, st,
                           p);
      return hipGetLastError();
    }
  } else {
    if (split_chunks > 1) {
      // split tails: whole tiles of every group (at most grid_rows_upper / BM row tiles in all), then
      // split_chunks tail units per (group, column tile); the workspace holds a counter and split_chunks slots
      // per (group, column tile)
      const size_t slot = (size_t)C::FM * C::FN * 16 * sizeof(float) * C::NT;
      const int64_t tail_tiles = (int64_t)p.groups * tiles_n;
      const int64_t full_slots = (int64_t)(grid_rows_upper / C::BM) * tiles_n;
      const int64_t units = full_slots + tail_tiles * split_chunks;
      if (tail_tiles > kSplitMaxTiles || units > 0x7FFFFFFF || !p.ws ||
          p.ws_bytes < kSplitCounterBytes + (size_t)tail_tiles * split_chunks * slot)
        return hipErrorInvalidValue;
      p.sk_chunks = split_chunks;
      p.sk_slot_tiles = (int)tail_tiles;
      p.sk_full_slots = (int)full_slots;
      p.sk_cnt = static_cast<int*>(p.ws);
      p.sk_ws = reinterpret_cast<float*>(static_cast<char*>(p.ws) + kSplitCounterBytes);
      if (kfull)
        hipLaunchKernelGGL((gemm_kernel<C, MODE, true, true, true, AT, BT, EPI, F8>), dim3((unsigned)units), dim3(C::NT), 0, st, p);
      else
        hipLaunchKernelGGL((gemm_kernel<C, MODE, true, false, true, AT, BT, EPI, F8>), dim3((unsigned)units), dim3(C::NT), 0, st,
                           p);
      return hipGetLastError();
    }
  }
  if (kfull)
    hipLaunchKernelGGL((gemm_kernel<C, MODE, GROUPED, true, false, AT, BT, EPI, F8>), dim3((unsigned)tiles), dim3(C::NT), 0, st,
                       p);
  else
    hipLaunchKernelGGL((gemm_kernel<C, MODE, GROUPED, false, false, AT, BT, EPI, F8>), dim3((unsigned)tiles), dim3(C::NT), 0,
                       st, p);
  return hipGetLastError();
}

#ifndef MTP_HALF_CFG
#define MTP_HALF_CFG 256, 128, 4, 2, 32, 4, true
#endif
#ifndef MTP_SMALL_CFG
#define MTP_SMALL_CFG 128, 128, 4, 2, 64, 4, true
#endif
// The large tiles run the split ring with a 64-deep K step (A tiles in two stages, B tiles in three), each
// stage reloaded two steps ahead (step_spread_ab), in every form: bf16 forward (plain and grouped), E4M3
// (K counted in pairs of codes) and backward (row-major-K operands).  256 x 256: 8 waves of 64 x 128 (against
// 128 x 64 wave tiles 1.25-1.45x faster on some MI355X boards and even on the others, outputs bitwise equal),
// 2 x 32 + 3 x 32 KB, the whole LDS.  Against the plain two-stage 64-deep ring (both operands reloaded one step
// ahead) at the 70B-shard shapes: the layer step 828 -> 785 us cold (fc1 457 -> 427, QKV 142 -> 127), 8192^3
// 852 -> 830 us; with both operands cached 0-8% slower, at K = 1024 (345M fc1) 1-7%.  Against the 32-deep
// four-stage ring (128-byte rows per DMA instead of 64): the E4M3 175B-shard linears 11-12% faster, the
// backward dgrad 9-21% and wgrad 2-5%.  The split-K forms spill some registers outside the main loop (bias,
// norm and split epilogue state).  The grouped (MoE) products run 2781 against 2944 us on it (before the A
// stages were reloaded early) where every expert's weights stream from HBM.
using BigFwdTile = Cfg<256, 256, 4, 2, 64, 2, false, 3>;  // 8 waves (64 x 128), split ring, 160 KB
using GroupedTile = BigFwdTile;
// Likewise the 256 x 192 tile (2 x 32 + 3 x 24 KB): against the plain two-stage ring at the 175B-shard shapes,
// 3-6% faster with the weight cached and 8-14% with it streaming from HBM (QKV 236.7 -> 204.4 us, fc1 267.0 ->
// 234.5, fc2 270.5 -> 244.8); reloading the A stages early then took the cold shapes a further 9-16% (QKV
// 258 -> 221 us, fc1 299 -> 252, fc2 290 -> 264).  It beats the 256 x 256 tile where its tile count fills
// whole waves.
using WideFwdTile = Cfg<256, 192, 4, 2, 64, 2, false, 3>;  // 8 waves (64 x 96), split ring, 136 KB
using HalfTile = Cfg<MTP_HALF_CFG>;            // 8 waves (64 x 64), 32-deep four-stage ring, 96 KB
using SmallTile = Cfg<MTP_SMALL_CFG>;          // 8 waves (32 x 64), 128 KB
using SmallTTile = Cfg<128, 128, 4, 2, 32, 4, true>;  // row-major-K operands: 8 waves (32 x 64), 64 KB


// Forward dispatch of one mode and epilogue: the planner's tile and schedule (within the caller's workspace).
template <int MODE, int EPI = EPI_PLAIN>
static hipError_t dispatch_fwd(const GemmParams& p, hipStream_t st) {
  const GemmPlan pl = gemm_plan(MODE, p.M, p.Nout, p.K, 0, true, p.ws ? p.ws_bytes : 0);
  switch (pl.id) {
    case 0:
      return launch_cfg<BigFwdTile, MODE, false, false, false, EPI>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles,
                                                                    pl.share);
    case 1:
      if constexpr (MODE != MODE_SWIGLU)
        return launch_cfg<WideFwdTile, MODE, false, false, false, EPI>(p, 0, st, pl.split_groups, pl.split_chunks,
                                                                       pl.dp_tiles, pl.share);
      return hipErrorInvalidValue;
    case 2: return launch_cfg<HalfTile, MODE, false, false, false, EPI>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles);
    default: return launch_cfg<SmallTile, MODE, false, false, false, EPI>(p, 0, st);  // (never split)
  }
}

// Backward products: dgrad reads B row-major-K (AT = false, BT = true), wgrad both operands.
template <bool AT, bool BT>
static hipError_t dispatch_bwd(const GemmParams& p, hipStream_t st) {
  const GemmPlan pl = gemm_plan(MODE_ROW, p.M, p.Nout, p.K, AT ? 2 : 1, true, p.ws ? p.ws_bytes : 0);
  if (pl.id == 0) return launch_cfg<BigFwdTile, MODE_ROW, false, AT, BT>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles);
  if (pl.id == 4) return launch_cfg<SmallTTile, MODE_ROW, false, AT, BT>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles);
  if (pl.id == 1) return launch_cfg<WideFwdTile, MODE_ROW, false, AT, BT>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles);
  return launch_cfg<HalfTile, MODE_ROW, false, AT, BT>(p, 0, st, pl.split_groups, pl.split_chunks, pl.dp_tiles);
}

}  // namespace mtp
