// bf16 MFMA GEMM family for gfx950 with fused tensor-parallel epilogues.
//
// Every linear of the layer is C = A . B^T with both operands K-contiguous:
// A = activations [M x K], B = weights stored [out x in] = [N x K] (the
// F.linear layout of the pages' ColumnParallelLinear / RowParallelLinear
// pseudo-code, "ai阅读megatron").  One kernel template covers
//   MODE_COL    : column-parallel output, bf16(act(acc + bias)), act in {none, erf-GeLU}
//   MODE_SWIGLU : column-parallel gate+up, bf16(silu(gate + bg) * (up + bu))
//   MODE_ROW    : row-parallel partial in fp32 (Yacc = P or Yacc += P), and on the
//                 last shard bf16(Yacc + bias): the local form of Y = sum_i Y_i
//   MODE_COMBINE: MoE expert output, Yacc[token] += w * acc (fp32 atomics)
// and a grouped variant (MoE experts) whose row tiles are laid over the
// ragged per-expert row ranges read from device memory.
//
// Design (gfx950, CDNA4):
//  * Block tile BM x BN, K step 64, waves in a WAVES_M x WAVES_N grid; each wave
//    owns a (BM/WAVES_M) x (BN/WAVES_N) tile of v_mfma_f32_32x32x16_bf16
//    fragments accumulated in fp32 (the 32x32x16 form sustains ~97% of the
//    dense bf16 rate on gfx950; the 16x16x32 form measured ~85%).  The large
//    tile is 256 x 256 with 8 waves (two per SIMD, 128 accumulators each) so
//    one wave's MFMAs cover the other's LDS traffic and barrier waits.
//  * Operands are swapped in the MFMA (weights as the first operand) so a
//    lane's accumulators hold runs of 4 consecutive output columns of one row:
//    the epilogue stores 8 B (bf16) or 16 B (fp32) per lane.
//  * Global -> LDS: buffer_load_dwordx4 ... lds (direct to LDS, no VGPR
//    round trip, no ds_write), 8 lanes per 128-byte row segment, one K step
//    ahead, LDS double-buffered, one barrier per K step.  Buffer resources
//    make out-of-range rows read as zero without faulting.
//  * LDS rows are 128 B; 16-byte chunks are XOR-swizzled by (row >> 1) & 7 so
//    the fragment reads (16 consecutive rows at one chunk per 16 lanes) and the
//    staging writes (two rows per 16 lanes) both hit distinct banks of the
//    64-bank LDS (bank conflicts measured with SQ_LDS_BANK_CONFLICT).
//  * Tile order is XCD-aware: consecutive workgroup ids land on different XCDs
//    (8 L2 slices), so ids are remapped to give each XCD a contiguous band of
//    tiles, grouped GROUP_M rows at a time for A/B panel reuse in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm.h"

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;          // K elements per stage: 128 bytes per row
constexpr int kChunks = BK / 8; // 16-byte chunks per LDS row

// LDS layout of a 128-byte row: its eight 16-byte chunks are permuted by XOR with (row >> 1) & 7.  The
// LDS serves 256 bytes (64 banks) per cycle, i.e. two rows; a fragment read has 16 lanes read one chunk
// of 16 consecutive rows, which this permutation spreads over all 16 bank groups.
__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3); }

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)to_bf16(lo) | ((uint32_t)to_bf16(hi) << 16);
}

__device__ __forceinline__ float from_bf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float gelu_erf(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f)); }

__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// Tile coordinates of this workgroup: XCD-aware remap, then GROUP_M row grouping.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  const int total = tiles_m * tiles_n;
  int id = blockIdx.x;
  if ((total & 7) == 0) id = (id & 7) * (total >> 3) + (id >> 3);
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, bool GROUPED, bool KFULL>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void gemm_kernel(GemmParams p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int FM = TM / 32, FN = TN / 32;   // 32 x 32 MFMA tiles per wave
  constexpr int ROWS_PER_PASS = NT / kChunks; // tile rows one load instruction covers
  constexpr int A_IT = BM / ROWS_PER_PASS, B_IT = BN / ROWS_PER_PASS;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32 x 32 fragments");
  static_assert(MODE != MODE_SWIGLU || TN % 64 == 0, "gate/up fragment pairs");
  static_assert(BM % ROWS_PER_PASS == 0 && BN % ROWS_PER_PASS == 0, "load split");
  constexpr int NB_OUT = MODE == MODE_SWIGLU ? BN / 2 : BN;  // output columns per tile

  // two separate LDS arrays (not one indexed by parity) so the compiler can tell that the DMA into one
  // does not alias the fragment reads from the other, and waits for it only where it is consumed
  __shared__ __attribute__((aligned(16))) uint16_t smem0[(BM + BN) * BK];
  __shared__ __attribute__((aligned(16))) uint16_t smem1[(BM + BN) * BK];

  // ---- tile placement
  int tm, tn;
  int row_base = 0, rows = p.M;  // rows of this tile's group (all rows when ungrouped)
  const uint16_t* __restrict__ B = p.B;
  if constexpr (GROUPED) {
    // blockIdx.x = row-tile slot * tiles_n + tn; slots are laid over the groups in order.
    const int tiles_n = (p.Nout + NB_OUT - 1) / NB_OUT;
    int slot = blockIdx.x / tiles_n;
    tn = blockIdx.x - slot * tiles_n;
    int g = 0;
    for (; g < p.groups; ++g) {
      const int lo = p.group_offsets[g], hi = p.group_offsets[g + 1];
      const int nt = (hi - lo + BM - 1) / BM;
      if (slot < nt) { row_base = lo; rows = hi - lo; break; }
      slot -= nt;
    }
    if (g == p.groups) return;  // spare slot of the upper-bound grid
    tm = slot;
    B += (int64_t)g * p.group_stride_B;
  } else {
    tile_coords((p.M + BM - 1) / BM, (p.Nout + NB_OUT - 1) / NB_OUT, tm, tn);
  }
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
  if (p.a_rows) {
    a_base = p.A;
    a_extent = p.a_src_rows * p.lda;
  } else {
    a_base = p.A + (int64_t)(row_base + m0) * p.lda;
    a_extent = (p.a_src_rows - (row_base + m0)) * p.lda;
  }
  const int nbase = tn * NB_OUT;
  const uint16_t* b_base = B + (int64_t)nbase * p.ldb;
  const int64_t b_extent = ((MODE == MODE_SWIGLU ? p.up_offset : 0) + p.Nout - nbase) * p.ldb;
  // (integer clamps written out: the device min() overload for 64-bit integers goes through double, and a
  // converted value lands in a vector register, which turns every buffer load into a waterfall loop)
  const __amdgpu_buffer_rsrc_t a_rsrc = make_rsrc(a_base, 2 * a_extent < (int64_t)kOOB ? 2 * a_extent : (int64_t)kOOB);
  const __amdgpu_buffer_rsrc_t b_rsrc = make_rsrc(b_base, 2 * b_extent < (int64_t)kOOB ? 2 * b_extent : (int64_t)kOOB);
  // Direct-to-LDS loads: one buffer_load_dwordx4 ... lds moves 64 lanes x 16 B = eight 128-byte LDS rows,
  // lane l filling row (l >> 3), chunk (l & 7) of its group.  The LDS layout is swizzled (see swz), so each
  // lane loads the global chunk that lands at its slot: c = (l & 7) ^ ((row >> 1) & 7).
  constexpr int NWAVES = WAVES_M * WAVES_N;
  constexpr int A_G = BM / 8 / NWAVES, B_G = BN / 8 / NWAVES;  // 8-row groups per wave
  static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "DMA split");
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int lrow = lane >> 3;
  uint32_t a_off[A_G], b_off[B_G];
  int a_kc[A_G], b_kc[B_G];  // K element offset of each lane's chunk
#pragma unroll
  for (int i = 0; i < A_G; ++i) {
    const int r = 8 * (wave_u * A_G + i) + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    a_kc[i] = 8 * c;
    if (p.a_rows) {
      const int m = m0 + r;
      a_off[i] = m < rows ? 2u * (uint32_t)((int64_t)p.a_rows[row_base + m] * p.lda + 8 * c) : kOOB;
    } else {
      a_off[i] = 2u * (uint32_t)(r * p.lda + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < B_G; ++i) {
    const int r = 8 * (wave_u * B_G + i) + lrow;
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    b_kc[i] = 8 * c;
    int n = r;
    if constexpr (MODE == MODE_SWIGLU) {
      const int g32 = r >> 5;
      n = 32 * (g32 >> 1) + (r & 31) + ((g32 & 1) ? (int)p.up_offset : 0);
    }
    b_off[i] = 2u * (uint32_t)(n * p.ldb + 8 * c);
  }
  typedef __attribute__((address_space(3))) void* lds_ptr;
  // The scalar offset is not part of the hardware range check (only the per-lane offset is), so it stays
  // inside the rows: a prefetch past the last K step re-reads step 0 into a buffer that is never consumed
  // (KFULL) or is redirected out of range per lane (!KFULL, reading zeros).
  auto dma_stage = [&](int k0, uint16_t* sbuf) {
    const int soff = k0 < p.K ? 2 * k0 : 0;
#pragma unroll
    for (int i = 0; i < A_G; ++i) {
      uint32_t vo = a_off[i];
      if constexpr (!KFULL) vo = k0 + a_kc[i] < p.K ? vo : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_ptr)(sbuf + (wave_u * A_G + i) * 8 * BK), 16, vo, soff, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_G; ++i) {
      uint32_t vo = b_off[i];
      if constexpr (!KFULL) vo = k0 + b_kc[i] < p.K ? vo : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(b_rsrc, (lds_ptr)(sbuf + BM * BK + (wave_u * B_G + i) * 8 * BK), 16, vo,
                                               soff, 0, 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  // 32 x 32 x 16 fragments: lane holds row (lane & 31), k = 8 * (lane >> 5) .. +7 of a 16-wide k step
  const int fr = lane & 31, fk = lane >> 5;
  auto mma_step = [&](const uint16_t* sA, const uint16_t* sB, int ks) {
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm0 + 32 * i + fr, 2 * ks + fk));
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(sB + swz(wn0 + 32 * j + fr, 2 * ks + fk));
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  };
  // K steps, rounded up to an even count: the loop body covers two steps (one per LDS buffer) and has no
  // branches, so the compiler's wait counts stay exact.  With KFULL the step count is even and every chunk
  // is in range; otherwise chunks at or past K read as zero, so an odd step count runs one all-zero step.
  const int KT2 = ((p.K + BK - 1) / BK + 1) & ~1;
  // One K step on LDS buffer P: start the DMA of step kt + 1 into the other buffer, run this step's MFMAs,
  // then wait for this wave's DMA and meet the other waves at the barrier.
  auto body = [&](auto parity, int kt) {
    constexpr int P = decltype(parity)::value;
    uint16_t* cur = P == 0 ? smem0 : smem1;
    uint16_t* nxt = P == 0 ? smem1 : smem0;
    dma_stage((kt + 1) * BK, nxt);
    __builtin_amdgcn_sched_barrier(0);  // keep the DMA issue at the top: the scheduler would sink it
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) mma_step(cur, cur + BM * BK, ks);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMA into the other buffer has landed
    __syncthreads();
  };
  dma_stage(0, smem0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int kt = 0; kt < KT2; kt += 2) {
    body(std::integral_constant<int, 0>{}, kt);
    body(std::integral_constant<int, 1>{}, kt + 1);
  }

  // ---- epilogue.  Weights were the MFMA's first operand, so lane holds output row (lane & 31) of its
  // 32-row fragment and, in register 4*jj + r, column 8*jj + 4*(lane >> 5) + r of its 32-column fragment.
  const int col4 = 4 * (lane >> 5);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm0 + 32 * i + fr;
    if (m >= rows) continue;
    const int64_t orow = (int64_t)row_base + m;
    if constexpr (MODE == MODE_SWIGLU) {
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
        const int g32 = wn0 / 32 + j;  // even: gate rows; g32 + 1: the matching up rows
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = tn * NB_OUT + 32 * (g32 >> 1) + 8 * jj + col4;
          if (n >= p.Nout) continue;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float g = acc[i][j][4 * jj + r], u = acc[i][j + 1][4 * jj + r];
            if (p.bias && n + r < p.Nout) {
              g += from_bf16(p.bias[n + r]);
              u += from_bf16(p.bias[p.up_offset + n + r]);
            }
            v[r] = silu(g) * u;
          }
          store4_bf16(p.Y + orow * p.ldy + n, v, p.Nout - n);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = tn * BN + wn0 + 32 * j + 8 * jj + col4;
          if (n >= p.Nout) continue;
          const int valid = p.Nout - n;
          float v[4] = {acc[i][j][4 * jj], acc[i][j][4 * jj + 1], acc[i][j][4 * jj + 2], acc[i][j][4 * jj + 3]};
          if constexpr (MODE == MODE_COL) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if (p.bias && r < valid) v[r] += from_bf16(p.bias[n + r]);
              if (p.act == 1) v[r] = gelu_erf(v[r]);
            }
            store4_bf16(p.Y + orow * p.ldy + n, v, valid);
          } else if constexpr (MODE == MODE_ROW) {
            if (p.Yacc) {
              float* dst = p.Yacc + orow * p.ldacc + n;
              if (valid >= 4) {
                if (p.accumulate) {
                  const float4 o = *reinterpret_cast<const float4*>(dst);
                  v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
                }
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
              } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                  if (r < valid) {
                    if (p.accumulate) v[r] += dst[r];
                    dst[r] = v[r];
                  }
              }
            }
            if (p.Y) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (p.bias && r < valid) v[r] += from_bf16(p.bias[n + r]);
              store4_bf16(p.Y + orow * p.ldy + n, v, valid);
            }
          } else {  // MODE_COMBINE
            const float w = p.row_w[orow];
            float* dst = p.Yacc + (int64_t)p.out_rows[orow] * p.ldacc + n;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (r < valid) atomicAdd(dst + r, w * v[r]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------ launch
template <int BM, int BN, int WM, int WN, int MODE, bool GROUPED>
static hipError_t launch_cfg(const GemmParams& p, int grid_rows_upper, hipStream_t st) {
  const int nb = MODE == MODE_SWIGLU ? BN / 2 : BN;
  const int tiles_n = (p.Nout + nb - 1) / nb;
  int64_t tiles;
  if (GROUPED)
    tiles = (int64_t)((grid_rows_upper + BM - 1) / BM + p.groups) * tiles_n;
  else
    tiles = (int64_t)((p.M + BM - 1) / BM) * tiles_n;
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool kfull = p.K % (2 * BK) == 0;  // whole chunks and an even number of K steps
  if (kfull)
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, GROUPED, true>), dim3((unsigned)tiles), dim3(64 * WM * WN),
                       0, st, p);
  else
    hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, GROUPED, false>), dim3((unsigned)tiles), dim3(64 * WM * WN),
                       0, st, p);
  return hipGetLastError();
}

// Tile choice: the largest tile that still gives every CU work, else the
// 128 x 128 tile.  (The 256 x 256 tile needs about 256 tiles to fill the chip.)
template <int MODE>
static hipError_t dispatch(const GemmParams& p, hipStream_t st) {
  const int64_t nb_big = MODE == MODE_SWIGLU ? 128 : 256;
  const int64_t big_tiles = ((p.M + 255) / 256) * ((p.Nout + nb_big - 1) / nb_big);
  if (big_tiles >= 192) return launch_cfg<256, 256, 2, 4, MODE, false>(p, 0, st);
  return launch_cfg<128, 128, 2, 2, MODE, false>(p, 0, st);
}

hipError_t gemm(const GemmParams& p, int mode, hipStream_t st) {
  switch (mode) {
    case MODE_COL: return dispatch<MODE_COL>(p, st);
    case MODE_SWIGLU: return dispatch<MODE_SWIGLU>(p, st);
    case MODE_ROW: return dispatch<MODE_ROW>(p, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t gemm_grouped(const GemmParams& p, int mode, int rows_upper, hipStream_t st) {
  switch (mode) {
    case MODE_SWIGLU: return launch_cfg<256, 256, 2, 4, MODE_SWIGLU, true>(p, rows_upper, st);
    case MODE_COMBINE: return launch_cfg<256, 256, 2, 4, MODE_COMBINE, true>(p, rows_upper, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
