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
//  * 256 threads = 4 wave64s in a WAVES_M x WAVES_N grid; block tile BM x BN,
//    K step 64.  Each wave owns a (BM/WAVES_M) x (BN/WAVES_N) tile of
//    v_mfma_f32_16x16x32_bf16 fragments accumulated in fp32.
//  * Operands are swapped in the MFMA (weights as the first operand) so a
//    lane's accumulator holds 4 consecutive output columns of one row: the
//    epilogue stores 8 B (bf16) or 16 B (fp32) per lane.
//  * Global -> LDS: 16-byte coalesced loads (8 lanes cover one 128-byte row
//    segment), staged through registers one K step ahead of the MFMAs, LDS
//    double-buffered, one barrier per K step.
//  * LDS rows are 128 B; 16-byte chunks are XOR-swizzled by (row & 7) so the
//    fragment reads (16 rows x one chunk per quarter-wave) hit distinct banks.
//  * Tile order is XCD-aware: consecutive workgroup ids land on different XCDs
//    (8 L2 slices), so ids are remapped to give each XCD a contiguous band of
//    tiles, grouped GROUP_M rows at a time for A/B panel reuse in its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BK = 64;          // K elements per stage: 128 bytes per row
constexpr int kChunks = BK / 8; // 16-byte chunks per LDS row

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

__device__ __forceinline__ uint16_t to_bf16(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
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

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, bool GROUPED>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmParams p) {
  constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_IT = BM * kChunks / kThreads, B_IT = BN * kChunks / kThreads;
  static_assert(WAVES_M * WAVES_N == 4, "four waves");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "fragment multiples");
  static_assert(MODE != MODE_SWIGLU || TN % 32 == 0, "gate/up fragment pairs");
  static_assert(BM * kChunks % kThreads == 0 && BN * kChunks % kThreads == 0, "load split");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (BM + BN) * BK];

  // ---- tile placement
  int tm, tn;
  int row_base = 0, rows = p.M;  // output/A rows handled by this tile's group
  const uint16_t* __restrict__ B = p.B;
  if constexpr (GROUPED) {
    // blockIdx.x = row-tile slot * tiles_n + tn; slots are laid over the groups in order.
    const int tiles_n = (p.Nout + (MODE == MODE_SWIGLU ? BN / 2 : BN) - 1) / (MODE == MODE_SWIGLU ? BN / 2 : BN);
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
    const int tiles_m = (p.M + BM - 1) / BM;
    const int nb = MODE == MODE_SWIGLU ? BN / 2 : BN;
    const int tiles_n = (p.Nout + nb - 1) / nb;
    tile_coords(tiles_m, tiles_n, tm, tn);
  }
  const int m0 = tm * BM;  // relative to row_base
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WAVES_N) * TM, wn0 = (wave % WAVES_N) * TN;

  // ---- per-thread global source rows (fixed across K steps)
  const uint16_t* __restrict__ A = p.A;
  int64_t a_off[A_IT];
  bool a_ok[A_IT];
#pragma unroll
  for (int i = 0; i < A_IT; ++i) {
    const int r = (tid + kThreads * i) >> 3;
    const int m = m0 + r;
    a_ok[i] = m < rows;
    int src = row_base + (a_ok[i] ? m : 0);
    if (p.a_rows) src = a_ok[i] ? p.a_rows[src] : 0;
    a_off[i] = (int64_t)src * p.lda;
  }
  int64_t b_off[B_IT];
  bool b_ok[B_IT];
#pragma unroll
  for (int i = 0; i < B_IT; ++i) {
    const int r = (tid + kThreads * i) >> 3;
    int n;
    if constexpr (MODE == MODE_SWIGLU) {
      const int g16 = r >> 4;
      const int outc = tn * (BN / 2) + 16 * (g16 >> 1) + (r & 15);
      b_ok[i] = outc < p.Nout;
      n = (g16 & 1) ? p.up_offset + outc : outc;
    } else {
      n = tn * BN + r;
      b_ok[i] = n < p.Nout;
    }
    b_off[i] = b_ok[i] ? (int64_t)n * p.ldb : 0;
  }
  const int ch = tid & 7;

  uint4 ra[A_IT], rb[B_IT];
  auto load_stage = [&](int k0) {
    const int gk = k0 + ch * 8;
    const bool k_ok = gk < p.K;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const bool ok = a_ok[i] && k_ok;
      uint4 v = *reinterpret_cast<const uint4*>(A + (ok ? a_off[i] + gk : 0));
      ra[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const bool ok = b_ok[i] && k_ok;
      uint4 v = *reinterpret_cast<const uint4*>(B + (ok ? b_off[i] + gk : 0));
      rb[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int s) {
    uint16_t* sA = smem + s * (BM + BN) * BK;
    uint16_t* sB = sA + BM * BK;
#pragma unroll
    for (int i = 0; i < A_IT; ++i) {
      const int r = (tid + kThreads * i) >> 3;
      *reinterpret_cast<uint4*>(sA + swz(r, ch)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_IT; ++i) {
      const int r = (tid + kThreads * i) >> 3;
      *reinterpret_cast<uint4*>(sB + swz(r, ch)) = rb[i];
    }
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = (p.K + BK - 1) / BK;
  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int fr = lane & 15, fq = lane >> 4;
  for (int kt = 0; kt < KT; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < KT) load_stage((kt + 1) * BK);
    const uint16_t* sA = smem + s * (BM + BN) * BK;
    const uint16_t* sB = sA + BM * BK;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(sA + swz(wm0 + 16 * i + fr, 4 * ks + fq));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(sB + swz(wn0 + 16 * j + fr, 4 * ks + fq));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_stage(s ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane owns output row (m0 + wm0 + 16i + fr), columns 4 fq .. 4 fq + 3 of fragment j
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm0 + 16 * i + fr;
    if (m >= rows) continue;
    const int64_t orow = (int64_t)row_base + m;
    if constexpr (MODE == MODE_SWIGLU) {
#pragma unroll
      for (int j = 0; j < FN; j += 2) {
        const int n = tn * (BN / 2) + 16 * ((wn0 >> 5) + (j >> 1)) + 4 * fq;
        uint16_t out[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float g = acc[i][j][r], u = acc[i][j + 1][r];
          if (p.bias && n + r < p.Nout) {
            g += from_bf16(p.bias[n + r]);
            u += from_bf16(p.bias[p.up_offset + n + r]);
          }
          out[r] = to_bf16(silu(g) * u);
        }
        uint16_t* dst = p.Y + orow * p.ldy + n;
        if (n + 3 < p.Nout) {
          *reinterpret_cast<uint2*>(dst) = make_uint2(out[0] | ((uint32_t)out[1] << 16), out[2] | ((uint32_t)out[3] << 16));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.Nout) dst[r] = out[r];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = tn * BN + wn0 + 16 * j + 4 * fq;
        if (n >= p.Nout) continue;
        const bool full = n + 3 < p.Nout;
        if constexpr (MODE == MODE_COL) {
          uint16_t out[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = acc[i][j][r];
            if (p.bias && n + r < p.Nout) v += from_bf16(p.bias[n + r]);
            if (p.act == 1) v = gelu_erf(v);
            out[r] = to_bf16(v);
          }
          uint16_t* dst = p.Y + orow * p.ldy + n;
          if (full) {
            *reinterpret_cast<uint2*>(dst) = make_uint2(out[0] | ((uint32_t)out[1] << 16), out[2] | ((uint32_t)out[3] << 16));
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < p.Nout) dst[r] = out[r];
          }
        } else if constexpr (MODE == MODE_ROW) {
          float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          if (p.Yacc) {
            float* dst = p.Yacc + orow * p.ldacc + n;
            if (full) {
              if (p.accumulate) {
                float4 o = *reinterpret_cast<const float4*>(dst);
                v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
              }
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < p.Nout) {
                  if (p.accumulate) v[r] += dst[r];
                  dst[r] = v[r];
                }
            }
          }
          if (p.Y) {
            uint16_t out[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float y = v[r];
              if (p.bias && n + r < p.Nout) y += from_bf16(p.bias[n + r]);
              out[r] = to_bf16(y);
            }
            uint16_t* dst = p.Y + orow * p.ldy + n;
            if (full) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(out[0] | ((uint32_t)out[1] << 16), out[2] | ((uint32_t)out[3] << 16));
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (n + r < p.Nout) dst[r] = out[r];
            }
          }
        } else {  // MODE_COMBINE
          const float w = p.row_w[orow];
          float* dst = p.Yacc + (int64_t)p.out_rows[orow] * p.ldacc + n;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (n + r < p.Nout) atomicAdd(dst + r, w * acc[i][j][r]);
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
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, MODE, GROUPED>), dim3((unsigned)tiles), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

// Tile choice: the largest tile that still gives every CU work, else the
// 128 x 128 tile.  (The 256 x 256 tile needs about 256 tiles to fill the chip.)
template <int MODE>
static hipError_t dispatch(const GemmParams& p, hipStream_t st) {
  const int64_t nb_big = MODE == MODE_SWIGLU ? 128 : 256;
  const int64_t big_tiles = ((p.M + 255) / 256) * ((p.Nout + nb_big - 1) / nb_big);
  if (big_tiles >= 192) return launch_cfg<256, 256, 2, 2, MODE, false>(p, 0, st);
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
    case MODE_SWIGLU: return launch_cfg<256, 256, 2, 2, MODE_SWIGLU, true>(p, rows_upper, st);
    case MODE_COMBINE: return launch_cfg<256, 256, 2, 2, MODE_COMBINE, true>(p, rows_upper, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
