// Internal interface of the GEMM kernel family (not part of the C ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

constexpr int kMaxExperts = 64;

enum GemmMode { MODE_COL = 0, MODE_SWIGLU = 1, MODE_ROW = 2 };

// C = A . B^T over K, A [rows x K] (pitch lda, optional row gather), B [N x K] (pitch ldb).
struct GemmParams {
  const uint16_t* A = nullptr;
  int64_t lda = 0;
  const int32_t* a_rows = nullptr;  // A row of output row j is a_rows[j] (grouped fc1 gather)
  int64_t a_src_rows = 0;           // rows of A addressable from p.A (bounds its buffer resource)
  const uint16_t* B = nullptr;
  int64_t ldb = 0;
  int64_t up_offset = 0;            // SWIGLU: row offset of the up half within B (= Nout)
  const uint16_t* bias = nullptr;   // [N] (COL/ROW) or [2 * Nout] (SWIGLU)
  uint16_t* Y = nullptr;            // bf16 output
  int64_t ldy = 0;
  float* Yacc = nullptr;            // fp32 partial (grouped: the rows' fp32 outputs)
  int64_t ldacc = 0;
  int M = 0;                        // rows (ungrouped)
  int Nout = 0;                     // output columns (SWIGLU: half the B rows used)
  int K = 0;
  int act = 0;                      // COL: 0 none, 1 erf-GeLU
  int accumulate = 0;               // ROW: Yacc += P
  const int32_t* group_offsets = nullptr;  // grouped: [groups + 1] row offsets in device memory
  int groups = 0;
  int64_t group_stride_B = 0;       // grouped: elements between consecutive groups' B
  // EPI_NORM (COL/SWIGLU): out = act(rstd_m * (acc - mean_m * colsum_n) + bias_f_n), the norm prologue
  // folded through the product (the scale is already folded into B)
  const float* norm_stats = nullptr;  // [rows] x (mean, rstd)
  const float* norm_colsum = nullptr; // [N] (NULL: no centring term)
  const float* bias_f32 = nullptr;    // [N] fp32 bias (NULL: none)
  // EPI_BDA (ROW, bf16 output): Y = resid + dropout(P + bias), kept elements scaled by drop_scale
  const uint16_t* resid = nullptr;
  int64_t ldr = 0;
  const uint8_t* keep = nullptr;      // packed keep bits (column c: bit c % 8 of byte c / 8), NULL: no dropout
  int64_t ldk = 0;                    // bytes per keep row
  float drop_scale = 1.f;
  // E4M3 products: device pointers to the two operands' dequantization factors (the product is scaled by
  // both before the epilogue); K, lda and ldb then count pairs of one-byte codes
  const float* f8_scale_a = nullptr;
  const float* f8_scale_b = nullptr;
  // Caller-owned workspace of the split schedule (NULL / 0: plans that need none): per-tile arrival counters
  // (int32, zero between launches) in the first kSplitCounterBytes bytes, then the partial-tile slots.
  void* ws = nullptr;
  size_t ws_bytes = 0;
  float* sk_ws = nullptr;           // split schedule: partial-tile slots (set at launch)
  int sk_chunks = 0;                // split schedule: K chunks per tile
  int sk_dp_tiles = 0;              // split schedule: leading tiles run whole (a multiple of the grid)
  int sk_slot_tiles = 0;            // split schedule: tiles with partial slots in the workspace (set at launch)
  int sk_full_slots = 0;            // grouped split-tail schedule: workgroups of whole tiles before the tail units
  int sk_share = 0;                 // shared-tail split: tiles whose K tails one workgroup runs (0: other forms)
  int sk_cut = 0;                   // shared-tail split: ring passes of each tile's first piece
  int* sk_cnt = nullptr;            // split schedule: per-tile arrival counters (set at launch)
};

// The split schedule's workspace starts with a counter block of fixed size (one int32 per output tile, for up
// to kSplitMaxTiles tiles; split plans are only made for launches with at most that many), then the slots.  The
// block's size does not depend on the launch, so a launch's slots never overlap the counters of another launch
// that shares the workspace.
constexpr int64_t kSplitMaxTiles = 4096;
constexpr size_t kSplitCounterBytes = 4 * kSplitMaxTiles;

// Tile and schedule of a launch (split_groups 0: one workgroup per tile) and the workspace it needs.
// share > 0: the shared-tail split (fewer tiles than CUs): each tile's first K passes in a workgroup of its own,
// the remaining passes of `share` tiles in one further workgroup (split_chunks = 2, split_groups = tiles +
// tiles / share).
struct GemmPlan {
  int bm = 0, bn = 0, split_groups = 0, id = 0, split_chunks = 0, dp_tiles = 0;
  size_t ws_bytes = 0;
  int share = 0;
};
// row_major_k: 0 both operands K-contiguous; 1 B row-major-K (dgrad); 2 both row-major-K (wgrad).  Only
// schedules whose workspace fits in ws_avail bytes are considered (one tile per workgroup needs none).
// The E4M3 products plan with K counted in pairs of codes and allow_small = false.
GemmPlan gemm_plan(int mode, int64_t M, int64_t Nout, int64_t K, int row_major_k = 0, bool allow_small = true,
                   size_t ws_avail = SIZE_MAX);

enum GemmEpilogue { EPI_PLAIN = 0, EPI_NORM = 1, EPI_BDA = 2 };
hipError_t gemm(const GemmParams& p, int mode, hipStream_t st, int epi = EPI_PLAIN);
// per-mode forward dispatch (gemm_fwd_col.hip, gemm_fwd_swiglu.hip, gemm_fwd_row.hip) and the backward products
// (gemm_bwd_dgrad.hip, gemm_bwd_wgrad.hip)
hipError_t gemm_fwd_col(const GemmParams& p, hipStream_t st, int epi);
hipError_t gemm_fwd_swiglu(const GemmParams& p, hipStream_t st, int epi);
hipError_t gemm_fwd_row(const GemmParams& p, hipStream_t st, int epi);
hipError_t gemm_dgrad(const GemmParams& p, hipStream_t st);
hipError_t gemm_wgrad(const GemmParams& p, hipStream_t st);
// COL / SWIGLU product whose split-K workspace is the library's static scratch (static_scratch.hip), at most
// scratch_bytes of it (p.ws is ignored).
hipError_t gemm_column_static(GemmParams p, int mode, size_t scratch_bytes, hipStream_t st);
// MODE_ROW products whose A (and/or B) operand is stored [K x M] ([K x N]): lda / ldb are those pitches.
hipError_t gemm_backward(const GemmParams& p, bool a_row_major_k, bool b_row_major_k, hipStream_t st);
// E4M3 x E4M3 products (gemm_f8.hip): COL (none / GeLU), SWIGLU and ROW epilogues.
hipError_t gemm_f8(const GemmParams& p, int mode, hipStream_t st);
// Per-tensor E4M3 quantization (fp8.hip): amax of X, then codes = E4M3(fp32(x * s)), s = fp32(448 / amax),
// and scale_inv = fp32(1 / s).  ws: kFp8QuantBlocks fp32 of device scratch (per-block partial maxima).
constexpr int kFp8QuantBlocks = 1024;
hipError_t fp8_quantize(const uint16_t* X, int64_t ldx, int M, int K, uint8_t* Xq, int64_t ldq, float* ws,
                        float* scale_inv, hipStream_t st);
// Delayed scaling: s from the max of hist[0 .. hlen-1]; this tensor's amax then goes to hist[step % hlen].
hipError_t fp8_quantize_delayed(const uint16_t* X, int64_t ldx, int M, int K, uint8_t* Xq, int64_t ldq, float* hist,
                                int hlen, int64_t step, float* ws, float* scale_inv, hipStream_t st);
// rows_upper: total rows over all groups (an upper bound is enough; spare tiles exit).  split_chunks > 1: the
// split-tail schedule (each group's last, partial row tile in split_chunks K chunks, in p.ws).
hipError_t gemm_grouped(const GemmParams& p, int mode, int rows_upper, hipStream_t st, int split_chunks = 0);
// Split-tail plan of a grouped product (SWIGLU or ROW, 256 x 256 tiles): K chunks per tail tile (0: none) and
// the workspace it needs.
struct GroupedPlan {
  int split_chunks = 0;
  size_t ws_bytes = 0;
};
GroupedPlan grouped_plan(int mode, int64_t rows_upper, int groups, int64_t Nout, int64_t K);

// MFMA-only loop over `blocks` workgroups of 8 waves, `iters` x 8 products of 32 x 32 x 16 per wave (calibrate.hip).
hipError_t mfma_calibrate(float* out, int blocks, int iters, hipStream_t st);

// Rotary position embedding of the first `heads` heads of each row, in place (rope.hip).
hipError_t rope_qk(uint16_t* qkv, int64_t ldo, int M, const int32_t* positions, int heads, int head_dim,
                   int rotary_dim, double base, bool interleaved, hipStream_t st);

// Norm prologue pieces (norm.hip): per-row (mean, rstd), and the scale/shift folded into a weight.
hipError_t norm_stats(const uint16_t* X, int64_t ldx, int M, int H, int kind, float eps, float* stats,
                      hipStream_t st);
hipError_t norm_fold(const uint16_t* Wt, int64_t ldw, int N, int K, const uint16_t* gamma, const uint16_t* beta,
                     const uint16_t* bias, int one_plus, uint16_t* Wf, int64_t ldwf, float* colsum, float* bias_f,
                     hipStream_t st);

// MoE helpers (moe.hip).
hipError_t moe_route(const float* logits, int T, int E, int k, int32_t* offsets, int32_t* token_idx,
                     float* token_w, int32_t* token_rows, hipStream_t st);
// out[t] = bf16(sum over s < k, in slot order, of token_w[r] * rows[r]), r = token_rows[t * k + s]; H % 4 == 0.
hipError_t moe_combine(const float* rows, int64_t ldr, const int32_t* token_rows, const float* token_w, int T, int k,
                       int H, uint16_t* out, int64_t ldo, hipStream_t st);

}  // namespace mtp
