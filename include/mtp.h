/*
 * mtp.h - one tensor-parallel rank's share of a Megatron-style Transformer
 * layer forward, on an AMD Instinct MI355X (gfx950).
 *
 * The operations follow the pages' statement of tensor parallelism:
 *  - "Megatron-LM 深度学习与源码分析文档", part 2 (核心并行技术), section 2
 *    (Tensor Parallel): ColumnParallelLinear W = [W_1..W_p], Y_i = X W_i with
 *    an optional all-gather Y = [Y_1..Y_p]; RowParallelLinear
 *    W = [W_1; ..; W_p], X = [X_1..X_p], Y_i = X_i W_i, Y = sum_i Y_i (an
 *    all-reduce); QKV projection [Q,K,V] = X W_qkv with num_heads/TP heads
 *    per rank; MLP Z = phi(X W_1), Y = Z W_2 with fc1 column-parallel (4H/TP,
 *    wider for SwiGLU) and fc2 row-parallel.
 *  - "ai阅读megatron": ColumnParallelLinear / RowParallelLinear forward
 *    (F.linear(x, weight): weights stored [out x in]); TransformerConfig
 *    (activation_func = F.gelu, gated_linear_unit, num_query_groups,
 *    num_moe_experts, moe_router_topk); MoELayer forward (router logits,
 *    top-k, dispatch, expert MLPs, weighted combine).
 *  - "快速入门" section 5.1 (weight mapping): linear_qkv = [q; k; v],
 *    linear_fc1 = [gate_proj; up_proj], down_proj split along its input.
 *
 * On one GPU the cross-rank collectives become identities: the all-gather is
 * each shard writing its own column block of one output (through ldy), and
 * the all-reduce is an fp32 sum of the shards' partial products in rank order.
 *
 * Conventions for every call:
 *  - bf16 tensors are raw bit patterns (uint16_t), row-major with the given
 *    row pitch (in elements).  Weights are [out x in].  Accumulation is fp32;
 *    every conversion to bf16 rounds to nearest, ties to even.
 *  - Pointers are device pointers owned by the caller; the library keeps none
 *    after returning, and it never allocates, frees or synchronises.
 *  - Workspace.  The GEMM calls take `workspace` (device memory, 16-byte
 *    aligned, or NULL) and its size `workspace_bytes`.  It is used only by
 *    the split-K schedule (see mtp_gemm_plan, which reports the bytes a plan
 *    needs): a call whose best plan needs more workspace than it is given
 *    takes the best plan that fits (one workgroup per tile needs none), so
 *    NULL / 0 is always valid.  Its first 16 KiB hold int32 arrival counters
 *    (one per output tile of a split launch; such launches have at most 4096
 *    tiles): they must be zero before the workspace is first used (allocate
 *    it zero-filled), and every call that completes leaves them zero again;
 *    the partial sums follow them.  Calls that may run at the same time (on
 *    different streams, or in graphs replayed concurrently) need distinct
 *    workspaces; calls ordered on one stream may share one, whatever their
 *    shapes.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *    and the call returns at once.  Faults surface at the caller's next sync.
 *  - Every argument is validated before anything is enqueued; on an error
 *    nothing is launched and no output is touched.  Requirements: required
 *    pointers non-NULL; sizes >= 1; K (the inner dimension) and every row
 *    pitch multiples of 8; pitches at least the row width; bf16/fp32 pointers
 *    16-byte aligned; the current device a gfx950.
 *  - Outputs must not alias inputs.  Calls are reentrant; the only shared
 *    state is an immutable per-device property cache (architecture, CU count)
 *    filled on first use.
 */
#ifndef MTP_H_
#define MTP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTP_ABI_VERSION 2

typedef uint16_t mtp_bf16;

typedef enum {
  MTP_OK = 0,
  MTP_ERR_NULL = 1,        /* a required pointer is NULL */
  MTP_ERR_SHAPE = 2,       /* a size, pitch, rank range or head/group rule is violated */
  MTP_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  MTP_ERR_UNSUPPORTED = 4, /* no device, or the current device is not a gfx950 */
  MTP_ERR_LAUNCH = 5       /* the runtime refused a kernel launch */
} mtp_status;

typedef enum { MTP_ACT_NONE = 0, MTP_ACT_GELU = 1, MTP_ACT_SWIGLU = 2 } mtp_act;

typedef enum { MTP_NORM_LAYER = 0, MTP_NORM_RMS = 1 } mtp_norm;

#define MTP_FP8_WS_FLOATS 1024 /* scratch of mtp_fp8_quantize, in fp32 elements */

/*
 * ColumnParallelLinear forward of one shard (part 2 section 2, Y_i = X W_i),
 * with its bias and activation fused:
 *   Y[M x Nout] = act(X[M x K] . Wt[N x K]^T + bias[N])
 *   NONE, GELU (exact erf form):  Nout = N.
 *   SWIGLU: the N rows of Wt are [gate (N/2 rows) ; up (N/2 rows)] and
 *           Y[i][j] = silu(pre[i][j]) * pre[i][N/2 + j], Nout = N/2; N even.
 * bias may be NULL.  The all-gather of the shards is the identity when each
 * shard r writes to Y + r * Nout with ldy = p * Nout.
 */
mtp_status mtp_column_linear(const mtp_bf16* X, int64_t ldx, const mtp_bf16* Wt, int64_t ldw,
                             const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy, int64_t M, int64_t N,
                             int64_t K, mtp_act act, void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): mtp_column_linear with the split-K
 * workspace taken from a static device array of the library,
 * MTP_STATIC_SCRATCH_BYTES per GPU (held until the process ends), instead of a
 * caller argument.  The call allocates nothing.  scratch_bytes (at most
 * MTP_STATIC_SCRATCH_BYTES, else MTP_ERR_SHAPE) is how much of it the plan may
 * use, as workspace_bytes for mtp_column_linear: the same value gives the
 * same plan and bitwise the same output (0: one workgroup per tile).  Every
 * call on a GPU shares that GPU's array and each call that splits first
 * clears its counter block, so calls that overlap on one GPU (different
 * streams, concurrent graphs) race; calls ordered on one stream do not.
 */
#define MTP_STATIC_SCRATCH_BYTES (32u << 20)
mtp_status mtp_column_linear_static(const mtp_bf16* X, int64_t ldx, const mtp_bf16* Wt, int64_t ldw,
                                    const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy, int64_t M, int64_t N,
                                    int64_t K, mtp_act act, size_t scratch_bytes, void* stream);

/*
 * RowParallelLinear partial product of one shard (Y_i = X_i W_i) and the
 * local form of the all-reduce Y = sum_i Y_i:
 *   P = Z[M x Kp] . Wt[N x Kp]^T in fp32, no bias.  Wt is this rank's input
 *   block of the full [N x K] weight: pass Wt + r*Kp with ldw = K.
 *   accumulate = 0: Yacc = P;  accumulate = 1: Yacc += P  (fp32).
 *   If Y != NULL (the last shard): Y = bf16(Yacc_after + bias), bias added
 *   once here (bias may be NULL).  Yacc may be NULL only when
 *   accumulate == 0 and Y != NULL (a single shard: Y = bf16(P + bias)).
 * Summing the shards by calling r = 0..p-1 in order on one stream is
 * deterministic.
 */
mtp_status mtp_row_linear_partial(const mtp_bf16* Z, int64_t ldz, const mtp_bf16* Wt, int64_t ldw,
                                  float* Yacc, int64_t ldacc, int accumulate, const mtp_bf16* bias,
                                  mtp_bf16* Y, int64_t ldy, int64_t M, int64_t N, int64_t Kp,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tensor-parallel MLP, Z = phi(X W_1), Y = Z W_2, for shards r0..r1-1 of a
 * p-way split, computed in turn:
 *   Z_r   = act(X . W1t_r^T + b1_r)       -> Z_ws (bf16, [M x F/p])
 *   Yacc (+)= Z_r . W2t_r^T               (fp32, rank order)
 * X is [M x H] (pitch H).  W1t is rank-major [p * N1 x H] with N1 = F/p
 * (GELU/NONE) or 2F/p holding [gate_r ; up_r] (SWIGLU); b1 is [p * N1] or
 * NULL.  W2t is [H x F] (pitch F); rank r owns its columns r*F/p..(r+1)*F/p.
 * When [r0, r1) = [0, p) the last shard writes Y = bf16(Yacc + b2) (b2 may be
 * NULL); with p = 1 Yacc may be NULL and Y is written directly.  Otherwise Y
 * must be NULL and Yacc holds the partial sum over [r0, r1).  Requires
 * F % p == 0, 0 <= r0 < r1 <= p, H % 8 == 0, (F/p) % 8 == 0.
 */
mtp_status mtp_mlp_forward(const mtp_bf16* X, int64_t M, int64_t H, int64_t F, int p, int r0, int r1,
                           const mtp_bf16* W1t, const mtp_bf16* b1, const mtp_bf16* W2t,
                           const mtp_bf16* b2, mtp_act act, mtp_bf16* Z_ws, float* Yacc, mtp_bf16* Y,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * QKV projection of one rank (part 2 section 2, [Q,K,V] = X W_qkv, heads/TP
 * per rank; grouped-query attention keeps num_query_groups/TP key/value
 * groups per rank):
 *   QKV[M x Nq] = X[M x H] . Wqkv_t^T + bias, Nq = (nq_local + 2*ng_local) * head_dim,
 * columns [Q_r (nq_local*head_dim) | K_r (ng_local*head_dim) | V_r (same)].
 * Wqkv_t is [Nq x H] with pitch ldw; bias is [Nq] or NULL; output pitch ldo.
 * Requires nq_local % ng_local == 0 and head_dim % 8 == 0.
 */
mtp_status mtp_qkv_forward(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t H, const mtp_bf16* Wqkv_t,
                           int64_t ldw, const mtp_bf16* bias, int nq_local, int ng_local, int head_dim,
                           mtp_bf16* QKV, int64_t ldo, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The norm prologue of a column-parallel linear ("快速入门", model
 * implementation: the layer spec's QKV linear is the LayerNorm-fused
 * column-parallel linear and pre_mlp_layernorm precedes fc1; the LLaMA layer
 * tree uses RMSNorm; "Megatron-LM 深度学习与源码分析文档", part 3: LayerNorm
 * among the layer's elementwise kernels).  LayerNorm: mean and biased
 * variance over the row, y = (x - mean) / sqrt(var + eps) * g + beta.
 * RMSNorm: y = x / sqrt(mean(x^2) + eps) * g.  g = gamma, or 1 + gamma when
 * one_plus (zero-centred storage, the pages' --apply-layernorm-1p).
 *
 * The norm is folded through the product instead of materialising the
 * normalized activations:
 *   norm(X) . Wt^T + b = rstd * (X . Wf^T - mean * colsum) + bias_f,
 * Wf = Wt scaled by g along K (bf16, rounded to nearest even),
 * colsum[n] = sum_k Wf[n][k], bias_f[n] = b[n] + sum_k beta[k] Wt[n][k].
 *
 * mtp_norm_stats: per-row (mean, rstd) of X [M x H] into stats[2 M] (fp32,
 *   8-byte aligned; RMSNorm writes mean = 0).  H % 8 == 0; eps >= 0.
 * mtp_norm_fold_weights: Wf [N x K] (pitch ldwf), colsum [N] (may be NULL:
 *   only LayerNorm needs it), bias_f [N] (fp32) from Wt [N x K], gamma [K],
 *   beta [K] (NULL: none), bias [N] (NULL: none).  Once per weight update.
 *   A SwiGLU weight [gate ; up] folds as one N = 2F matrix.
 * mtp_norm_column_linear: Y = act(rstd_m * (X . Wf^T - mean_m * colsum) +
 *   bias_f) with the same shapes, activations and output rules as
 *   mtp_column_linear; colsum NULL drops the centring term (RMSNorm),
 *   bias_f NULL means no bias.
 */
mtp_status mtp_norm_stats(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t H, mtp_norm kind, float eps,
                          float* stats, void* stream);
mtp_status mtp_norm_fold_weights(const mtp_bf16* Wt, int64_t ldw, int64_t N, int64_t K, const mtp_bf16* gamma,
                                 const mtp_bf16* beta, const mtp_bf16* bias, int one_plus, mtp_bf16* Wf,
                                 int64_t ldwf, float* colsum, float* bias_f, void* stream);
mtp_status mtp_norm_column_linear(const mtp_bf16* X, int64_t ldx, const float* stats, const mtp_bf16* Wf,
                                  int64_t ldw, const float* colsum, const float* bias_f, mtp_bf16* Y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t K, mtp_act act, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Row-parallel partial with the bias-dropout-add epilogue ("快速入门", model
 * implementation: self_attn_bda and mlp_bda follow the attention output
 * projection and fc2; "Megatron-LM 深度学习与源码分析文档", part 3:
 * bias+dropout+add among the fused elementwise kernels).  As
 * mtp_row_linear_partial (Yacc optional: NULL for a single shard), and the
 * bf16 output is the new residual stream:
 *   Y = bf16(residual + keep * (P + bias) / (1 - p_drop))
 * (P the fp32 sum of the shards so far).  keep: packed dropout keep bits
 * (the random draw, made by the caller), column c of row i in bit c % 8 of
 * byte i * ldk + c / 8, ldk >= ceil(N / 8); NULL means no dropout and then
 * p_drop must be 0.  residual [M x N] (pitch ldr) is required; Y may not
 * alias it.  Only the call that finishes the sum should take this form.
 */
mtp_status mtp_row_linear_bda(const mtp_bf16* Z, int64_t ldz, const mtp_bf16* Wt, int64_t ldw, float* Yacc,
                              int64_t ldacc, int accumulate, const mtp_bf16* bias, const mtp_bf16* residual,
                              int64_t ldr, const uint8_t* keep, int64_t ldk, float p_drop, mtp_bf16* Y, int64_t ldy,
                              int64_t M, int64_t N, int64_t Kp, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * FP8 (E4M3) forward GEMMs with per-tensor scaling ("快速入门", FP8 training:
 * E4M3 in the forward pass, an amax-derived scaling factor per tensor;
 * "Megatron-LM 深度学习与源码分析文档", part 5: FP8 quant/dequant and scaling
 * among the kernel priorities).  E4M3 as defined by the FP8 formats paper
 * (OCP): bias 7, max 448, S.1111.111 = NaN, no infinities.
 *
 * mtp_fp8_quantize: Xq = E4M3(fp32(x * s)), nearest with ties to even,
 *   saturating; s = fp32(448 / amax) (1 if amax = 0), amax = max |x| of X
 *   [M x K]; *scale_inv = fp32(1 / s) (the dequantization factor), one
 *   fp32 in device memory.  amax_ws: MTP_FP8_WS_FLOATS fp32 of device
 *   scratch (per-block partial maxima; calls sharing it on one stream are
 *   ordered, on different streams they race).  M K < 2^34.  K % 8 == 0; Xq pitch
 *   ldq (bytes) >= K and a multiple of 8; X and Xq 16-byte aligned.
 * mtp_fp8_column_linear: Y = act(x_scale_inv * w_scale_inv * (Xq . Wq^T) +
 *   bias), shapes, activations and output rules as mtp_column_linear; Wq
 *   [N x K] codes (weights quantized once per update); the scale factors are
 *   device pointers (as mtp_fp8_quantize writes them).
 * mtp_fp8_row_linear_partial: as mtp_row_linear_partial with the product
 *   x_scale_inv * w_scale_inv * (Zq . Wq^T) (fp32 partials, bf16 last shard).
 * For both GEMMs: K and the code pitches (bytes) are multiples of 16; fp32
 * accumulation; code matrices 16-byte aligned and under 2 GiB per 256 rows.
 */
mtp_status mtp_fp8_quantize(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Xq, int64_t ldq,
                            float* amax_ws, float* scale_inv, void* stream);
/* Delayed scaling (the pages' recipe: an amax history, reduced by max): s = fp32(448 / max(amax_history[0 ..
 * history_len-1])) (1 if 0), codes as mtp_fp8_quantize (values past the history's max saturate at +-448),
 * one pass over X; afterwards this tensor's amax is stored in amax_history[step % history_len].  The history
 * (device fp32, 1 <= history_len <= 4096) is the caller's; ws as in mtp_fp8_quantize. */
mtp_status mtp_fp8_quantize_delayed(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Xq, int64_t ldq,
                                    float* amax_history, int history_len, int64_t step, float* ws, float* scale_inv,
                                    void* stream);
mtp_status mtp_fp8_column_linear(const uint8_t* Xq, int64_t ldx, const float* x_scale_inv, const uint8_t* Wq,
                                 int64_t ldw, const float* w_scale_inv, const mtp_bf16* bias, mtp_bf16* Y,
                                 int64_t ldy, int64_t M, int64_t N, int64_t K, mtp_act act, void* workspace,
                                 size_t workspace_bytes, void* stream);
mtp_status mtp_fp8_row_linear_partial(const uint8_t* Zq, int64_t ldz, const float* z_scale_inv, const uint8_t* Wq,
                                      int64_t ldw, const float* w_scale_inv, float* Yacc, int64_t ldacc,
                                      int accumulate, const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy, int64_t M,
                                      int64_t N, int64_t Kp, void* workspace, size_t workspace_bytes,
                                      void* stream);
/* The launch plan and workspace of an E4M3 GEMM (mtp_fp8_column_linear with activation act, or
 * mtp_fp8_row_linear_partial with act = NONE), as mtp_gemm_plan reports them for the bf16 calls; launches
 * nothing. */
mtp_status mtp_fp8_gemm_plan(int64_t M, int64_t N, int64_t K, mtp_act act, int* tile_m, int* tile_n, int* split_k,
                             size_t* workspace_bytes);

/*
 * Backward GEMMs of a linear Y = X . Wt^T ("Megatron-LM 深度学习与源码分析文档",
 * part 2 section 2: each parallel linear's backward computes the input and
 * weight gradients; the column-parallel one all-reduces dX across ranks, the
 * row-parallel one needs no exchange for dX; "ai阅读megatron": train_step's
 * backward pass).  fp32 accumulation, bf16 inputs (raw bits).
 *
 * mtp_linear_dgrad: dX [M x K] = dY [M x N] . Wt [N x K].  dXacc (fp32,
 * pitch ldacc) receives dX (accumulate = 0) or adds it (accumulate = 1: the
 * local form of the column-parallel all-reduce over ranks); if dX != NULL
 * it also receives bf16(result).  At least one of dXacc, dX is non-NULL;
 * accumulate needs dXacc.  N (the contraction) % 8 == 0.
 *
 * mtp_linear_wgrad: dWt [N x K] = dY^T . X, summed over the M rows
 * (dY [M x N], X [M x K]), into fp32 dW (pitch lddw): dW = result
 * (accumulate = 0) or dW += result (accumulate = 1, gradient accumulation).
 *
 * Both read their row-major-K operands with the gfx950 LDS transpose load,
 * so no transposed copy is made.  Same pointer, pitch and alignment rules as
 * the forward calls, except that only dgrad's N must be a multiple of 8
 * (K, and wgrad's M, N, K are free).  A row-major-K operand is read in
 * 8-column chunks, so each of its rows is read up to the next multiple of 8
 * past its width (inside the pitch; those columns reach no output); each
 * such operand must span less than 2 GiB.
 */
mtp_status mtp_linear_dgrad(const mtp_bf16* dY, int64_t lddy, const mtp_bf16* Wt, int64_t ldw, float* dXacc,
                            int64_t ldacc, int accumulate, mtp_bf16* dX, int64_t lddx, int64_t M, int64_t N,
                            int64_t K, void* workspace, size_t workspace_bytes, void* stream);
mtp_status mtp_linear_wgrad(const mtp_bf16* dY, int64_t lddy, const mtp_bf16* X, int64_t ldx, float* dW,
                            int64_t lddw, int accumulate, int64_t M, int64_t N, int64_t K, void* workspace,
                            size_t workspace_bytes, void* stream);
/* The launch plan of a backward product with output [M x N] and contraction K (dgrad: M, K_out, N; wgrad:
 * N, K, M in the names above; wgrad != 0 selects mtp_linear_wgrad's plan) and the workspace it needs, as
 * mtp_gemm_plan; launches nothing. */
mtp_status mtp_gemm_plan_backward(int64_t M, int64_t N, int64_t K, int wgrad, int* tile_m, int* tile_n,
                                  int* split_k, size_t* workspace_bytes);

/*
 * Rotary position embedding of the query and key heads of one rank's QKV
 * output, in place ("Megatron-LM 深度学习与源码分析文档", part 2 sections 3
 * and 6: RoPE as a fused elementwise kernel on the QKV output, with
 * rotary_base and rotary_percent; the rotation is RoFormer's, cited there):
 * for row i at position m = positions[i] and pair j < rotary_dim/2 of each
 * of the nq_local query and ng_local key heads (the first nq_local + ng_local
 * heads of the row; value heads are untouched),
 *   (x_a, x_b) <- (x_a cos(m t_j) - x_b sin(m t_j), x_b cos(m t_j) + x_a sin(m t_j)),
 *   t_j = base^(-2j / rotary_dim),
 * with b = a + rotary_dim/2, a = j ("rotate half", interleaved = 0) or
 * a = 2j, b = 2j + 1 (interleaved = 1); head dimensions from rotary_dim on
 * pass through.  Computed in fp32 from the bf16 values (angle reduced in
 * double precision), rounded to bf16.  QKV is [M x ldo] bf16 as written by
 * mtp_qkv_forward; positions is an int32 device array [M].  Requires
 * nq_local % ng_local == 0, head_dim % 8 == 0, rotary_dim % 8 == 0 with
 * 8 <= rotary_dim <= min(head_dim, 512), base > 1.
 */
mtp_status mtp_rope_qk(mtp_bf16* QKV, int64_t ldo, int64_t M, const int32_t* positions, int nq_local,
                       int ng_local, int head_dim, int rotary_dim, double base, int interleaved,
                       void* stream);

/*
 * MoE router ("ai阅读megatron", MoELayer forward: router logits, top-k):
 * softmax over the E experts of each token (fp32), then the k most probable
 * experts (ties to the lower index).  Outputs, rows grouped by expert in
 * ascending expert order and ascending token order within an expert:
 *   expert_offsets [E+1] (int32, offsets[0] = 0, offsets[E] = T*k),
 *   token_idx [T*k] (int32 token of each dispatched row),
 *   token_w  [T*k] (fp32 softmax probability of each dispatched row, not
 *            renormalised),
 * and the inverse map token_rows [T*k] (int32): token_rows[t*k + s] is the
 * dispatched row of token t's s-th choice, most probable first.
 * logits is [T x E] fp32 (pitch E).  Requires 1 <= k <= min(E, 8), E <= 64.
 */
mtp_status mtp_moe_route(const float* logits, int64_t T, int E, int k, int32_t* expert_offsets,
                         int32_t* token_idx, float* token_w, int32_t* token_rows, void* stream);

/*
 * Expert MLPs of an MoE layer as grouped GEMMs over the routed rows, and the
 * weighted combine:
 *   for each dispatched row j of expert e (token t = token_idx[j]):
 *     z_j = SwiGLU(X[t] . W1t_e^T)            -> Z_ws[j]   (bf16, [T*k x F])
 *     y_j = z_j . W2t_e^T                     -> Y_rows[j] (fp32, [T*k x H])
 *   Y[t] = bf16(sum over s = 0..k-1 of token_w[r_s] * y_{r_s}),
 *          r_s = token_rows[t*k + s], added in that order in fp32
 *          ([T x H]; deterministic for every k).
 * W1t is [E][2F x H] ([gate; up] per expert), W2t is [E][H x F].  The routing
 * tables are device arrays as written by mtp_moe_route (no host copy is
 * made).  Z_ws and Y_rows are caller-owned scratch; nothing needs zeroing.
 * workspace: as for the GEMM calls (16-byte aligned or NULL, first 16 KiB
 * zero before first use and left zero).  When it holds the bytes that
 * mtp_moe_plan reports, the fc2 product runs each expert's last, partial
 * row tile in K chunks on otherwise idle CUs, the chunks added in a fixed
 * order (deterministic; the sum order of those rows differs from the
 * unsplit one by fp32 rounding only); with less, or NULL, it runs unsplit.
 */
mtp_status mtp_moe_mlp_forward(const mtp_bf16* X, int64_t T, int64_t H, int E, int64_t F, int k,
                               const int32_t* expert_offsets, const int32_t* token_idx,
                               const float* token_w, const int32_t* token_rows, const mtp_bf16* W1t,
                               const mtp_bf16* W2t, mtp_bf16* Z_ws, float* Y_rows, mtp_bf16* Y,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The split of mtp_moe_mlp_forward's fc2 product for these sizes on the
 * current device: K chunks per expert tail tile (0: none) and the workspace
 * bytes that split needs (0 when none).  Rejects what mtp_moe_mlp_forward
 * rejects for the same sizes.
 */
mtp_status mtp_moe_plan(int64_t T, int64_t H, int E, int64_t F, int k, int* split_chunks,
                        size_t* workspace_bytes);

/*
 * The launch plan the GEMM calls would use for an [M x K] . [N x K]^T
 * product with activation act (SWIGLU: N counts gate and up rows): the tile
 * (*tile_m x *tile_n output elements; the MFMA tiles are 256 x 256,
 * 256 x 192, 256 x 128 and 128 x 128) and *split_k, 0 for one workgroup per
 * tile, else the number of K chunks each tile is cut into (split-K: one
 * workgroup per CU works through the (tile, chunk) units and the tile's last
 * finisher adds the chunks' fp32 partial sums in chunk order, so results are
 * deterministic but round differently from the unsplit schedule).  Split-K is
 * chosen when whole waves of tiles would leave many CUs idle and the K range
 * is long enough to pay for the partial sums' traffic; when whole waves fill
 * the CUs and a ragged last wave does not, the whole waves may run one tile
 * per workgroup and only the remaining tiles split (*split_k is then their
 * chunk count).  *workspace_bytes (may be NULL) receives the workspace that
 * plan needs (0 for one workgroup per tile): a GEMM call given at least that
 * much takes this plan.  The same size rules as mtp_column_linear apply;
 * nothing is launched.  mtp_row_linear_partial plans as act = NONE; an MLP
 * (mtp_mlp_forward) needs the larger of its fc1 and fc2 plans' workspaces.
 */
mtp_status mtp_gemm_plan(int64_t M, int64_t N, int64_t K, mtp_act act, int* tile_m, int* tile_n,
                         int* split_k, size_t* workspace_bytes);

/*
 * Measurement helper (not part of the layer): an MFMA-only loop of `blocks`
 * workgroups of 8 waves, each wave issuing iters x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each) with no memory traffic, to
 * calibrate the bf16 rate the chip sustains at the clock it runs under such
 * a load.  FLOP = blocks * 8 * iters * 8 * 32768.  out: blocks fp32 (device,
 * written only in a case that does not occur; it keeps the work live).
 */
mtp_status mtp_mfma_calibrate(float* out, int blocks, int iters, void* stream);

/* Static text for a status code. */
const char* mtp_status_string(mtp_status s);
/* Detail of the last failing call on this thread ("" if none). */
const char* mtp_last_error(void);
/* MTP_ABI_VERSION of the built library. */
int mtp_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTP_H_ */
