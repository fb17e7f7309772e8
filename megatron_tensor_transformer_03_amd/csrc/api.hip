// The C ABI (include/mtp.h): argument validation, then launches on the caller's stream.
//
// Every check runs before the first launch, so a rejected call enqueues
// nothing and touches no output.  The only state is a per-device cache of
// "is this a gfx950" and of the CU count, filled on first use; the library
// allocates, frees and synchronises nothing.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>

#include "../../include/mtp.h"
#include "gemm.h"

namespace {

thread_local char g_err[512] = "";

mtp_status fail(mtp_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

constexpr int64_t kIntMax = 0x7FFFFFFF;

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_ok[64];

mtp_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(MTP_ERR_UNSUPPORTED, "no HIP device is available");
  if (dev < 64) {
    int c = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return MTP_OK;
    if (c == 2) return fail(MTP_ERR_UNSUPPORTED, "device %d is not a gfx950", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(MTP_ERR_UNSUPPORTED, "cannot read the properties of device %d", dev);
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  if (!ok) return fail(MTP_ERR_UNSUPPORTED, "device %d is %s, not a gfx950", dev, prop.gcnArchName);
  return MTP_OK;
}

mtp_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MTP_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  g_err[0] = 0;
  return MTP_OK;
}

// A bf16 operand of `rows` x `cols` with pitch ld: non-NULL, aligned, pitch a multiple of 8 covering the row.
mtp_status check_mat(const void* p, const char* name, int64_t cols, int64_t ld) {
  if (!p) return fail(MTP_ERR_NULL, "%s is NULL", name);
  if (misaligned(p)) return fail(MTP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (ld < cols || ld % 8 != 0) return fail(MTP_ERR_SHAPE, "%s: pitch %lld must be >= %lld and a multiple of 8", name,
                                            (long long)ld, (long long)cols);
  return MTP_OK;
}

mtp_status check_vec(const void* p, const char* name) {
  if (p && misaligned(p)) return fail(MTP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return MTP_OK;
}

mtp_status check_dims(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return fail(MTP_ERR_SHAPE, "sizes must be >= 1 (M=%lld N=%lld K=%lld)", (long long)M,
                                           (long long)N, (long long)K);
  if (M > kIntMax || N > kIntMax || K > kIntMax) return fail(MTP_ERR_SHAPE, "a size exceeds 2^31-1");
  if (K % 8 != 0) return fail(MTP_ERR_SHAPE, "the inner dimension %lld is not a multiple of 8", (long long)K);
  return MTP_OK;
}

// The GEMM kernels address each operand through a buffer resource based at the tile's first row, with
// 32-bit byte offsets: a tile's rows (up to 256, plus the up-projection offset for SwiGLU) must span
// less than 2 GiB.
constexpr int64_t kWindow = (int64_t)1 << 31;

// The caller's split-schedule workspace: NULL (then its size counts as 0) or 16-byte aligned.
mtp_status check_ws(const void* ws, size_t bytes, size_t* avail) {
  if (ws && misaligned(ws)) return fail(MTP_ERR_ALIGN, "workspace is not 16-byte aligned");
  *avail = ws ? bytes : 0;
  return MTP_OK;
}
mtp_status check_window(const char* name, int64_t rows, int64_t ld) {
  if (2 * rows * ld >= kWindow - 64)
    return fail(MTP_ERR_SHAPE, "%s: %lld rows of pitch %lld exceed the 2 GiB addressing window", name,
                (long long)rows, (long long)ld);
  return MTP_OK;
}

#define TRY(x)                     \
  do {                             \
    mtp_status s_ = (x);           \
    if (s_ != MTP_OK) return s_;   \
  } while (0)

}  // namespace

extern "C" {

int mtp_abi_version(void) { return MTP_ABI_VERSION; }

const char* mtp_last_error(void) { return g_err; }

const char* mtp_status_string(mtp_status s) {
  switch (s) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "invalid size, pitch or rank range";
    case MTP_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MTP_ERR_UNSUPPORTED: return "no gfx950 device";
    case MTP_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

mtp_status mtp_gemm_plan(int64_t M, int64_t N, int64_t K, mtp_act act, int* tile_m, int* tile_n, int* split_k,
                         size_t* workspace_bytes) {
  TRY(check_dims(M, N, K));
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  if (!tile_m || !tile_n || !split_k) return fail(MTP_ERR_NULL, "an output pointer is NULL");
  TRY(check_device());
  const mtp::GemmPlan pl = mtp::gemm_plan(act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, M,
                                          act == MTP_ACT_SWIGLU ? N / 2 : N, K);
  *tile_m = pl.bm;
  *tile_n = pl.bn;
  *split_k = pl.split_groups > 0 ? pl.split_chunks : 0;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  g_err[0] = 0;
  return MTP_OK;
}

mtp_status mtp_fp8_gemm_plan(int64_t M, int64_t N, int64_t K, mtp_act act, int* tile_m, int* tile_n, int* split_k,
                             size_t* workspace_bytes) {
  TRY(check_dims(M, N, K));
  if (K % 16 != 0) return fail(MTP_ERR_SHAPE, "the inner dimension %lld is not a multiple of 16", (long long)K);
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  if (!tile_m || !tile_n || !split_k) return fail(MTP_ERR_NULL, "an output pointer is NULL");
  TRY(check_device());
  // (the E4M3 kernels count K in pairs of codes and have no 128 x 128 tile with a 64-deep step)
  const mtp::GemmPlan pl = mtp::gemm_plan(act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, M,
                                          act == MTP_ACT_SWIGLU ? N / 2 : N, K / 2, 0, false, SIZE_MAX);
  *tile_m = pl.bm;
  *tile_n = pl.bn;
  *split_k = pl.split_groups > 0 ? pl.split_chunks : 0;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  g_err[0] = 0;
  return MTP_OK;
}

mtp_status mtp_gemm_plan_backward(int64_t M, int64_t N, int64_t K, int wgrad, int* tile_m, int* tile_n,
                                  int* split_k, size_t* workspace_bytes) {
  if (M < 1 || N < 1 || K < 1 || M > kIntMax || N > kIntMax || K > kIntMax)
    return fail(MTP_ERR_SHAPE, "sizes must be in [1, 2^31-1] (M=%lld N=%lld K=%lld)", (long long)M, (long long)N,
                (long long)K);
  if (!tile_m || !tile_n || !split_k) return fail(MTP_ERR_NULL, "an output pointer is NULL");
  TRY(check_device());
  const mtp::GemmPlan pl = mtp::gemm_plan(mtp::MODE_ROW, M, N, K, wgrad ? 2 : 1);
  *tile_m = pl.bm;
  *tile_n = pl.bn;
  *split_k = pl.split_groups > 0 ? pl.split_chunks : 0;
  if (workspace_bytes) *workspace_bytes = pl.ws_bytes;
  g_err[0] = 0;
  return MTP_OK;
}

mtp_status mtp_column_linear(const mtp_bf16* X, int64_t ldx, const mtp_bf16* Wt, int64_t ldw, const mtp_bf16* bias,
                             mtp_bf16* Y, int64_t ldy, int64_t M, int64_t N, int64_t K, mtp_act act,
                             void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, K));
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  const int64_t nout = act == MTP_ACT_SWIGLU ? N / 2 : N;
  TRY(check_mat(X, "X", K, ldx));
  TRY(check_mat(Wt, "Wt", K, ldw));
  TRY(check_mat(Y, "Y", nout, ldy));
  TRY(check_vec(bias, "bias"));
  TRY(check_window("X", 256, ldx));
  TRY(check_window("Wt", (act == MTP_ACT_SWIGLU ? nout : 0) + 256, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = X; p.lda = ldx; p.B = Wt; p.ldb = ldw; p.bias = bias; p.Y = Y; p.ldy = ldy;
  p.M = (int)M; p.Nout = (int)nout; p.K = (int)K; p.up_offset = nout; p.a_src_rows = M;
  p.act = act == MTP_ACT_GELU ? 1 : 0;
  return launched(mtp::gemm(p, act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, (hipStream_t)stream),
                  "column linear");
}

mtp_status mtp_column_linear_static(const mtp_bf16* X, int64_t ldx, const mtp_bf16* Wt, int64_t ldw,
                                    const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                    mtp_act act, size_t scratch_bytes, void* stream) {
  TRY(check_dims(M, N, K));
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  if (scratch_bytes > (size_t)MTP_STATIC_SCRATCH_BYTES)
    return fail(MTP_ERR_SHAPE, "scratch_bytes %zu exceeds the static scratch of %zu bytes", scratch_bytes,
                (size_t)MTP_STATIC_SCRATCH_BYTES);
  const int64_t nout = act == MTP_ACT_SWIGLU ? N / 2 : N;
  TRY(check_mat(X, "X", K, ldx));
  TRY(check_mat(Wt, "Wt", K, ldw));
  TRY(check_mat(Y, "Y", nout, ldy));
  TRY(check_vec(bias, "bias"));
  TRY(check_window("X", 256, ldx));
  TRY(check_window("Wt", (act == MTP_ACT_SWIGLU ? nout : 0) + 256, ldw));
  TRY(check_device());
  mtp::GemmParams p;
  p.A = X; p.lda = ldx; p.B = Wt; p.ldb = ldw; p.bias = bias; p.Y = Y; p.ldy = ldy;
  p.M = (int)M; p.Nout = (int)nout; p.K = (int)K; p.up_offset = nout; p.a_src_rows = M;
  p.act = act == MTP_ACT_GELU ? 1 : 0;
  return launched(mtp::gemm_column_static(p, act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, scratch_bytes,
                                          (hipStream_t)stream),
                  "column linear (static scratch)");
}

mtp_status mtp_row_linear_partial(const mtp_bf16* Z, int64_t ldz, const mtp_bf16* Wt, int64_t ldw, float* Yacc,
                                  int64_t ldacc, int accumulate, const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t Kp,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, Kp));
  TRY(check_mat(Z, "Z", Kp, ldz));
  TRY(check_mat(Wt, "Wt", Kp, ldw));
  if (!Yacc && !Y) return fail(MTP_ERR_NULL, "Yacc and Y are both NULL");
  if (!Yacc && accumulate) return fail(MTP_ERR_NULL, "accumulate needs Yacc");
  if (Yacc) TRY(check_mat(Yacc, "Yacc", N, ldacc));
  if (Y) TRY(check_mat(Y, "Y", N, ldy));
  TRY(check_vec(bias, "bias"));
  TRY(check_window("Z", 256, ldz));
  TRY(check_window("Wt", 256, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = Z; p.lda = ldz; p.B = Wt; p.ldb = ldw; p.Yacc = Yacc; p.ldacc = ldacc; p.accumulate = accumulate ? 1 : 0;
  p.bias = bias; p.Y = Y; p.ldy = ldy; p.M = (int)M; p.Nout = (int)N; p.K = (int)Kp; p.a_src_rows = M;
  return launched(mtp::gemm(p, mtp::MODE_ROW, (hipStream_t)stream), "row-parallel partial");
}

mtp_status mtp_row_linear_bda(const mtp_bf16* Z, int64_t ldz, const mtp_bf16* Wt, int64_t ldw, float* Yacc,
                              int64_t ldacc, int accumulate, const mtp_bf16* bias, const mtp_bf16* residual,
                              int64_t ldr, const uint8_t* keep, int64_t ldk, float p_drop, mtp_bf16* Y, int64_t ldy,
                              int64_t M, int64_t N, int64_t Kp,
                              void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, Kp));
  TRY(check_mat(Z, "Z", Kp, ldz));
  TRY(check_mat(Wt, "Wt", Kp, ldw));
  if (!Yacc && accumulate) return fail(MTP_ERR_NULL, "accumulate needs Yacc");
  if (Yacc) TRY(check_mat(Yacc, "Yacc", N, ldacc));
  TRY(check_mat(Y, "Y", N, ldy));
  TRY(check_mat(residual, "residual", N, ldr));
  TRY(check_vec(bias, "bias"));
  if (!(p_drop >= 0.f && p_drop < 1.f)) return fail(MTP_ERR_SHAPE, "dropout probability %g is not in [0, 1)", (double)p_drop);
  if (keep) {
    if (ldk < (N + 7) / 8) return fail(MTP_ERR_SHAPE, "keep: %lld bytes per row < %lld", (long long)ldk, (long long)((N + 7) / 8));
    if (M * ldk >= kWindow - 64) return fail(MTP_ERR_SHAPE, "keep: the mask exceeds the 2 GiB addressing window");
  } else if (p_drop != 0.f) {
    return fail(MTP_ERR_NULL, "dropout probability %g without a keep mask", (double)p_drop);
  }
  TRY(check_window("residual", M, ldr));
  TRY(check_window("Z", 256, ldz));
  TRY(check_window("Wt", 256, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = Z; p.lda = ldz; p.B = Wt; p.ldb = ldw; p.Yacc = Yacc; p.ldacc = Yacc ? ldacc : 0;
  p.accumulate = accumulate ? 1 : 0; p.bias = bias; p.Y = Y; p.ldy = ldy;
  p.M = (int)M; p.Nout = (int)N; p.K = (int)Kp; p.a_src_rows = M;
  p.resid = residual; p.ldr = ldr; p.keep = keep; p.ldk = keep ? ldk : 0;
  p.drop_scale = keep ? 1.f / (1.f - p_drop) : 1.f;
  return launched(mtp::gemm(p, mtp::MODE_ROW, (hipStream_t)stream, mtp::EPI_BDA), "row-parallel bias-dropout-add");
}

mtp_status mtp_norm_stats(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t H, mtp_norm kind, float eps,
                          float* stats, void* stream) {
  TRY(check_dims(M, 8, H));
  TRY(check_mat(X, "X", H, ldx));
  if (kind != MTP_NORM_LAYER && kind != MTP_NORM_RMS) return fail(MTP_ERR_SHAPE, "unknown norm kind %d", (int)kind);
  if (!(eps >= 0.f && eps < 1e30f)) return fail(MTP_ERR_SHAPE, "eps %g must be finite and >= 0", (double)eps);
  if (!stats) return fail(MTP_ERR_NULL, "stats is NULL");
  if (reinterpret_cast<uintptr_t>(stats) & 7u) return fail(MTP_ERR_ALIGN, "stats is not 8-byte aligned");
  TRY(check_device());
  return launched(mtp::norm_stats(X, ldx, (int)M, (int)H, (int)kind, eps, stats, (hipStream_t)stream), "norm stats");
}

mtp_status mtp_norm_fold_weights(const mtp_bf16* Wt, int64_t ldw, int64_t N, int64_t K, const mtp_bf16* gamma,
                                 const mtp_bf16* beta, const mtp_bf16* bias, int one_plus, mtp_bf16* Wf,
                                 int64_t ldwf, float* colsum, float* bias_f, void* stream) {
  TRY(check_dims(N, 8, K));
  TRY(check_mat(Wt, "Wt", K, ldw));
  TRY(check_mat(Wf, "Wf", K, ldwf));
  if (!gamma) return fail(MTP_ERR_NULL, "gamma is NULL");
  TRY(check_vec(gamma, "gamma"));
  TRY(check_vec(beta, "beta"));
  TRY(check_vec(bias, "bias"));
  if (!bias_f) return fail(MTP_ERR_NULL, "bias_f is NULL");
  TRY(check_vec(bias_f, "bias_f"));
  TRY(check_vec(colsum, "colsum"));
  TRY(check_device());
  return launched(mtp::norm_fold(Wt, ldw, (int)N, (int)K, gamma, beta, bias, one_plus ? 1 : 0, Wf, ldwf, colsum,
                                 bias_f, (hipStream_t)stream),
                  "norm fold");
}

mtp_status mtp_norm_column_linear(const mtp_bf16* X, int64_t ldx, const float* stats, const mtp_bf16* Wf,
                                  int64_t ldw, const float* colsum, const float* bias_f, mtp_bf16* Y, int64_t ldy,
                                  int64_t M, int64_t N, int64_t K, mtp_act act,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, K));
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  const int64_t nout = act == MTP_ACT_SWIGLU ? N / 2 : N;
  TRY(check_mat(X, "X", K, ldx));
  TRY(check_mat(Wf, "Wf", K, ldw));
  TRY(check_mat(Y, "Y", nout, ldy));
  if (!stats) return fail(MTP_ERR_NULL, "stats is NULL");
  if (reinterpret_cast<uintptr_t>(stats) & 7u) return fail(MTP_ERR_ALIGN, "stats is not 8-byte aligned");
  TRY(check_vec(colsum, "colsum"));
  TRY(check_vec(bias_f, "bias_f"));
  TRY(check_window("X", 256, ldx));
  TRY(check_window("Wf", (act == MTP_ACT_SWIGLU ? nout : 0) + 256, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = X; p.lda = ldx; p.B = Wf; p.ldb = ldw; p.Y = Y; p.ldy = ldy;
  p.M = (int)M; p.Nout = (int)nout; p.K = (int)K; p.up_offset = nout; p.a_src_rows = M;
  p.act = act == MTP_ACT_GELU ? 1 : 0;
  p.norm_stats = stats; p.norm_colsum = colsum; p.bias_f32 = bias_f;
  return launched(mtp::gemm(p, act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, (hipStream_t)stream,
                            mtp::EPI_NORM),
                  "norm column linear");
}

mtp_status mtp_fp8_quantize(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Xq, int64_t ldq,
                            float* amax_ws, float* scale_inv, void* stream) {
  TRY(check_dims(M, 8, K));
  TRY(check_mat(X, "X", K, ldx));
  TRY(check_mat(Xq, "Xq", K, ldq));
  if (!amax_ws || !scale_inv) return fail(MTP_ERR_NULL, "amax_ws and scale_inv are required");
  if ((reinterpret_cast<uintptr_t>(amax_ws) | reinterpret_cast<uintptr_t>(scale_inv)) & 3u)
    return fail(MTP_ERR_ALIGN, "amax_ws / scale_inv are not 4-byte aligned");
  if (M * (K / 8) >= ((int64_t)1 << 31)) return fail(MTP_ERR_SHAPE, "X has 2^34 or more elements");
  TRY(check_device());
  return launched(mtp::fp8_quantize(X, ldx, (int)M, (int)K, Xq, ldq, amax_ws, scale_inv, (hipStream_t)stream),
                  "fp8 quantize");
}

mtp_status mtp_fp8_quantize_delayed(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t K, uint8_t* Xq, int64_t ldq,
                                    float* amax_history, int history_len, int64_t step, float* ws, float* scale_inv,
                                    void* stream) {
  TRY(check_dims(M, 8, K));
  TRY(check_mat(X, "X", K, ldx));
  TRY(check_mat(Xq, "Xq", K, ldq));
  if (!amax_history || !ws || !scale_inv) return fail(MTP_ERR_NULL, "amax_history, ws and scale_inv are required");
  if ((reinterpret_cast<uintptr_t>(amax_history) | reinterpret_cast<uintptr_t>(ws) |
       reinterpret_cast<uintptr_t>(scale_inv)) & 3u)
    return fail(MTP_ERR_ALIGN, "amax_history / ws / scale_inv are not 4-byte aligned");
  if (history_len < 1 || history_len > 4096) return fail(MTP_ERR_SHAPE, "history_len %d is not in [1, 4096]", history_len);
  if (step < 0) return fail(MTP_ERR_SHAPE, "step %lld is negative", (long long)step);
  if (M * (K / 8) >= ((int64_t)1 << 31)) return fail(MTP_ERR_SHAPE, "X has 2^34 or more elements");
  TRY(check_device());
  return launched(mtp::fp8_quantize_delayed(X, ldx, (int)M, (int)K, Xq, ldq, amax_history, history_len, step, ws,
                                            scale_inv, (hipStream_t)stream),
                  "fp8 quantize (delayed scaling)");
}

// E4M3 operands: K, and the pitches in bytes, multiples of 16 (the kernels count pairs of codes)
static mtp_status check_f8(const void* p, const char* name, int64_t K, int64_t ld, const float* sinv,
                           const char* sname) {
  if (!p) return fail(MTP_ERR_NULL, "%s is NULL", name);
  if (misaligned(p)) return fail(MTP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  if (ld < K || ld % 16 != 0) return fail(MTP_ERR_SHAPE, "%s: pitch %lld must be >= %lld and a multiple of 16", name,
                                          (long long)ld, (long long)K);
  if (!sinv) return fail(MTP_ERR_NULL, "%s is NULL", sname);
  if (reinterpret_cast<uintptr_t>(sinv) & 3u) return fail(MTP_ERR_ALIGN, "%s is not 4-byte aligned", sname);
  return MTP_OK;
}

mtp_status mtp_fp8_column_linear(const uint8_t* Xq, int64_t ldx, const float* x_scale_inv, const uint8_t* Wq,
                                 int64_t ldw, const float* w_scale_inv, const mtp_bf16* bias, mtp_bf16* Y,
                                 int64_t ldy, int64_t M, int64_t N, int64_t K, mtp_act act,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, K));
  if (K % 16 != 0) return fail(MTP_ERR_SHAPE, "the inner dimension %lld is not a multiple of 16", (long long)K);
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  if (act == MTP_ACT_SWIGLU && N % 2 != 0) return fail(MTP_ERR_SHAPE, "SwiGLU needs an even N (got %lld)", (long long)N);
  const int64_t nout = act == MTP_ACT_SWIGLU ? N / 2 : N;
  TRY(check_f8(Xq, "Xq", K, ldx, x_scale_inv, "x_scale_inv"));
  TRY(check_f8(Wq, "Wq", K, ldw, w_scale_inv, "w_scale_inv"));
  TRY(check_mat(Y, "Y", nout, ldy));
  TRY(check_vec(bias, "bias"));
  TRY(check_window("Xq", 128, ldx));
  TRY(check_window("Wq", ((act == MTP_ACT_SWIGLU ? nout : 0) + 256) / 2 + 1, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = reinterpret_cast<const uint16_t*>(Xq); p.lda = ldx / 2;
  p.B = reinterpret_cast<const uint16_t*>(Wq); p.ldb = ldw / 2;
  p.bias = bias; p.Y = Y; p.ldy = ldy;
  p.M = (int)M; p.Nout = (int)nout; p.K = (int)(K / 2); p.up_offset = nout; p.a_src_rows = M;
  p.act = act == MTP_ACT_GELU ? 1 : 0;
  p.f8_scale_a = x_scale_inv; p.f8_scale_b = w_scale_inv;
  return launched(mtp::gemm_f8(p, act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, (hipStream_t)stream),
                  "fp8 column linear");
}

mtp_status mtp_fp8_row_linear_partial(const uint8_t* Zq, int64_t ldz, const float* z_scale_inv, const uint8_t* Wq,
                                      int64_t ldw, const float* w_scale_inv, float* Yacc, int64_t ldacc,
                                      int accumulate, const mtp_bf16* bias, mtp_bf16* Y, int64_t ldy, int64_t M,
                                      int64_t N, int64_t Kp, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dims(M, N, Kp));
  if (Kp % 16 != 0) return fail(MTP_ERR_SHAPE, "the inner dimension %lld is not a multiple of 16", (long long)Kp);
  TRY(check_f8(Zq, "Zq", Kp, ldz, z_scale_inv, "z_scale_inv"));
  TRY(check_f8(Wq, "Wq", Kp, ldw, w_scale_inv, "w_scale_inv"));
  if (!Yacc && !Y) return fail(MTP_ERR_NULL, "Yacc and Y are both NULL");
  if (!Yacc && accumulate) return fail(MTP_ERR_NULL, "accumulate needs Yacc");
  if (Yacc) TRY(check_mat(Yacc, "Yacc", N, ldacc));
  if (Y) TRY(check_mat(Y, "Y", N, ldy));
  TRY(check_vec(bias, "bias"));
  TRY(check_window("Zq", 128, ldz));
  TRY(check_window("Wq", 128, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = reinterpret_cast<const uint16_t*>(Zq); p.lda = ldz / 2;
  p.B = reinterpret_cast<const uint16_t*>(Wq); p.ldb = ldw / 2;
  p.Yacc = Yacc; p.ldacc = Yacc ? ldacc : 0; p.accumulate = accumulate ? 1 : 0;
  p.bias = bias; p.Y = Y; p.ldy = Y ? ldy : 0; p.M = (int)M; p.Nout = (int)N; p.K = (int)(Kp / 2); p.a_src_rows = M;
  p.f8_scale_a = z_scale_inv; p.f8_scale_b = w_scale_inv;
  return launched(mtp::gemm_f8(p, mtp::MODE_ROW, (hipStream_t)stream), "fp8 row-parallel partial");
}

mtp_status mtp_mlp_forward(const mtp_bf16* X, int64_t M, int64_t H, int64_t F, int p, int r0, int r1,
                           const mtp_bf16* W1t, const mtp_bf16* b1, const mtp_bf16* W2t, const mtp_bf16* b2,
                           mtp_act act, mtp_bf16* Z_ws, float* Yacc, mtp_bf16* Y,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (p < 1 || F < 1 || F % p != 0) return fail(MTP_ERR_SHAPE, "F=%lld must be a positive multiple of p=%d", (long long)F, p);
  if (r0 < 0 || r1 > p || r0 >= r1) return fail(MTP_ERR_SHAPE, "rank range [%d, %d) is not inside [0, %d)", r0, r1, p);
  if (act != MTP_ACT_NONE && act != MTP_ACT_GELU && act != MTP_ACT_SWIGLU)
    return fail(MTP_ERR_SHAPE, "unknown activation %d", (int)act);
  const int64_t Fl = F / p;
  const int64_t N1 = act == MTP_ACT_SWIGLU ? 2 * Fl : Fl;
  TRY(check_dims(M, N1, H));
  TRY(check_dims(M, H, Fl));
  if ((int64_t)p * N1 > kIntMax) return fail(MTP_ERR_SHAPE, "fc1 weight has too many rows");
  TRY(check_mat(X, "X", H, H));
  TRY(check_mat(W1t, "W1t", H, H));
  TRY(check_mat(W2t, "W2t", F, F));
  TRY(check_mat(Z_ws, "Z_ws", Fl, Fl));
  TRY(check_vec(b1, "b1"));
  TRY(check_vec(b2, "b2"));
  const bool full = r0 == 0 && r1 == p;
  if (!full && Y) return fail(MTP_ERR_SHAPE, "Y is written only when all p shards are computed");
  if (!Yacc && !(full && p == 1 && Y)) return fail(MTP_ERR_NULL, "Yacc is NULL");
  if (Yacc) TRY(check_mat(Yacc, "Yacc", H, H));
  if (Y) TRY(check_mat(Y, "Y", H, H));
  TRY(check_window("X", 256, H));
  TRY(check_window("W1t", (act == MTP_ACT_SWIGLU ? Fl : 0) + 256, H));
  TRY(check_window("W2t", 256, F));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  for (int r = r0; r < r1; ++r) {
    mtp::GemmParams f1;
    f1.ws = workspace; f1.ws_bytes = ws_avail;
    f1.A = X; f1.lda = H; f1.B = W1t + (int64_t)r * N1 * H; f1.ldb = H;
    f1.bias = b1 ? b1 + (int64_t)r * N1 : nullptr;
    f1.Y = Z_ws; f1.ldy = Fl; f1.M = (int)M; f1.Nout = (int)Fl; f1.K = (int)H; f1.up_offset = Fl; f1.a_src_rows = M;
    f1.act = act == MTP_ACT_GELU ? 1 : 0;
    mtp_status s = launched(mtp::gemm(f1, act == MTP_ACT_SWIGLU ? mtp::MODE_SWIGLU : mtp::MODE_COL, st), "fc1");
    if (s != MTP_OK) return s;
    mtp::GemmParams f2;
    f2.ws = workspace; f2.ws_bytes = ws_avail;
    f2.A = Z_ws; f2.lda = Fl; f2.B = W2t + (int64_t)r * Fl; f2.ldb = F;
    f2.Yacc = Yacc; f2.ldacc = H; f2.accumulate = r > r0 ? 1 : 0;
    const bool last = full && r == p - 1;
    f2.Y = last ? Y : nullptr; f2.ldy = H; f2.bias = last ? b2 : nullptr;
    f2.M = (int)M; f2.Nout = (int)H; f2.K = (int)Fl; f2.a_src_rows = M;
    s = launched(mtp::gemm(f2, mtp::MODE_ROW, st), "fc2");
    if (s != MTP_OK) return s;
  }
  return MTP_OK;
}

mtp_status mtp_qkv_forward(const mtp_bf16* X, int64_t ldx, int64_t M, int64_t H, const mtp_bf16* Wqkv_t, int64_t ldw,
                           const mtp_bf16* bias, int nq_local, int ng_local, int head_dim, mtp_bf16* QKV, int64_t ldo,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (nq_local < 1 || ng_local < 1 || head_dim < 1)
    return fail(MTP_ERR_SHAPE, "heads, groups and head_dim must be >= 1");
  if (nq_local % ng_local != 0)
    return fail(MTP_ERR_SHAPE, "query heads per rank (%d) must be a multiple of key/value groups per rank (%d)",
                nq_local, ng_local);
  const int64_t N = ((int64_t)nq_local + 2 * (int64_t)ng_local) * head_dim;
  return mtp_column_linear(X, ldx, Wqkv_t, ldw, bias, QKV, ldo, M, N, H, MTP_ACT_NONE, workspace, workspace_bytes,
                           stream);
}

mtp_status mtp_linear_dgrad(const mtp_bf16* dY, int64_t lddy, const mtp_bf16* Wt, int64_t ldw, float* dXacc,
                            int64_t ldacc, int accumulate, mtp_bf16* dX, int64_t lddx, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream) {
  // dX [M x K] = dY [M x N] . Wt [N x K]: the product C = A B^T with A = dY (contraction N along its rows'
  // columns) and B = Wt read row-major-K (its rows are the contraction index)
  TRY(check_dims(M, K, N));
  TRY(check_mat(dY, "dY", N, lddy));
  TRY(check_mat(Wt, "Wt", K, ldw));
  if (!dXacc && !dX) return fail(MTP_ERR_NULL, "dXacc and dX are both NULL");
  if (!dXacc && accumulate) return fail(MTP_ERR_NULL, "accumulate needs dXacc");
  if (dXacc) {
    if (misaligned(dXacc)) return fail(MTP_ERR_ALIGN, "dXacc is not 16-byte aligned");
    if (ldacc < K || ldacc % 8 != 0) return fail(MTP_ERR_SHAPE, "dXacc: pitch %lld must be >= %lld and a multiple of 8",
                                                 (long long)ldacc, (long long)K);
  }
  if (dX) TRY(check_mat(dX, "dX", K, lddx));
  TRY(check_window("dY", 256, lddy));
  TRY(check_window("Wt", N, ldw));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = dY; p.lda = lddy; p.B = Wt; p.ldb = ldw; p.Y = dX; p.ldy = dX ? lddx : 0; p.Yacc = dXacc;
  p.ldacc = dXacc ? ldacc : 0; p.accumulate = accumulate ? 1 : 0;
  p.M = (int)M; p.Nout = (int)K; p.K = (int)N; p.a_src_rows = M;
  return launched(mtp::gemm_backward(p, false, true, (hipStream_t)stream), "linear dgrad");
}

mtp_status mtp_linear_wgrad(const mtp_bf16* dY, int64_t lddy, const mtp_bf16* X, int64_t ldx, float* dW, int64_t lddw,
                            int accumulate, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream) {
  // dWt [N x K] (+)= dY^T [N x M] . X [M x K]: C = A B^T with A = dY and B = X both read row-major-K (their
  // rows are the contraction index M)
  if (M < 1 || N < 1 || K < 1) return fail(MTP_ERR_SHAPE, "sizes must be >= 1 (M=%lld N=%lld K=%lld)", (long long)M,
                                           (long long)N, (long long)K);
  if (M > kIntMax || N > kIntMax || K > kIntMax) return fail(MTP_ERR_SHAPE, "a size exceeds 2^31-1");
  TRY(check_mat(dY, "dY", N, lddy));
  TRY(check_mat(X, "X", K, ldx));
  if (!dW) return fail(MTP_ERR_NULL, "dW is NULL");
  if (misaligned(dW)) return fail(MTP_ERR_ALIGN, "dW is not 16-byte aligned");
  if (lddw < K || lddw % 8 != 0) return fail(MTP_ERR_SHAPE, "dW: pitch %lld must be >= %lld and a multiple of 8",
                                             (long long)lddw, (long long)K);
  TRY(check_window("dY", M, lddy));
  TRY(check_window("X", M, ldx));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  mtp::GemmParams p;
  p.ws = workspace; p.ws_bytes = ws_avail;
  p.A = dY; p.lda = lddy; p.B = X; p.ldb = ldx; p.Yacc = dW; p.ldacc = lddw; p.accumulate = accumulate ? 1 : 0;
  p.M = (int)N; p.Nout = (int)K; p.K = (int)M; p.a_src_rows = N;
  return launched(mtp::gemm_backward(p, true, true, (hipStream_t)stream), "linear wgrad");
}

mtp_status mtp_rope_qk(mtp_bf16* QKV, int64_t ldo, int64_t M, const int32_t* positions, int nq_local, int ng_local,
                       int head_dim, int rotary_dim, double base, int interleaved, void* stream) {
  if (!QKV || !positions) return fail(MTP_ERR_NULL, "QKV or positions is NULL");
  if (misaligned(QKV)) return fail(MTP_ERR_ALIGN, "QKV is not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(positions) & 3u) != 0) return fail(MTP_ERR_ALIGN, "positions is not 4-byte aligned");
  if (M < 1 || M > kIntMax) return fail(MTP_ERR_SHAPE, "M = %lld must be in [1, 2^31-1]", (long long)M);
  if (nq_local < 1 || ng_local < 1 || nq_local % ng_local != 0)
    return fail(MTP_ERR_SHAPE, "query heads per rank (%d) must be a positive multiple of key/value groups (%d)",
                nq_local, ng_local);
  if (head_dim < 8 || head_dim % 8 != 0) return fail(MTP_ERR_SHAPE, "head_dim %d must be a multiple of 8", head_dim);
  if (rotary_dim < 8 || rotary_dim % 8 != 0 || rotary_dim > head_dim || rotary_dim > 512)
    return fail(MTP_ERR_SHAPE, "rotary_dim %d must be a multiple of 8 in [8, min(head_dim, 512)]", rotary_dim);
  if (!(base > 1.0) || base > 1e300) return fail(MTP_ERR_SHAPE, "rotary base must be a finite number > 1");
  const int64_t width = ((int64_t)nq_local + 2 * (int64_t)ng_local) * head_dim;
  if (ldo < width || ldo % 8 != 0)
    return fail(MTP_ERR_SHAPE, "QKV: pitch %lld must be >= %lld and a multiple of 8", (long long)ldo, (long long)width);
  TRY(check_device());
  return launched(mtp::rope_qk(QKV, ldo, (int)M, positions, nq_local + ng_local, head_dim, rotary_dim, base,
                               interleaved != 0, (hipStream_t)stream),
                  "rope");
}

mtp_status mtp_moe_route(const float* logits, int64_t T, int E, int k, int32_t* expert_offsets, int32_t* token_idx,
                         float* token_w, int32_t* token_rows, void* stream) {
  if (!logits || !expert_offsets || !token_idx || !token_w || !token_rows)
    return fail(MTP_ERR_NULL, "a routing pointer is NULL");
  if (misaligned(logits) || misaligned(expert_offsets) || misaligned(token_idx) || misaligned(token_w) ||
      misaligned(token_rows))
    return fail(MTP_ERR_ALIGN, "routing arrays must be 16-byte aligned");
  if (E < 1 || E > mtp::kMaxExperts) return fail(MTP_ERR_SHAPE, "E=%d must be in [1, %d]", E, mtp::kMaxExperts);
  if (k < 1 || k > E || k > 8) return fail(MTP_ERR_SHAPE, "k=%d must be in [1, min(E, 8)]", k);
  if (T < 1 || T * k > kIntMax) return fail(MTP_ERR_SHAPE, "T=%lld out of range", (long long)T);
  TRY(check_device());
  return launched(mtp::moe_route(logits, (int)T, E, k, expert_offsets, token_idx, token_w, token_rows,
                                 (hipStream_t)stream),
                  "router");
}

mtp_status mtp_moe_mlp_forward(const mtp_bf16* X, int64_t T, int64_t H, int E, int64_t F, int k,
                               const int32_t* expert_offsets, const int32_t* token_idx, const float* token_w,
                               const int32_t* token_rows, const mtp_bf16* W1t, const mtp_bf16* W2t, mtp_bf16* Z_ws,
                               float* Y_rows, mtp_bf16* Y, void* workspace, size_t workspace_bytes, void* stream) {
  if (!expert_offsets || !token_idx || !token_w || !token_rows) return fail(MTP_ERR_NULL, "a routing table is NULL");
  if (misaligned(expert_offsets) || misaligned(token_idx) || misaligned(token_w) || misaligned(token_rows))
    return fail(MTP_ERR_ALIGN, "routing tables must be 16-byte aligned");
  if (E < 1 || E > mtp::kMaxExperts) return fail(MTP_ERR_SHAPE, "E=%d must be in [1, %d]", E, mtp::kMaxExperts);
  if (k < 1 || k > E || k > 8) return fail(MTP_ERR_SHAPE, "k=%d must be in [1, min(E, 8)]", k);
  TRY(check_dims(T, 2 * F, H));
  TRY(check_dims(T, H, F));
  if (T * k > kIntMax) return fail(MTP_ERR_SHAPE, "T*k exceeds 2^31-1");
  TRY(check_mat(X, "X", H, H));
  TRY(check_mat(W1t, "W1t", H, H));
  TRY(check_mat(W2t, "W2t", F, F));
  TRY(check_mat(Z_ws, "Z_ws", F, F));
  TRY(check_mat(Y_rows, "Y_rows", H, H));
  TRY(check_mat(Y, "Y", H, H));
  TRY(check_window("X", T, H));
  TRY(check_window("W1t", F + 256, H));
  TRY(check_window("W2t", 256, F));
  TRY(check_window("Z_ws", 256, F));
  size_t ws_avail = 0;
  TRY(check_ws(workspace, workspace_bytes, &ws_avail));
  TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  // grouped fc1: gather each dispatched row's token, SwiGLU epilogue -> Z_ws (dispatched order)
  mtp::GemmParams f1;
  f1.A = X; f1.lda = H; f1.a_rows = token_idx; f1.B = W1t; f1.ldb = H; f1.up_offset = F;
  f1.Y = Z_ws; f1.ldy = F; f1.Nout = (int)F; f1.K = (int)H; f1.a_src_rows = T;
  f1.group_offsets = expert_offsets; f1.groups = E; f1.group_stride_B = 2 * F * H;
  mtp_status s = launched(mtp::gemm_grouped(f1, mtp::MODE_SWIGLU, (int)(T * k), st), "grouped fc1");
  if (s != MTP_OK) return s;
  // grouped fc2: each dispatched row's fp32 output -> Y_rows
  mtp::GemmParams f2;
  f2.A = Z_ws; f2.lda = F; f2.B = W2t; f2.ldb = F; f2.Yacc = Y_rows; f2.ldacc = H;
  f2.Nout = (int)H; f2.K = (int)F; f2.a_src_rows = T * k;
  f2.group_offsets = expert_offsets; f2.groups = E; f2.group_stride_B = H * F;
  // split tails when the plan asks for them and the caller's workspace holds them
  const mtp::GroupedPlan pl = mtp::grouped_plan(mtp::MODE_ROW, T * k, E, H, F);
  const int chunks = pl.split_chunks > 1 && pl.ws_bytes <= ws_avail ? pl.split_chunks : 0;
  f2.ws = workspace; f2.ws_bytes = ws_avail;
  s = launched(mtp::gemm_grouped(f2, mtp::MODE_ROW, (int)(T * k), st, chunks), "grouped fc2");
  if (s != MTP_OK) return s;
  // weighted combine in each token's slot order, one bf16 rounding
  return launched(mtp::moe_combine(Y_rows, H, token_rows, token_w, (int)T, k, (int)H, Y, H, st), "combine");
}

mtp_status mtp_moe_plan(int64_t T, int64_t H, int E, int64_t F, int k, int* split_chunks, size_t* workspace_bytes) {
  if (!split_chunks || !workspace_bytes) return fail(MTP_ERR_NULL, "an output pointer is NULL");
  if (E < 1 || E > mtp::kMaxExperts) return fail(MTP_ERR_SHAPE, "E=%d must be in [1, %d]", E, mtp::kMaxExperts);
  if (k < 1 || k > E || k > 8) return fail(MTP_ERR_SHAPE, "k=%d must be in [1, min(E, 8)]", k);
  TRY(check_dims(T, 2 * F, H));
  TRY(check_dims(T, H, F));
  if (T * k > kIntMax) return fail(MTP_ERR_SHAPE, "T*k exceeds 2^31-1");
  TRY(check_device());
  const mtp::GroupedPlan pl = mtp::grouped_plan(mtp::MODE_ROW, T * k, E, H, F);
  *split_chunks = pl.split_chunks;
  *workspace_bytes = pl.ws_bytes;
  g_err[0] = 0;
  return MTP_OK;
}

mtp_status mtp_mfma_calibrate(float* out, int blocks, int iters, void* stream) {
  if (!out) return fail(MTP_ERR_NULL, "out is NULL");
  if (reinterpret_cast<uintptr_t>(out) & 3u) return fail(MTP_ERR_ALIGN, "out is not 4-byte aligned");
  if (blocks < 1 || iters < 1) return fail(MTP_ERR_SHAPE, "blocks and iters must be >= 1");
  TRY(check_device());
  return launched(mtp::mfma_calibrate(out, blocks, iters, (hipStream_t)stream), "mfma calibration");
}

}  // extern "C"
