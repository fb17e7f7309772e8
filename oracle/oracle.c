/*
 * CPU oracle for one tensor-parallel rank's Transformer-layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the GPU library and is deliberately plain and slow: a triple loop in fp64
 * over bf16 inputs widened exactly, k ascending, no fused multiply-add
 * (built with -ffp-contract=off), activations from libm in double.
 *
 * Sources (page titles as published):
 *  - "Megatron-LM 深度学习与源码分析文档", part 2 (核心并行技术), section 2
 *    (Tensor Parallel): Y = XW; the column split W = [W1..Wp] with
 *    Y_i = X W_i and Y = [Y_1..Y_p]; the row split with Y_i = X_i W_i and
 *    Y = sum_i Y_i; [Q,K,V] = X W_qkv with heads/TP per rank; the MLP
 *    Z = phi(X W1), Y = Z W2.
 *  - "ai阅读megatron", TransformerConfig: activation_func = F.gelu (the erf
 *    form), gated_linear_unit; ColumnParallelLinear / RowParallelLinear
 *    forward pseudo-code: F.linear(x, weight), i.e. weights stored
 *    [out x in].
 *  - "快速入门" (Pai-Megatron-Patch), section 5.1 weight mapping: linear_fc1
 *    holds gate_proj in its first half and up_proj in its second half.
 *
 * Every function here is pinned by tests/test_oracle_pins.py against exact
 * rational arithmetic, closed forms and textbook values.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <string.h>

enum { ACT_NONE = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a double to the nearest bf16, ties to even, in one step (no
 * intermediate float).  Overflow goes to infinity, NaN stays NaN. */
uint16_t oracle_f64_to_bf16(double x) {
  if (isnan(x)) return 0x7FC0u;
  uint16_t sign = signbit(x) ? 0x8000u : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
  /* bf16 normal numbers carry 8 significant bits; below 2^-126 the spacing is 2^-133. */
  int q = e - 8;
  if (q < -133) q = -133;
  double step = ldexp(1.0, q);
  double n = a / step; /* exact: a has 53 bits, dividing by a power of two */
  double fl = floor(n);
  double rem = n - fl;
  if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
  double r = fl * step;
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80u;
  float f = (float)r; /* exact: r is a bf16 value */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

double oracle_gelu(double x) { return 0.5 * x * (1.0 + erf(x / sqrt(2.0))); }

double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/*
 * The column-parallel linear of one shard, in full precision:
 *   pre[i][j] = sum_{k<K} X[i][k] * Wt[j][k]  (+ bias[j])
 *   NONE:   Y[i][j] = pre[i][j]                         (Nout = N)
 *   GELU:   Y[i][j] = gelu(pre[i][j])                   (Nout = N)
 *   SWIGLU: Y[i][j] = silu(pre[i][j]) * pre[i][N/2 + j] (Nout = N/2; rows of
 *           Wt are [gate ; up])
 * X is [M x K] with row pitch ldx, Wt is [N x K] with pitch ldw (weights
 * stored [out x in]), bias is NULL or [N], Y is [M x Nout] fp64 with pitch ldy.
 */
void oracle_linear(const uint16_t *X, int64_t ldx, const uint16_t *Wt, int64_t ldw,
                   const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K, double *Y,
                   int64_t ldy) {
  const int64_t nout = act == ACT_SWIGLU ? N / 2 : N;
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < nout; ++j) {
      double pre = 0.0;
      for (int64_t k = 0; k < K; ++k)
        pre += oracle_bf16_to_f64(X[i * ldx + k]) * oracle_bf16_to_f64(Wt[j * ldw + k]);
      if (bias) pre += oracle_bf16_to_f64(bias[j]);
      if (act == ACT_NONE) {
        Y[i * ldy + j] = pre;
      } else if (act == ACT_GELU) {
        Y[i * ldy + j] = oracle_gelu(pre);
      } else {
        const int64_t ju = nout + j;
        double up = 0.0;
        for (int64_t k = 0; k < K; ++k)
          up += oracle_bf16_to_f64(X[i * ldx + k]) * oracle_bf16_to_f64(Wt[ju * ldw + k]);
        if (bias) up += oracle_bf16_to_f64(bias[ju]);
        Y[i * ldy + j] = oracle_silu(pre) * up;
      }
    }
  }
}

/* The same product over an fp64 left operand A [M x K] (normalized activations kept in fp64). */
void oracle_linear_f64(const double *A, int64_t lda, const uint16_t *Wt, int64_t ldw, const uint16_t *bias,
                       int act, int64_t M, int64_t N, int64_t K, double *Y, int64_t ldy) {
  const int64_t nout = act == ACT_SWIGLU ? N / 2 : N;
#pragma omp parallel for collapse(2) schedule(dynamic, 64)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < nout; ++j) {
      double pre = 0.0;
      for (int64_t k = 0; k < K; ++k) pre += A[i * lda + k] * oracle_bf16_to_f64(Wt[j * ldw + k]);
      if (bias) pre += oracle_bf16_to_f64(bias[j]);
      if (act == ACT_NONE) {
        Y[i * ldy + j] = pre;
      } else if (act == ACT_GELU) {
        Y[i * ldy + j] = oracle_gelu(pre);
      } else {
        const int64_t ju = nout + j;
        double up = 0.0;
        for (int64_t k = 0; k < K; ++k) up += A[i * lda + k] * oracle_bf16_to_f64(Wt[ju * ldw + k]);
        if (bias) up += oracle_bf16_to_f64(bias[ju]);
        Y[i * ldy + j] = oracle_silu(pre) * up;
      }
    }
  }
}

/* Round an fp64 [rows x cols] array to bf16 (the stored precision of the
 * intermediate activation Z between fc1 and fc2). */
void oracle_round_bf16(const double *src, int64_t n, uint16_t *dst) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) dst[i] = oracle_f64_to_bf16(src[i]);
}

/* Threads an OpenMP loop of this library uses (for reporting the CPU baseline's core count). */
int oracle_num_threads(void) { return omp_get_max_threads(); }
