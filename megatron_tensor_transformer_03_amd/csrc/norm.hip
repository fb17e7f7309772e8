// The norm prologue of a column-parallel linear, folded through the product.
//
// The layer normalizes its input before the QKV projection and before fc1 (LayerNorm, or RMSNorm for the
// LLaMA shapes; "快速入门", model implementation: the layer spec fuses the norm into the column-parallel QKV
// linear, and the LLaMA layer tree names input_layernorm / pre_mlp_layernorm).  With per-row statistics
// (mean_m, rstd_m), scale g and shift beta,
//   sum_k ((x_mk - mean_m) rstd_m g_k + beta_k) W_nk + b_n
//     = rstd_m (sum_k x_mk W'_nk - mean_m c_n) + b'_n,   W'_nk = g_k W_nk,  c_n = sum_k W'_nk,
//                                                          b'_n = b_n + sum_k beta_k W_nk,
// so the product runs on the raw input X and the normalization becomes a per-row affine map in the GEMM
// epilogue.  This file computes the two pieces around the product: the row statistics (one read of X) and
// the folded weight W' with c and b' (once per weight update).  c is summed from the rounded W' so that the
// centring term cancels exactly what the product accumulates.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "gemm.h"

namespace mtp {
namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Per-row (mean, rstd).  A wave holds its row in registers (CPL 16-byte chunks per lane, every load issued
// before the first use), so LayerNorm's second pass over the centred squares reads registers, not memory;
// rows wider than 24 chunks per lane (H > 12288) take the streaming form, which re-reads the row from the
// cache.  Each lane
// sums its chunks in order, then the wave adds the lanes' sums in a fixed butterfly: deterministic.
template <bool RMS, int CPL>
__global__ __launch_bounds__(64 * kRowsPerBlock) void stats_kernel(const uint16_t* __restrict__ X, int64_t ldx,
                                                                    int M, int H, float eps,
                                                                    float* __restrict__ stats) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= M) return;
  const uint4* x = reinterpret_cast<const uint4*>(X + (int64_t)row * ldx);
  const int chunks = H / 8;
  auto chunk_sum = [](const uint4& v) {
    return (lo_bf16(v.x) + hi_bf16(v.x)) + (lo_bf16(v.y) + hi_bf16(v.y)) + (lo_bf16(v.z) + hi_bf16(v.z)) +
           (lo_bf16(v.w) + hi_bf16(v.w));
  };
  auto chunk_sq = [](const uint4& v, float mean, float q) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float a = lo_bf16(w[t]) - mean, b = hi_bf16(w[t]) - mean;
      q = fmaf(a, a, q);
      q = fmaf(b, b, q);
    }
    return q;
  };
  float mean = 0.f, q = 0.f;
  if constexpr (CPL > 0) {
    uint4 v[CPL];
#pragma unroll
    for (int t = 0; t < CPL; ++t) {
      const int c = lane + 64 * t;
      v[t] = c < chunks ? x[c] : make_uint4(0, 0, 0, 0);  // zero chunks add nothing to the sums
    }
    if constexpr (!RMS) {
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < CPL; ++t) s += chunk_sum(v[t]);
      mean = wave_sum(s) / (float)H;
    }
#pragma unroll
    for (int t = 0; t < CPL; ++t)
      if (lane + 64 * t < chunks) q = chunk_sq(v[t], mean, q);
  } else {
    if constexpr (!RMS) {
      float s = 0.f;
      for (int c = lane; c < chunks; c += 64) s += chunk_sum(x[c]);
      mean = wave_sum(s) / (float)H;
    }
    for (int c = lane; c < chunks; c += 64) q = chunk_sq(x[c], mean, q);
  }
  const float var = wave_sum(q) / (float)H;
  if (lane == 0) {
    // 1 / sqrt in double: one per row
    const float rstd = (float)(1.0 / sqrt((double)var + (double)eps));
    *reinterpret_cast<float2*>(stats + 2 * (int64_t)row) = make_float2(mean, rstd);
  }
}

__device__ __forceinline__ uint32_t to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// One wave per weight row n: W'_nk = bf16(g_k W_nk), c_n = sum_k W'_nk, b'_n = b_n + sum_k beta_k W_nk.
__global__ __launch_bounds__(64 * kRowsPerBlock) void fold_kernel(const uint16_t* __restrict__ Wt, int64_t ldw,
                                                                   int N, int K, const uint16_t* __restrict__ gamma,
                                                                   const uint16_t* __restrict__ beta,
                                                                   const uint16_t* __restrict__ bias, int one_plus,
                                                                   uint16_t* __restrict__ Wf, int64_t ldwf,
                                                                   float* __restrict__ colsum,
                                                                   float* __restrict__ bias_f) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint4* w = reinterpret_cast<const uint4*>(Wt + (int64_t)n * ldw);
  const uint4* g = reinterpret_cast<const uint4*>(gamma);
  const uint4* bt = reinterpret_cast<const uint4*>(beta);
  uint4* out = reinterpret_cast<uint4*>(Wf + (int64_t)n * ldwf);
  const float g1 = one_plus ? 1.f : 0.f;
  float cs = 0.f, sb = 0.f;
  for (int c = lane; c < K / 8; c += 64) {
    const uint4 wv = w[c], gv = g[c];
    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w}, gg[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t a = to_bf16_rne((lo_bf16(gg[t]) + g1) * lo_bf16(ww[t]));
      const uint32_t b = to_bf16_rne((hi_bf16(gg[t]) + g1) * hi_bf16(ww[t]));
      cs += lo_bf16(a) + lo_bf16(b);
      o[t] = a | (b << 16);
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
    if (beta) {
      const uint4 bv = bt[c];
      const uint32_t bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sb = fmaf(lo_bf16(bb[t]), lo_bf16(ww[t]), sb);
        sb = fmaf(hi_bf16(bb[t]), hi_bf16(ww[t]), sb);
      }
    }
  }
  cs = wave_sum(cs);
  sb = wave_sum(sb);
  if (lane == 0) {
    if (colsum) colsum[n] = cs;
    bias_f[n] = sb + (bias ? __uint_as_float((uint32_t)bias[n] << 16) : 0.f);
  }
}

}  // namespace

hipError_t norm_stats(const uint16_t* X, int64_t ldx, int M, int H, int kind, float eps, float* stats,
                      hipStream_t st) {
  const dim3 grid((M + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  const int cpl = (H / 8 + 63) / 64;  // 16-byte chunks per lane
  auto go = [&](auto RMSC, auto CPLC) {
    hipLaunchKernelGGL((stats_kernel<decltype(RMSC)::value, decltype(CPLC)::value>), grid, block, 0, st, X, ldx, M,
                       H, eps, stats);
  };
  auto by_width = [&](auto RMSC) {
    if (cpl <= 1) go(RMSC, std::integral_constant<int, 1>{});
    else if (cpl <= 2) go(RMSC, std::integral_constant<int, 2>{});
    else if (cpl <= 4) go(RMSC, std::integral_constant<int, 4>{});
    else if (cpl <= 8) go(RMSC, std::integral_constant<int, 8>{});
    else if (cpl <= 16) go(RMSC, std::integral_constant<int, 16>{});
    else if (cpl <= 24) go(RMSC, std::integral_constant<int, 24>{});
    else go(RMSC, std::integral_constant<int, 0>{});
  };
  if (kind == 1) by_width(std::true_type{});
  else by_width(std::false_type{});
  return hipGetLastError();
}

hipError_t norm_fold(const uint16_t* Wt, int64_t ldw, int N, int K, const uint16_t* gamma, const uint16_t* beta,
                     const uint16_t* bias, int one_plus, uint16_t* Wf, int64_t ldwf, float* colsum, float* bias_f,
                     hipStream_t st) {
  const dim3 grid((N + kRowsPerBlock - 1) / kRowsPerBlock), block(64 * kRowsPerBlock);
  hipLaunchKernelGGL(fold_kernel, grid, block, 0, st, Wt, ldw, N, K, gamma, beta, bias, one_plus, Wf, ldwf, colsum,
                     bias_f);
  return hipGetLastError();
}

}  // namespace mtp
