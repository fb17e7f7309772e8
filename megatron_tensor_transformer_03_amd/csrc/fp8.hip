// Per-tensor E4M3 quantization of a bf16 tensor for the FP8 GEMMs ("快速入门", FP8 training: a scaling
// factor per tensor from its amax, E4M3 in the forward pass).  Two launches on the stream: per-block maxima
// of |x| into the scratch, then (every block reducing the partials to amax) scale, round and store the codes
// with the dequantization factor.  The
// scaling decisions are fp32 operations with IEEE rounding: s = 448 / amax, v = x * s, scale_inv = 1 / s.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {
namespace {

constexpr int kU = 4;  // chunks in flight per thread

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Per-block maxima of |x| (no atomics: the quantize kernel reduces the partials, which a single address
// could not take from a thousand blocks without serializing them).  Chunk c of the flat index is 8
// elements of row c / cpr.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ X, int64_t ldx, int cpr,
                                                   uint32_t total, float* __restrict__ part) {
  float m = 0.f;
  const uint32_t stride = gridDim.x * 256u;
  // kU chunks per thread per pass, all loads issued before the first use (one load in flight per thread
  // would leave the loop waiting on memory latency)
  for (uint32_t c0 = blockIdx.x * 256u + threadIdx.x; c0 < total; c0 += kU * stride) {
    uint4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u * stride;
      const uint32_t r = c / (uint32_t)cpr;
      v[u] = c < total ? *reinterpret_cast<const uint4*>(X + (int64_t)r * ldx + 8 * (c - r * (uint32_t)cpr))
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(lo_bf16(w[t])), fabsf(hi_bf16(w[t]))));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Two fp32 -> E4M3 codes (nearest, ties to even: gfx950's v_cvt_pk_fp8_f32 in the default round mode) into
// half `hi` of `old`; values are clamped to +-448 first, so the cast saturates (a value in (448, 464) rounds
// to 448 either way).  X must be finite.
__device__ __forceinline__ int cvt2(float a, float b, int old, int hi) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true) : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ X, int64_t ldx, int cpr,
                                                    uint32_t total, const float* __restrict__ part,
                                                    uint8_t* __restrict__ Q, int64_t ldq, float* scale_inv) {
  // amax: the maximum of the amax kernel's per-block partials (one per block of this grid)
  float m = 0.f;
  for (uint32_t b = threadIdx.x; b < gridDim.x; b += 256u) m = fmaxf(m, part[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = __fdiv_rn(1.f, s);
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t c0 = blockIdx.x * 256u + threadIdx.x; c0 < total; c0 += kU * stride) {
    uint4 v[kU];
    uint32_t rr[kU], kk[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u * stride;
      rr[u] = c / (uint32_t)cpr;
      kk[u] = 8 * (c - rr[u] * (uint32_t)cpr);
      v[u] = c < total ? *reinterpret_cast<const uint4*>(X + (int64_t)rr[u] * ldx + kk[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c0 + u * stride >= total) break;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      int o[2] = {0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t >> 1] = cvt2(__fmul_rn(lo_bf16(w[t]), s), __fmul_rn(hi_bf16(w[t]), s), o[t >> 1], t & 1);
      *reinterpret_cast<uint2*>(Q + (int64_t)rr[u] * ldq + kk[u]) = make_uint2((uint32_t)o[0], (uint32_t)o[1]);
    }
  }
}

// Delayed scaling: the scale comes from the max of an amax history (earlier steps), so one pass quantizes and
// takes this tensor's max |x| at once (per-block maxima into the scratch; record_kernel then writes their
// max into the history slot, after every block has read the history).
__global__ __launch_bounds__(256) void quant_delayed_kernel(const uint16_t* __restrict__ X, int64_t ldx, int cpr,
                                                            uint32_t total, const float* __restrict__ hist, int hlen,
                                                            uint8_t* __restrict__ Q, int64_t ldq, float* scale_inv,
                                                            float* __restrict__ part) {
  float hm = 0.f;
  for (int b = threadIdx.x; b < hlen; b += 256) hm = fmaxf(hm, hist[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) hm = fmaxf(hm, __shfl_xor(hm, o, 64));
  __shared__ float red[4], red2[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = hm;
  __syncthreads();
  const float hmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = hmax > 0.f ? __fdiv_rn(448.f, hmax) : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = __fdiv_rn(1.f, s);
  float m = 0.f;
  const uint32_t stride = gridDim.x * 256u;
  for (uint32_t c0 = blockIdx.x * 256u + threadIdx.x; c0 < total; c0 += kU * stride) {
    uint4 v[kU];
    uint32_t rr[kU], kk[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const uint32_t c = c0 + u * stride;
      rr[u] = c / (uint32_t)cpr;
      kk[u] = 8 * (c - rr[u] * (uint32_t)cpr);
      v[u] = c < total ? *reinterpret_cast<const uint4*>(X + (int64_t)rr[u] * ldx + kk[u]) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c0 + u * stride >= total) break;
      const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
      int o[2] = {0, 0};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float lo = lo_bf16(w[t]), hi = hi_bf16(w[t]);
        m = fmaxf(m, fmaxf(fabsf(lo), fabsf(hi)));
        o[t >> 1] = cvt2(__fmul_rn(lo, s), __fmul_rn(hi, s), o[t >> 1], t & 1);
      }
      *reinterpret_cast<uint2*>(Q + (int64_t)rr[u] * ldq + kk[u]) = make_uint2((uint32_t)o[0], (uint32_t)o[1]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red2[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red2[0], red2[1]), fmaxf(red2[2], red2[3]));
}

__global__ __launch_bounds__(256) void record_kernel(const float* __restrict__ part, int n, float* slot) {
  float m = 0.f;
  for (int b = threadIdx.x; b < n; b += 256) m = fmaxf(m, part[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) *slot = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

}  // namespace

hipError_t fp8_quantize(const uint16_t* X, int64_t ldx, int M, int K, uint8_t* Xq, int64_t ldq, float* ws,
                        float* scale_inv, hipStream_t st) {
  const uint32_t total = (uint32_t)((int64_t)M * (K / 8));
  const uint32_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < (uint32_t)kFp8QuantBlocks ? blocks : (uint32_t)kFp8QuantBlocks);
  hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(256), 0, st, X, ldx, K / 8, total, ws);
  hipLaunchKernelGGL(quant_kernel, dim3(grid), dim3(256), 0, st, X, ldx, K / 8, total, ws, Xq, ldq, scale_inv);
  return hipGetLastError();
}

hipError_t fp8_quantize_delayed(const uint16_t* X, int64_t ldx, int M, int K, uint8_t* Xq, int64_t ldq, float* hist,
                                int hlen, int64_t step, float* ws, float* scale_inv, hipStream_t st) {
  const uint32_t total = (uint32_t)((int64_t)M * (K / 8));
  const uint32_t blocks = (total + 255) / 256;
  const int grid = (int)(blocks < (uint32_t)kFp8QuantBlocks ? blocks : (uint32_t)kFp8QuantBlocks);
  hipLaunchKernelGGL(quant_delayed_kernel, dim3(grid), dim3(256), 0, st, X, ldx, K / 8, total, hist, hlen, Xq, ldq,
                     scale_inv, ws);
  hipLaunchKernelGGL(record_kernel, dim3(1), dim3(256), 0, st, ws, grid, hist + step % hlen);
  return hipGetLastError();
}

}  // namespace mtp
