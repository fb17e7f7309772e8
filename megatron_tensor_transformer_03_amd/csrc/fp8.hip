// Per-tensor E4M3 quantization of a bf16 tensor for the FP8 GEMMs ("快速入门", FP8 training: a scaling
// factor per tensor from its amax, E4M3 in the forward pass).  Two launches on the stream: per-block maxima
// of |x| into the scratch, then (every block reducing the partials to amax) scale, round and store the codes
// with the dequantization factor.  The scaling decisions are fp32 operations with IEEE rounding:
// s = 448 / amax (1 unless amax > 0), v = x * s, scale_inv = 1 / s.
// Non-finite inputs follow the same fp32 arithmetic: max |x| is taken on the bit patterns (for a sign-cleared
// bf16 or fp32, integer order is magnitude order with NaN above infinity), so a NaN anywhere makes amax NaN
// and then s = 1; an infinity makes s = 0; and a product that is NaN (a NaN input, or inf * 0) is stored as
// the E4M3 NaN code S.1111.111 rather than clamped.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {
namespace {

constexpr int kU = 4;  // chunks in flight per thread

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// max |x| over the two bf16 of a word, as fp32 bits (sign cleared: integer order, NaN above infinity)
__device__ __forceinline__ uint32_t abs_max_bits(uint32_t w) {
  const uint32_t lo = (w & 0x7FFFu) << 16, hi = w & 0x7FFF0000u;
  return lo > hi ? lo : hi;
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
// NaN-propagating maximum of two fp32 values (fmaxf would drop a NaN)
__device__ __forceinline__ float nanmax(float a, float b) { return (a > b || a != a) ? a : b; }
// Maximum over the block of per-thread fp32 bit patterns of non-negative values (or NaN), in `red[4]`.
__device__ __forceinline__ uint32_t block_max_bits(uint32_t m, uint32_t* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = umax(m, (uint32_t)__shfl_xor((int)m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  return umax(umax(red[0], red[1]), umax(red[2], red[3]));
}

// Per-block maxima of |x| (no atomics: the quantize kernel reduces the partials, which a single address
// could not take from a thousand blocks without serializing them).  Chunk c of the flat index is 8
// elements of row c / cpr.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ X, int64_t ldx, int cpr,
                                                   uint32_t total, float* __restrict__ part) {
  uint32_t m = 0;
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
    for (int u = 0; u < kU; ++u)
      m = umax(m, umax(umax(abs_max_bits(v[u].x), abs_max_bits(v[u].y)), umax(abs_max_bits(v[u].z), abs_max_bits(v[u].w))));
  }
  __shared__ uint32_t red[4];
  const uint32_t bm = block_max_bits(m, red);
  if (threadIdx.x == 0) part[blockIdx.x] = __uint_as_float(bm);
}

// Two fp32 -> E4M3 codes (nearest, ties to even: gfx950's v_cvt_pk_fp8_f32 in the default round mode) into
// half `hi` of `old`; values are clamped to +-448 first, so the cast saturates (a value in (448, 464) rounds
// to 448 either way), and a NaN value becomes the NaN code S.1111.111 (the clamp would turn it into -448).
__device__ __forceinline__ int cvt2(float a, float b, int old, int hi) {
  const float ca = fminf(fmaxf(a, -448.f), 448.f);
  const float cb = fminf(fmaxf(b, -448.f), 448.f);
  uint32_t r = (uint32_t)(hi ? __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, old, true)
                             : __builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, old, false));
  const int sa = hi ? 16 : 0, sb = hi ? 24 : 8;
  if (a != a) r = (r & ~(0xFFu << sa)) | ((0x7Fu | ((__float_as_uint(a) >> 24) & 0x80u)) << sa);
  if (b != b) r = (r & ~(0xFFu << sb)) | ((0x7Fu | ((__float_as_uint(b) >> 24) & 0x80u)) << sb);
  return (int)r;
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ X, int64_t ldx, int cpr,
                                                    uint32_t total, const float* __restrict__ part,
                                                    uint8_t* __restrict__ Q, int64_t ldq, float* scale_inv) {
  // amax: the maximum of the amax kernel's per-block partials (one per block of this grid; bit patterns of
  // non-negative values or NaN, compared as integers)
  uint32_t m = 0;
  for (uint32_t b = threadIdx.x; b < gridDim.x; b += 256u) m = umax(m, __float_as_uint(part[b]));
  __shared__ uint32_t red[4];
  const float amax = __uint_as_float(block_max_bits(m, red));
  const float s = amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f;  // (NaN > 0 is false: s = 1)
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
  // the history's maximum, NaN-propagating (the history holds the caller's values, any sign)
  float hm = hlen > 0 ? hist[0] : 0.f;
  for (int b = threadIdx.x; b < hlen; b += 256) hm = nanmax(hm, hist[b]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) hm = nanmax(hm, __shfl_xor(hm, o, 64));
  __shared__ float red[4];
  __shared__ uint32_t red2[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = hm;
  __syncthreads();
  const float hmax = nanmax(nanmax(red[0], red[1]), nanmax(red[2], red[3]));
  const float s = hmax > 0.f ? __fdiv_rn(448.f, hmax) : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = __fdiv_rn(1.f, s);
  uint32_t m = 0;
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
        m = umax(m, abs_max_bits(w[t]));
        o[t >> 1] = cvt2(__fmul_rn(lo_bf16(w[t]), s), __fmul_rn(hi_bf16(w[t]), s), o[t >> 1], t & 1);
      }
      *reinterpret_cast<uint2*>(Q + (int64_t)rr[u] * ldq + kk[u]) = make_uint2((uint32_t)o[0], (uint32_t)o[1]);
    }
  }
  const uint32_t bm = block_max_bits(m, red2);
  if (threadIdx.x == 0) part[blockIdx.x] = __uint_as_float(bm);
}

__global__ __launch_bounds__(256) void record_kernel(const float* __restrict__ part, int n, float* slot) {
  uint32_t m = 0;
  for (int b = threadIdx.x; b < n; b += 256) m = umax(m, __float_as_uint(part[b]));
  __shared__ uint32_t red[4];
  const uint32_t bm = block_max_bits(m, red);
  if (threadIdx.x == 0) *slot = __uint_as_float(bm);
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
