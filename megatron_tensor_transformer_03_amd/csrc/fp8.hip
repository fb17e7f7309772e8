// Per-tensor E4M3 quantization of a bf16 tensor for the FP8 GEMMs ("快速入门", FP8 training: a scaling
// factor per tensor from its amax, E4M3 in the forward pass).  Three launches on the stream: clear the amax
// cell, reduce max |x| into it (an integer max on the fp32 bit patterns, which order like the values for
// non-negative floats), then scale, round and store the codes with the dequantization factor.  The
// scaling decisions are fp32 operations with IEEE rounding: s = 448 / amax, v = x * s, scale_inv = 1 / s.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {
namespace {

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__global__ void clear_kernel(float* amax) { *amax = 0.f; }

// Each thread takes 8-element chunks of rows; the block reduces through LDS, then one atomic per block.
__global__ __launch_bounds__(256) void amax_kernel(const uint16_t* __restrict__ X, int64_t ldx, int M, int K,
                                                   float* amax) {
  const int cpr = K / 8;
  const int64_t total = (int64_t)M * cpr;
  float m = 0.f;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / cpr;
    const uint4 v = *reinterpret_cast<const uint4*>(X + r * ldx + 8 * (c - r * cpr));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) m = fmaxf(m, fmaxf(fabsf(lo_bf16(w[t])), fabsf(hi_bf16(w[t]))));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
  }
}

// fp32 -> E4M3, nearest with ties to even, saturating at +-448; NaN -> S.1111.111.
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // |v| >= 448
  if (a < 0x3C800000u) {                      // |v| < 2^-6: multiples of 2^-9 (8 -> the first normal, code 8)
    return sign | (uint32_t)rintf(__uint_as_float(a) * 512.f);
  }
  int e = (int)(a >> 23) - 127;               // -6 .. 8
  uint32_t keep = (a >> 20) & 7u;
  const uint32_t rest = a & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) ++keep;
  if (keep == 8u) { keep = 0; ++e; }          // (448 <= |v| is excluded above, so e stays <= 8 here)
  return sign | ((uint32_t)(e + 7) << 3) | keep;
}

__global__ __launch_bounds__(256) void quant_kernel(const uint16_t* __restrict__ X, int64_t ldx, int M, int K,
                                                    const float* amax_p, uint8_t* __restrict__ Q, int64_t ldq,
                                                    float* scale_inv) {
  const float amax = *amax_p;
  const float s = amax > 0.f ? __fdiv_rn(448.f, amax) : 1.f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *scale_inv = __fdiv_rn(1.f, s);
  const int cpr = K / 8;
  const int64_t total = (int64_t)M * cpr;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = c / cpr, k = 8 * (c - r * cpr);
    const uint4 v = *reinterpret_cast<const uint4*>(X + r * ldx + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0, 0};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const uint32_t a = e4m3_rne(__fmul_rn(lo_bf16(w[t]), s)), b = e4m3_rne(__fmul_rn(hi_bf16(w[t]), s));
      o[t >> 1] |= (a | (b << 8)) << (16 * (t & 1));
    }
    *reinterpret_cast<uint2*>(Q + r * ldq + k) = make_uint2(o[0], o[1]);
  }
}

}  // namespace

hipError_t fp8_quantize(const uint16_t* X, int64_t ldx, int M, int K, uint8_t* Xq, int64_t ldq, float* amax_ws,
                        float* scale_inv, hipStream_t st) {
  const int64_t chunks = (int64_t)M * (K / 8);
  const int grid = (int)(chunks / 256 + 1 < 4096 ? chunks / 256 + 1 : 4096);
  hipLaunchKernelGGL(clear_kernel, dim3(1), dim3(1), 0, st, amax_ws);
  hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(256), 0, st, X, ldx, M, K, amax_ws);
  hipLaunchKernelGGL(quant_kernel, dim3(grid), dim3(256), 0, st, X, ldx, M, K, amax_ws, Xq, ldq, scale_inv);
  return hipGetLastError();
}

}  // namespace mtp
