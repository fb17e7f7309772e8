// Rotary position embedding of the query and key heads of one rank's QKV output, in place.
//
// The pages list RoPE among the layer's fused elementwise kernels applied to the QKV output
// ("Megatron-LM 深度学习与源码分析文档", part 2 sections 3 and 6: --use-rotary-position-embeddings,
// --use-fused-rotary-pos-emb, rotary_base, rotary_percent); the rotation is RoFormer's: the pair (x_a, x_b)
// of frequency theta_j = base^(-2j / rotary_dim) at position m becomes
// (x_a cos(m theta_j) - x_b sin(m theta_j), x_b cos(m theta_j) + x_a sin(m theta_j)), with b = a + rotary_dim/2
// (rotate half) or b = a + 1 (interleaved); dimensions from rotary_dim on are left alone.
//
// HBM-bound: every Q and K element is read and written once (4 bytes per element); cos/sin depend only on
// (row, pair) and are computed once per row into LDS, shared by all heads.  The angle m theta_j is formed and
// reduced to [-pi, pi] in double precision, then cos/sin are taken in single precision, so the rotation is
// accurate to a few fp32 ulps at any position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {
namespace {

constexpr int kRows = 4;       // rows per workgroup
constexpr int kThreads = 256;
constexpr int kMaxHalf = 256;  // rotary_dim / 2 <= 256

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));  // round to nearest even
}

template <bool INTERLEAVED>
__global__ __launch_bounds__(kThreads) void rope_kernel(uint16_t* __restrict__ qkv, int64_t ldo, int M,
                                                        const int32_t* __restrict__ positions, int heads,
                                                        int head_dim, int rotary_dim, double log2_base) {
  __shared__ float cs[kRows][kMaxHalf], sn[kRows][kMaxHalf];
  const int half = rotary_dim / 2;
  const int row0 = blockIdx.x * kRows;
  // cos/sin table of this workgroup's rows
  for (int t = threadIdx.x; t < kRows * half; t += kThreads) {
    const int r = t / half, j = t - r * half;
    const int row = row0 + r;
    float c = 1.f, s = 0.f;
    if (row < M) {
      const double theta = exp2(-2.0 * j / rotary_dim * log2_base);
      const double ang = (double)positions[row] * theta;
      const double red = ang - 6.283185307179586476925 * rint(ang * 0.15915494309189533576888);
      sincosf((float)red, &s, &c);
    }
    cs[r][j] = c;
    sn[r][j] = s;
  }
  __syncthreads();
  // items: (row, head, group of 4 pairs)
  const int groups = half / 4;
  const int per_row = heads * groups;
  for (int t = threadIdx.x; t < kRows * per_row; t += kThreads) {
    const int r = t / per_row, rem = t - r * per_row;
    const int row = row0 + r;
    if (row >= M) break;  // rows are in order within the workgroup: the rest are past M too
    const int h = rem / groups, g = rem - h * groups;
    uint16_t* base = qkv + (int64_t)row * ldo + (int64_t)h * head_dim;
    const int j0 = 4 * g;
    if constexpr (INTERLEAVED) {
      uint4* p = reinterpret_cast<uint4*>(base + 8 * g);
      const uint4 v = *p;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float xa = bf((uint16_t)w[q]), xb = bf((uint16_t)(w[q] >> 16));
        const float c = cs[r][j0 + q], s = sn[r][j0 + q];
        o[q] = pack2(xa * c - xb * s, xb * c + xa * s);
      }
      *p = make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      uint2* pa = reinterpret_cast<uint2*>(base + j0);
      uint2* pb = reinterpret_cast<uint2*>(base + half + j0);
      const uint2 va = *pa, vb = *pb;
      const float a[4] = {bf((uint16_t)va.x), bf((uint16_t)(va.x >> 16)), bf((uint16_t)va.y), bf((uint16_t)(va.y >> 16))};
      const float b[4] = {bf((uint16_t)vb.x), bf((uint16_t)(vb.x >> 16)), bf((uint16_t)vb.y), bf((uint16_t)(vb.y >> 16))};
      float ya[4], yb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float c = cs[r][j0 + q], s = sn[r][j0 + q];
        ya[q] = a[q] * c - b[q] * s;
        yb[q] = b[q] * c + a[q] * s;
      }
      *pa = make_uint2(pack2(ya[0], ya[1]), pack2(ya[2], ya[3]));
      *pb = make_uint2(pack2(yb[0], yb[1]), pack2(yb[2], yb[3]));
    }
  }
}

}  // namespace

hipError_t rope_qk(uint16_t* qkv, int64_t ldo, int M, const int32_t* positions, int heads, int head_dim,
                   int rotary_dim, double base, bool interleaved, hipStream_t st) {
  if (M <= 0) return hipSuccess;
  if (rotary_dim / 2 > kMaxHalf) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((M + kRows - 1) / kRows));
  const double l2b = log2(base);
  if (interleaved)
    hipLaunchKernelGGL(rope_kernel<true>, grid, dim3(kThreads), 0, st, qkv, ldo, M, positions, heads, head_dim,
                       rotary_dim, l2b);
  else
    hipLaunchKernelGGL(rope_kernel<false>, grid, dim3(kThreads), 0, st, qkv, ldo, M, positions, heads, head_dim,
                       rotary_dim, l2b);
  return hipGetLastError();
}

}  // namespace mtp
