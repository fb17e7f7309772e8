// Seeded synthetic input generator (device side).
//
// Test and benchmark infrastructure, not part of the layer library: fills
// device buffers with the exact bit patterns that synth/gen.c produces on the
// host for the same (seed, tensor shape, row block).  The definition is stated
// once, in gen.c; this file restates it for the GPU so that multi-gigabyte
// weight tensors need not cross PCIe.  Equality of the two sides is tested
// bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ double irwin_hall_z(uint64_t key, uint64_t e) {
  int64_t s = 0;
#pragma unroll
  for (uint64_t j = 0; j < 3; ++j) {
    uint64_t h = mix64(key + (3 * e + j + 1) * kGamma);
    s += (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
         (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48);
  }
  return (double)(s - 393210) * (1.0 / 65536.0);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// kind 0: normal bf16 (sigma), 1: ternary bf16, 2: normal fp32.
__global__ void fill_kernel(void* dst, int64_t ld, uint64_t key, double sigma, int64_t cols,
                            int64_t r0, int64_t nrows, int kind) {
  const int64_t total = nrows * cols;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t r = i / cols, c = i - r * cols;
    const uint64_t e = (uint64_t)(r0 + r) * (uint64_t)cols + (uint64_t)c;
    if (kind == 0) {
      double v = irwin_hall_z(key, e) * sigma;
      static_cast<uint16_t*>(dst)[r * ld + c] = f32_to_bf16_rne((float)v);
    } else if (kind == 1) {
      uint64_t h = mix64(key + (3 * e + 1) * kGamma);
      uint32_t t = (uint32_t)(((h >> 32) * 3) >> 32);
      static_cast<uint16_t*>(dst)[r * ld + c] = t == 0 ? 0xBF80u : (t == 1 ? 0x0000u : 0x3F80u);
    } else {
      static_cast<float*>(dst)[r * ld + c] = (float)irwin_hall_z(key, e);
    }
  }
}

int launch(void* dst, int64_t ld, uint64_t seed, double sigma, int64_t cols, int64_t r0,
           int64_t nrows, int kind, void* stream) {
  if (!dst || cols <= 0 || nrows < 0 || ld < cols || r0 < 0) return 1;
  if (nrows == 0) return 0;
  const int64_t total = nrows * cols;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, dst, ld,
                     mix64(seed + kGamma), sigma, cols, r0, nrows, kind);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {
// Rows [r0, r0 + nrows) of the tensor (.. x cols) with key `seed`, written at dst with row pitch ld
// (elements).  Returns 0 on success, 1 on bad arguments, 2 on launch failure.
int synth_gpu_normal_bf16(void* dst, int64_t ld, uint64_t seed, double sigma, int64_t cols,
                          int64_t r0, int64_t nrows, void* stream) {
  return launch(dst, ld, seed, sigma, cols, r0, nrows, 0, stream);
}
int synth_gpu_ternary_bf16(void* dst, int64_t ld, uint64_t seed, int64_t cols, int64_t r0,
                           int64_t nrows, void* stream) {
  return launch(dst, ld, seed, 0.0, cols, r0, nrows, 1, stream);
}
int synth_gpu_normal_f32(void* dst, int64_t ld, uint64_t seed, int64_t cols, int64_t r0,
                         int64_t nrows, void* stream) {
  return launch(dst, ld, seed, 0.0, cols, r0, nrows, 2, stream);
}
}
