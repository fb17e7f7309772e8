// MoE routing and small elementwise kernels.
//
// Router ("ai阅读megatron", MoELayer forward: router logits -> top-k ->
// dispatch -> weighted combine): per token, softmax over the E experts in fp32 and the k largest
// logits (softmax is monotone, so this is the k most probable experts; ties go
// to the lower expert index).  The dispatch tables group rows by expert in
// ascending expert order and keep tokens ascending within an expert, which
// needs a stable scatter: one workgroup walks the tokens in 1024-token
// chunks, ranks each token within its expert by wave ballots plus an
// across-wave prefix, and carries the running per-expert base between chunks.
// Each token's logits are read once into registers.  The work is O(T * E); it is not a GEMM.  The router
// also records, for each token, the dispatched row of each of its k choices (most probable first): the
// combine reads a token's k expert outputs through it in that fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"

namespace mtp {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxTopK = 8;

struct Choice {
  uint64_t mask;        // bit e set if expert e was chosen
  int e[kMaxTopK];      // chosen experts, most probable first
  float w[kMaxTopK];    // their softmax probabilities
};

// Softmax + top-k of one token whose logits are in registers (EMAX a compile-time capacity >= E, so every
// index below is static and nothing spills to scratch).  Selection compares the logits themselves (softmax
// is monotone); ties go to the lower expert index.
template <int EMAX>
__device__ __forceinline__ void choose(const float (&lg)[EMAX], int E, int k, Choice& c) {
  float mx = lg[0];
#pragma unroll
  for (int e = 1; e < EMAX; ++e)
    if (e < E) mx = fmaxf(mx, lg[e]);
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < EMAX; ++e)
    if (e < E) sum += expf(lg[e] - mx);
  c.mask = 0;
#pragma unroll
  for (int s = 0; s < kMaxTopK; ++s) {
    c.e[s] = -1;
    c.w[s] = 0.f;
    if (s < k) {
      int best = -1;
      float bv = 0.f;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (e >= E || ((c.mask >> e) & 1ull)) continue;
        const float v = lg[e];
        if (best < 0 || v > bv) { best = e; bv = v; }
      }
      c.mask |= 1ull << best;
      c.e[s] = best;
      c.w[s] = expf(bv - mx) / sum;
    }
  }
}

// The token's E logits into registers, read together (16-byte loads when the row allows).
template <int EMAX>
__device__ __forceinline__ void load_logits(const float* __restrict__ row, int E, float (&lg)[EMAX]) {
  if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(row) & 15) == 0) {
#pragma unroll
    for (int e = 0; e < EMAX; e += 4) {
      float4 v = e < E ? *reinterpret_cast<const float4*>(row + e) : make_float4(0.f, 0.f, 0.f, 0.f);
      lg[e] = v.x; lg[e + 1] = v.y; lg[e + 2] = v.z; lg[e + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) lg[e] = e < E ? row[e] : 0.f;
  }
}

template <int EMAX>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ token_idx,
                                                              float* __restrict__ token_w,
                                                              int32_t* __restrict__ token_rows) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kMaxExperts][kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < kMaxExperts) cnt[tid] = 0;
  __syncthreads();
  // pass 1: tokens per expert (integer sums: order-free)
  for (int t = tid; t < T; t += kRouteThreads) {
    float lg[EMAX];
    load_logits(logits + (int64_t)t * E, E, lg);
    Choice c;
    choose(lg, E, k, c);
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s)
      if (s < k) atomicAdd(&cnt[c.e[s]], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int e = 0; e < E; ++e) {
      offsets[e] = run;
      base[e] = run;
      run += cnt[e];
    }
    offsets[E] = run;
  }
  __syncthreads();
  // pass 2: stable scatter, 1024 tokens at a time; all lanes stay converged for the ballots
  const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < T; c0 += kRouteThreads) {
    const int t = c0 + tid;
    Choice c;
    c.mask = 0;
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) { c.e[s] = -1; c.w[s] = 0.f; }
    if (t < T) {
      float lg[EMAX];
      load_logits(logits + (int64_t)t * E, E, lg);
      choose(lg, E, k, c);
    }
    int rank[kMaxTopK];
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) rank[s] = 0;
    for (int e = 0; e < E; ++e) {
      const bool mine = (c.mask >> e) & 1ull;
      const uint64_t b = __ballot(mine);
      if (lane == 0) wcnt[e][wave] = __popcll(b);
      const int r = __popcll(b & lt_mask);
#pragma unroll
      for (int s = 0; s < kMaxTopK; ++s)
        if (c.e[s] == e) rank[s] = r;
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kMaxTopK; ++s) {
      if (s < k && t < T) {
        const int e = c.e[s];
        int pos = base[e] + rank[s];
        for (int w = 0; w < wave; ++w) pos += wcnt[e][w];
        token_idx[pos] = t;
        token_w[pos] = c.w[s];
        token_rows[(int64_t)t * k + s] = pos;
      }
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < kRouteWaves; ++w) add += wcnt[tid][w];
      base[tid] += add;
    }
    __syncthreads();
  }
}

// The weighted combine, token-major: thread i owns 4 consecutive columns of one token and adds the token's k
// expert outputs in slot order (fp32 fused multiply-adds in a fixed order, so the result does not depend on
// scheduling), then rounds once to bf16.  HBM-bound: T k H fp32 read, T H bf16 written.
__global__ void combine_kernel(const float* __restrict__ rows, int64_t ldr, const int32_t* __restrict__ token_rows,
                               const float* __restrict__ token_w, int T, int k, int H4,
                               uint16_t* __restrict__ out, int64_t ldo) {
  const int64_t total = (int64_t)T * H4;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / H4;
    const int c = 4 * (int)(i - t * H4);
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < k; ++s) {
      const int r = token_rows[t * k + s];
      const float w = token_w[r];
      const float4 y = *reinterpret_cast<const float4*>(rows + (int64_t)r * ldr + c);
      v.x = fmaf(w, y.x, v.x); v.y = fmaf(w, y.y, v.y); v.z = fmaf(w, y.z, v.z); v.w = fmaf(w, y.w, v.w);
    }
    const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v.x) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
    const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v.z) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
    *reinterpret_cast<uint2*>(out + t * ldo + c) = make_uint2(lo, hi);
  }
}

static unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

hipError_t moe_route(const float* logits, int T, int E, int k, int32_t* offsets, int32_t* token_idx, float* token_w,
                     int32_t* token_rows, hipStream_t st) {
  if (E <= 8)
    hipLaunchKernelGGL(route_kernel<8>, dim3(1), dim3(kRouteThreads), 0, st, logits, T, E, k, offsets, token_idx, token_w,
                       token_rows);
  else if (E <= 16)
    hipLaunchKernelGGL(route_kernel<16>, dim3(1), dim3(kRouteThreads), 0, st, logits, T, E, k, offsets, token_idx, token_w,
                       token_rows);
  else if (E <= 32)
    hipLaunchKernelGGL(route_kernel<32>, dim3(1), dim3(kRouteThreads), 0, st, logits, T, E, k, offsets, token_idx, token_w,
                       token_rows);
  else
    hipLaunchKernelGGL(route_kernel<64>, dim3(1), dim3(kRouteThreads), 0, st, logits, T, E, k, offsets, token_idx, token_w,
                       token_rows);
  return hipGetLastError();
}

// H must be a multiple of 4, and both pitches (callers validate them as multiples of 8).
hipError_t moe_combine(const float* rows, int64_t ldr, const int32_t* token_rows, const float* token_w, int T, int k,
                       int H, uint16_t* out, int64_t ldo, hipStream_t st) {
  hipLaunchKernelGGL(combine_kernel, dim3(grid_for((int64_t)T * (H / 4))), dim3(256), 0, st, rows, ldr, token_rows,
                     token_w, T, k, H / 4, out, ldo);
  return hipGetLastError();
}

}  // namespace mtp
