// The column-linear entry point that allocates nothing: mtp_column_linear with the split-K workspace taken from
// a fixed device array of this file instead of a caller argument, for callers that cannot allocate (code under
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// `scratch` is one array per GPU the library runs on, held until the process ends.  Host code never uses its
// name as an address: on each device, at that device's first call, hipGetSymbolAddress gives the device
// address, which is kept per device and passed to the kernels like a caller's workspace.  Every call on a GPU
// shares that GPU's array, so calls that overlap on one GPU (different streams, concurrent graphs) race; calls
// ordered on one stream do not.  The counter block must be zero when a split launch starts: each call that
// splits clears it first with a fill kernel (no memset, so the call stays capturable).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mtp.h"
#include "gemm.h"

namespace mtp {
namespace {

static __device__ __align__(256) uint8_t scratch[MTP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {nullptr};
std::mutex g_scratch_mu;

// Device address of this device's `scratch` (looked up once per device, with that device current).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

__global__ void clear_counters_kernel(uint32_t* __restrict__ cnt, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) cnt[i] = 0u;
}

}  // namespace

// Column GEMM on the static scratch: the plan is the one a caller's workspace of `scratch_bytes` would give.
hipError_t gemm_column_static(GemmParams p, int mode, size_t scratch_bytes, hipStream_t st) {
  void* ptr = nullptr;
  hipError_t e = scratch_address(&ptr);
  if (e != hipSuccess) return e;
  const GemmPlan pl = gemm_plan(mode, p.M, p.Nout, p.K, 0, true, scratch_bytes);
  if (pl.split_groups > 0) {
    hipLaunchKernelGGL(clear_counters_kernel, dim3(16), dim3(256), 0, st, static_cast<uint32_t*>(ptr),
                       (int)(kSplitCounterBytes / 4));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  p.ws = ptr;
  p.ws_bytes = scratch_bytes;
  return gemm(p, mode, st);
}

}  // namespace mtp
