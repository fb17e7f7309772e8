// Instantiations of the GEMM kernel template for the grouped (MoE expert) products: SwiGLU fc1 with a row
// gather, and fc2 writing each routed row's fp32 output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_grouped(const GemmParams& p, int mode, int rows_upper, hipStream_t st) {
  switch (mode) {
    case MODE_SWIGLU: return launch_cfg<BigFwdTile, MODE_SWIGLU, true>(p, rows_upper, st);
    case MODE_ROW: return launch_cfg<BigFwdTile, MODE_ROW, true>(p, rows_upper, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
