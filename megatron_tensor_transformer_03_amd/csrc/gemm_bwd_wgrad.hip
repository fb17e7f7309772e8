// Instantiations of the GEMM kernel template for the weight-gradient products dWt = dY^T . X (both operands read row-major-K).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_wgrad(const GemmParams& p, hipStream_t st) { return dispatch_bwd<true, true>(p, st); }

}  // namespace mtp
