// Instantiations of the GEMM kernel template for the input-gradient products dX = dY . Wt (Wt read row-major-K).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_dgrad(const GemmParams& p, hipStream_t st) { return dispatch_bwd<false, true>(p, st); }

}  // namespace mtp
