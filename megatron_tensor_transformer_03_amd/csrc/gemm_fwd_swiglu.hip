// Instantiations of the GEMM kernel template for the gate/up products with the SwiGLU epilogue (plain or with the norm epilogue).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_fwd_swiglu(const GemmParams& p, hipStream_t st, int epi) {
  if (epi == EPI_NORM) return dispatch_fwd<MODE_SWIGLU, EPI_NORM>(p, st);
  if (epi == EPI_PLAIN) return dispatch_fwd<MODE_SWIGLU>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace mtp
