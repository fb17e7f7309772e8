// Instantiations of the GEMM kernel template for the column-parallel products (bias and none / erf-GeLU, plain or with the norm epilogue).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_fwd_col(const GemmParams& p, hipStream_t st, int epi) {
  if (epi == EPI_NORM) return dispatch_fwd<MODE_COL, EPI_NORM>(p, st);
  if (epi == EPI_PLAIN) return dispatch_fwd<MODE_COL>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace mtp
