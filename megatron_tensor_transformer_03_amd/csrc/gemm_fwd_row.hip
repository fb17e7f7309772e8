// Instantiations of the GEMM kernel template for the row-parallel partial products (fp32 partial, accumulate, last-shard bf16; plain or with bias-dropout-add).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_fwd_row(const GemmParams& p, hipStream_t st, int epi) {
  if (epi == EPI_BDA) return dispatch_fwd<MODE_ROW, EPI_BDA>(p, st);
  if (epi == EPI_PLAIN) return dispatch_fwd<MODE_ROW>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace mtp
