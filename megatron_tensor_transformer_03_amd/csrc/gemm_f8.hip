// Dispatch of the E4M3 x E4M3 GEMMs: the kernel template of gemm_kernel.h with one-byte codes, one
// 32 x 32 x 64 MFMA per 64-code K step (twice the dense rate of the bf16 form on gfx950), and the product
// scaled by both operands' dequantization factors before the usual column / SwiGLU / row epilogues.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

template <int MODE>
static hipError_t dispatch_f8(const GemmParams& p, hipStream_t st) {
  const GemmPlan pl = gemm_plan(MODE, p.M, p.Nout, p.K, 0, false, p.ws ? p.ws_bytes : 0);
  switch (pl.id) {
    case 0:
      return launch_cfg<BigFwdTile, MODE, false, false, false, EPI_PLAIN, true>(p, 0, st, pl.split_groups, pl.split_chunks,
                                                                                pl.dp_tiles, pl.share);
    case 1:
      if constexpr (MODE != MODE_SWIGLU)
        return launch_cfg<WideFwdTile, MODE, false, false, false, EPI_PLAIN, true>(p, 0, st, pl.split_groups,
                                                                                   pl.split_chunks, pl.dp_tiles, pl.share);
      return hipErrorInvalidValue;
    default:
      return launch_cfg<HalfTile, MODE, false, false, false, EPI_PLAIN, true>(p, 0, st, pl.split_groups,
                                                                              pl.split_chunks, pl.dp_tiles);
  }
}

hipError_t gemm_f8(const GemmParams& p, int mode, hipStream_t st) {
  switch (mode) {
    case MODE_COL: return dispatch_f8<MODE_COL>(p, st);
    case MODE_SWIGLU: return dispatch_f8<MODE_SWIGLU>(p, st);
    case MODE_ROW: return dispatch_f8<MODE_ROW>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
