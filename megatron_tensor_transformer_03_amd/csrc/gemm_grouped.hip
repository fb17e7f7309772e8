// Instantiations of the GEMM kernel template for the grouped (MoE expert) products: SwiGLU fc1 with a row
// gather, and fc2 writing each routed row's fp32 output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_kernel.h"

namespace mtp {

hipError_t gemm_grouped(const GemmParams& p, int mode, int rows_upper, hipStream_t st, int split_chunks) {
  switch (mode) {
    case MODE_SWIGLU: return launch_cfg<GroupedTile, MODE_SWIGLU, true>(p, rows_upper, st, 0, split_chunks);
    case MODE_ROW: return launch_cfg<GroupedTile, MODE_ROW, true>(p, rows_upper, st, 0, split_chunks);
    default: return hipErrorInvalidValue;
  }
}

// The tail tiles (one partial row tile per group and column tile) matter where the whole tiles make few waves:
// there they form a last wave that leaves most CUs idle (the MoE fc2 at 8 experts x 16 column tiles: 432 whole
// tiles and 128 tail tiles, 2.2 waves run as 3).  Cut into S chunks they fill the CUs the whole tiles leave
// free.  S = 3: a list-scheduling model of the dispatch (workgroups in id order, each to the first free CU)
// puts that fc2 at 2.36-2.45 tile times for 416-464 whole tiles, against 2.53 with S = 2 and 2.28-2.56 with
// S = 4 (more partial traffic); S = 2 where 3 x (tail tiles) would pass two waves.  Launches of many waves
// keep their tails whole (the last wave is a small part of them, and the partial sums would cost traffic).
GroupedPlan grouped_plan(int mode, int64_t rows_upper, int groups, int64_t Nout, int64_t K) {
  GroupedPlan pl;
  const int cus = cu_count();
  if (cus <= 0 || groups <= 0 || rows_upper <= 0 || (mode != MODE_SWIGLU && mode != MODE_ROW)) return pl;
  using C = GroupedTile;
  const int64_t nb = mode == MODE_SWIGLU ? C::BN / 2 : C::BN;
  const int64_t tiles_n = (Nout + nb - 1) / nb;
  const int64_t tail = (int64_t)groups * tiles_n, full = rows_upper / C::BM * tiles_n;
  if (tail > kSplitMaxTiles || full + tail > 4 * (int64_t)cus) return pl;
  // (as the dense split: chunks of whole ring passes and at least 8 K steps)
  const int64_t passes = (K + C::BK * C::RING - 1) / (C::BK * C::RING);
  const int S = 3 * tail <= 2 * (int64_t)cus ? 3 : 2;
  if (passes * C::RING < 8 * S || passes < S) return pl;
  const size_t slot = (size_t)C::FM * C::FN * 16 * sizeof(float) * C::NT;
  pl.split_chunks = S;
  pl.ws_bytes = kSplitCounterBytes + (size_t)tail * S * slot;
  return pl;
}

}  // namespace mtp
