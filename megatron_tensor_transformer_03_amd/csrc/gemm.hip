// Launch planning of the GEMM kernels and the top-level dispatch by mode (the kernel template is in
// gemm_kernel.h; its instantiations are spread over gemm_fwd_*.hip, gemm_bwd_*.hip and gemm_grouped.hip so that
// they compile in parallel).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "gemm_kernel.h"

namespace mtp {

// ------------------------------------------------------------------------------------------ launch
namespace {
int g_cus[64] = {0};
}  // namespace

// CU count of the current device, read once per device (a plain attribute query: no allocation, no
// synchronisation).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

// Schedule choice, by a cost model in microseconds.  One workgroup per tile: (waves of tiles over the CUs) x
// (tile time), tile time = 2 BM BN K / (efficiency x R), R the sustained bf16 rate of one CU and efficiency
// the tile shape's measured rate relative to the 256 x 256 tile.  Split-K: every tile's K range in S chunks,
// one workgroup per CU working through the (tile, chunk) units, each chunk's fp32 partial tile written to
// the workspace and read back by the tile's last finisher: (waves of units) x (chunk time + pipeline fill)
// plus that partial traffic, tiles x S x (partial tile bytes) x 2, at the bandwidth BW it streams at.  The
// traffic term is what makes split-K lose on short K (4096 x 1024 x 1024: 134 MB of partials for a 16 MB
// output) and win on long K with few tiles (4096 x 1280 x 8192: 80 tiles of 256 x 256, 31% of the CUs
// busy, 240 units in 3 chunks).  Hybrid: whole waves of tiles one per workgroup, then only the remaining
// tiles split.  R and BW were fitted to the measured times of these schedules at the workloads' shapes
// (within ~10%).  A split schedule needs a workspace (the tiles' arrival counters, then the split tiles'
// partial slots); only schedules whose workspace fits in ws_avail are considered.
GemmPlan gemm_plan(int mode, int64_t M, int64_t Nout, int64_t K, int row_major_k, bool allow_small, size_t ws_avail) {
  struct Opt { int bm, bn; double eff; int id; int ns_bk; int64_t slot_bytes; int pad_k; };
  // Relative efficiencies per output, against the 256 x 256 tile: the 256 x 192 tile measured 0.80-0.86 at
  // the forward workload shapes (both in two 64-deep stages then; both run the split ring now), and its
  // 32-deep four-stage form 0.6-1.1 on the transposed (backward) forms depending on the board.
  const double wide_eff = row_major_k ? 0.95 : 0.85;
  const double half_eff = row_major_k ? 0.85 : 0.75;
  // ns_bk: K per ring pass (the split schedule's unit); pad_k: the granularity the step count is padded to
  // with zero steps, charged to the tile's time below.  The 256 x 256 and 256 x 192 tiles run the split ring
  // (passes of 6 K steps, no step past K) in every form.
  const Opt opts[] = {{256, 256, 1.00, 0, 384, 256 << 10, 64}, {256, 192, wide_eff, 1, 384, 192 << 10, 64},
                      {256, 128, half_eff, 2, 128, 128 << 10, 128}, {128, 128, 0.72, 3, 256, 0, 256},
                      {128, 128, 0.72, 4, 128, 64 << 10, 128}};
  constexpr double kR = 5.5e12 * 1e-6;   // FLOP per microsecond of one CU
  constexpr double kBW = 3.0e12 * 1e-6;  // bytes per microsecond of the partial-tile traffic
  const int cus = cu_count();
  GemmPlan best;
  best.bm = 128; best.bn = 128; best.id = 3;
  double best_t = 1e300;
  for (const Opt& o : opts) {
    if (mode == MODE_SWIGLU && o.id == 1) continue;  // gate/up pairs need wave tiles of 64 B rows
    // transposed operands: every tile but the 128 x 128 one with the 64-deep K step (id 3), and its 32-deep
    // form (id 4), which serves only them
    if (row_major_k ? o.id == 3 : o.id == 4) continue;
    // with both operands transposed the 192-wide tile measured slower than the 256 x 256 one (wgrad of the
    // 175B fc1: 411 against 372 us), so it is left out there
    if (row_major_k == 2 && o.id == 1) continue;
    if (!allow_small && o.id == 3) continue;                 // (its K step is 64 two-byte units)
    const int64_t nbo = mode == MODE_SWIGLU ? o.bn / 2 : o.bn;
    const int64_t tiles = ((M + o.bm - 1) / o.bm) * ((Nout + nbo - 1) / nbo);
    // (the backward products keep the relative model they were tuned with: tile time o.bm o.bn / eff, a
    // per-tile cost of 0.03 tile per chunk for the partial sums, no hybrid)
    const bool fwd = row_major_k == 0;
    const double kpad = (double)((K + o.pad_k - 1) / o.pad_k * o.pad_k) / (double)((K + 63) / 64 * 64);
    const double tile_t = fwd ? 2.0 * o.bm * o.bn * (double)K * kpad / (o.eff * kR) : o.bm * o.bn / o.eff;
    const int64_t full_waves = tiles / (cus > 0 ? cus : 1);
    const double t_dp = (double)((tiles + cus - 1) / (cus > 0 ? cus : 1)) * tile_t;
    if (t_dp < best_t * 0.999) { best_t = t_dp; best = GemmPlan{o.bm, (int)nbo, 0, o.id, 0, 0, 0}; }
    // split-K (all tiles, or the tiles past the whole waves): S chunks of whole ring passes and at least 8 K
    // steps of 64 (32-deep rings: 8 steps of 32 per chunk, K counted the same); per unit a pipeline fill of
    // about 192 K (3 steps of 64); chosen only when clearly faster
    const int64_t passes = (K + o.ns_bk - 1) / o.ns_bk;
    const int64_t pass_steps = o.ns_bk / 64;
    if (o.slot_bytes == 0 || cus < 8 || cus % 8 != 0 || tiles > kSplitMaxTiles) continue;
    for (int hybrid = 0; hybrid < 2; ++hybrid) {
      const int64_t dp_tiles = hybrid ? full_waves * cus : 0;
      const int64_t split_tiles = tiles - dp_tiles;
      // (the hybrid form was measured on the 256 x 256 tile only)
      if (hybrid && (!fwd || o.id != 0 || dp_tiles == 0 || split_tiles == 0)) continue;
      for (int S : {2, 3, 4, 5, 6, 8}) {
        if (passes * pass_steps < 8 * S || passes < S || split_tiles * S * o.slot_bytes > ((int64_t)512 << 20))
          continue;
        const size_t ws = kSplitCounterBytes + (size_t)(split_tiles * S * o.slot_bytes);
        if (ws > ws_avail) continue;
        const int64_t waves = (split_tiles * S + cus - 1) / cus;
        const double t_sk = full_waves * hybrid * tile_t + waves * tile_t * (1.0 / S + 192.0 / (double)K) +
                            (fwd ? 2.0 * split_tiles * S * o.slot_bytes / kBW : tile_t * 0.03 * S);
        if (t_sk < best_t * 0.95) {
          best_t = t_sk;
          best = GemmPlan{o.bm, (int)nbo, cus, o.id, S, (int)dp_tiles, ws};
        }
      }
    }
    // shared tails (the forward 256 x 192 tile, fewer tiles than CUs, both spread evenly over the 8 XCDs):
    // tiles / cus of each tile's K in a workgroup of its own, the rest of `share` tiles in one more; the time is
    // that share of a tile plus a fill, plus one partial tile per tile written and read back
    const int64_t extra = cus - tiles;
    if (fwd && o.id == 1 && extra > 0 && tiles % 8 == 0 && extra % 8 == 0 &&
        (tiles / 8) % (extra / 8) == 0 && passes >= 2) {
      const int share = (int)(tiles / extra);
      const size_t ws = kSplitCounterBytes + (size_t)(tiles * 2 * o.slot_bytes);
      const double t_sh = tile_t * ((double)tiles / cus + 192.0 / (double)K) + 2.0 * tiles * o.slot_bytes / kBW;
      if (ws <= ws_avail && t_sh < best_t * 0.95) {
        best_t = t_sh;
        best = GemmPlan{o.bm, (int)nbo, (int)(tiles + tiles / share), o.id, 2, 0, ws, share};
      }
    }
  }
  return best;
}

hipError_t gemm_backward(const GemmParams& p, bool a_row_major_k, bool b_row_major_k, hipStream_t st) {
  if (!a_row_major_k && b_row_major_k) return gemm_dgrad(p, st);
  if (a_row_major_k && b_row_major_k) return gemm_wgrad(p, st);
  return hipErrorInvalidValue;
}

hipError_t gemm(const GemmParams& p, int mode, hipStream_t st, int epi) {
  switch (mode) {
    case MODE_COL: return gemm_fwd_col(p, st, epi);
    case MODE_SWIGLU: return gemm_fwd_swiglu(p, st, epi);
    case MODE_ROW: return gemm_fwd_row(p, st, epi);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
