// Launch shape of the token-row kernels (one workgroup per token row).
#pragma once

#include <cstdint>

#include "common.h"

#ifndef MOE_ROW_MAX_THREADS
#define MOE_ROW_MAX_THREADS 512
#endif
#ifndef MOE_ROW_VPT
#define MOE_ROW_VPT 0
#endif
#ifndef MOE_GATHER_VPT
#define MOE_GATHER_VPT 2
#endif
// Streaming unpermute backwards with prob gradients (top-k and mask-map
// forms) as two launches, the dot products and then a scaled scatter, when
// the row fits one workgroup pass; 0 keeps the fused kernels.
#ifndef MOE_BWD_SPLIT
#define MOE_BWD_SPLIT 1
#endif

namespace moe {

// Largest row workgroup (512 keeps 256 VGPRs per lane available) and the
// units per lane (0: chosen per row length); build-time tuning constants.
constexpr int kRowThreads = MOE_ROW_MAX_THREADS;

// ------------------------------------------------------------ launch shape --

struct RowShape {
  int threads;  // workgroup size, multiple of 64
  int vpt;      // units per lane per row slice
  int ysplit;   // row slices per token (grid.y)
};

// A whole row in one pass with exactly `vpt` units per lane, when that fits
// `max_threads`; ysplit 0 when it does not.
inline RowShape row_shape_vpt(int64_t V, int vpt, int max_threads) {
  int64_t th = (V + vpt - 1) / vpt;
  th = ((th + kWave - 1) / kWave) * kWave;
  if (th > max_threads) return RowShape{0, 0, 0};
  return RowShape{(int)th, vpt, 1};
}

// One workgroup per token row (slice): cover V units with `threads` lanes of
// `vpt` units each, preferring the least idle lanes, then mid-size groups.
inline RowShape row_shape(int64_t V, bool allow_split) {
  const int kMaxThreads = kRowThreads;
  int ysplit = 1;
  if (allow_split && V > (int64_t)kMaxThreads * 4)
    ysplit = (int)((V + (int64_t)kMaxThreads * 4 - 1) / ((int64_t)kMaxThreads * 4));
  const int64_t Vs = (V + ysplit - 1) / ysplit;
  // Fallback for an unsplit row longer than one full-size pass.
  RowShape best{kMaxThreads, 4, ysplit};
  int64_t best_waste = -1;
  int best_score = 0;
  const int vpts[] = {1, 2, 4};
  for (int vpt : vpts) {
    if (MOE_ROW_VPT != 0 && vpt != MOE_ROW_VPT) continue;
    int64_t th = (Vs + vpt - 1) / vpt;
    th = ((th + kWave - 1) / kWave) * kWave;
    if (th > kMaxThreads) continue;
    const int64_t waste = th * vpt - Vs;
    // prefer 256..512 threads, then fewer units per lane
    const int score = (th >= 256 && th <= 512 ? 0 : (th < 256 ? 1 : 2)) * 8 + vpt;
    if (best_waste < 0 || waste < best_waste || (waste == best_waste && score < best_score)) {
      best = RowShape{(int)th, vpt, ysplit};
      best_waste = waste;
      best_score = score;
    }
  }
  return best;
}

// Shape of the combine (unpermute, permute backward): MOE_GATHER_VPT (two)
// units per lane while that takes at most 256 lanes, else four units per lane
// when the row fits one pass of up to kRowThreads lanes, else row_shape.
// Measured: 4 KiB rows (256 units) 19.3 us with two units per lane against
// 19.7 with four; 14 KiB rows (896 units, the 16384-token top-8 unpermute)
// 341-344 us warm and 344-346 cold with four units on 224 lanes, against
// 355-358 and 345-351 with two on 448 (one on 896: 350-353 and 338).
inline RowShape gather_shape(int64_t V) {
  RowShape sh = row_shape_vpt(V, MOE_GATHER_VPT, kRowThreads);
  if (sh.threads > 256) {
    const RowShape four = row_shape_vpt(V, 4, kRowThreads);
    if (four.threads != 0) sh = four;
  }
  if (sh.threads == 0) sh = row_shape(V, true);
  return sh;
}

}  // namespace moe
