// Host-side launch shapes of the scatter and combine kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "ep_device.h"

namespace ep {

// EP_MI355X_GRID_BLOCKS=<n> (1 <= n <= 2^20) in the environment replaces the
// grid size of the scatter and combine kernels (one wave per work item by
// default).  Their waves walk the work items cyclically, so the results are
// identical at any grid size (waves beyond the work return at once); the
// override serves grid sweeps in tests and launch tuning, and is read at
// every launch.
inline int64_t grid_override() {
  const char* s = getenv("EP_MI355X_GRID_BLOCKS");
  if (!s || !*s) return 0;
  const long long v = atoll(s);
  return v >= 1 && v <= (1LL << 20) ? v : 0;
}

// Blocks that give each wave one of `items` work items (at least one block,
// at most 2^24 - 1 so the grid's work-item count stays below 2^32; the
// kernels walk their items cyclically, so a capped grid still covers them).
inline unsigned wave_per_item_blocks(int64_t items, int waves_per_block = kWavesPerBlock) {
  const int64_t forced = grid_override();
  if (forced > 0) return static_cast<unsigned>(forced);
  constexpr int64_t kMaxBlocks = (1LL << 24) - 1;
  int64_t b = (items + waves_per_block - 1) / waves_per_block;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b < kMaxBlocks ? b : kMaxBlocks);
}

}  // namespace ep
