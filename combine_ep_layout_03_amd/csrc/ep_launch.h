// Host-side launch shapes for the persistent kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "ep_device.h"

namespace ep {

// Compute units of the current device (cached per device id).
inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  if (dev >= 64) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// EP_MI355X_GRID_BLOCKS=<n> (1 <= n <= 2^20) in the environment replaces the
// grid size of the scatter and combine kernels.  Their waves walk the work
// items cyclically, so the results are identical at any grid size (waves
// beyond the work return at once); the override serves grid sweeps in tests
// and launch tuning, and is read at every launch.
inline int64_t grid_override() {
  const char* s = getenv("EP_MI355X_GRID_BLOCKS");
  if (!s || !*s) return 0;
  const long long v = atoll(s);
  return v >= 1 && v <= (1LL << 20) ? v : 0;
}

// Blocks that give each wave one of `items` work items (at least one block,
// at most 2^24 - 1 so the grid's work-item count stays below 2^32; the
// kernels walk their items cyclically, so a capped grid still covers them).
inline unsigned wave_per_item_blocks(int64_t items) {
  const int64_t forced = grid_override();
  if (forced > 0) return static_cast<unsigned>(forced);
  constexpr int64_t kMaxBlocks = (1LL << 24) - 1;
  int64_t b = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b < kMaxBlocks ? b : kMaxBlocks);
}

// Blocks for a persistent launch of `Kern`: every block the device can keep
// resident at once, but no more blocks than needed to give each wave one of
// `items` work items.  Residency is queried once per kernel.
template <auto Kern>
inline unsigned persistent_blocks(int64_t items, size_t lds = 0) {
  const int64_t forced = grid_override();
  if (forced > 0) return static_cast<unsigned>(forced);
  static int occ = 0;
  if (occ == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, Kern, kBlock, lds) != hipSuccess || n < 1)
      n = 1;
    occ = n;
  }
  const int64_t full = static_cast<int64_t>(device_cus()) * occ;
  const int64_t need = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  int64_t b = need < full ? need : full;
  if (b < 1) b = 1;
  return static_cast<unsigned>(b);
}

}  // namespace ep
