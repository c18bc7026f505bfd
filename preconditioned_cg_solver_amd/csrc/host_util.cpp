// Host helpers shared by the PCG drivers (single and several right-hand
// sides): workspace alignment, launch grids, work-item counts of a matrix
// orientation, Infinity Cache budget, iteration batching and timing events.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>

#include "internal.h"

namespace sla {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int max_grid() {
  const int g = device_info().max_grid;
  return g > 0 ? g : 2048;
}

// Grid of a step kernel over `ntiles` tiles: at most the resident capacity,
// a multiple of 8 (one share per XCD) when large enough.
int step_grid(int ntiles) {
  int g = std::min(std::max(ntiles, 1), max_grid());
  if (g >= 8) g &= ~7;
  return std::max(g, 1);
}

// Work items of a product over one orientation: SELL slices grouped by
// workgroup (one per wavefront), LDS tiles, or BSR block-row tiles.
int view_tiles(const sla_mat& m, const MatView& v) {
  if (m.bs != 1 && v.sell) return (v.nslices + kWaves - 1) / kWaves;
  if (m.bs != 1) return (int)((m.nbr + kBsrTileRows - 1) / kBsrTileRows);
  if (v.sell) return (v.nslices + kWaves - 1) / kWaves;
  return v.ntiles;
}

size_t matrix_bytes(const sla_mat& m) {
  const size_t es = m.dtype == SLA_F64 ? 8 : 4;
  return (size_t)m.nnz() * es + (size_t)m.nnzb * 4 + (size_t)(m.nbr + 1) * 4;
}
size_t mall_budget() {
  static size_t b = [] {
    const char* e = getenv("SLA_MALL_BUDGET_MB");
    const long v = e ? atol(e) : 208;
    return (size_t)std::max(0L, v) << 20;
  }();
  return b;
}
// Events used only for timing: no system-scope fence when recorded, so the
// bracketed kernel is not slowed by cache write-back and invalidation.
hipEvent_t timing_event() {
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) == hipSuccess) return e;
  if (hipEventCreate(&e) == hipSuccess) return e;
  return nullptr;
}

int batch_iters() {
  static int b = [] {
    const char* e = getenv("SLA_BATCH_ITERS");
    int v = e ? atoi(e) : 16;
    return std::max(1, std::min(v, 4096));
  }();
  return b;
}

}  // namespace sla
