// Host helpers shared by the PCG drivers (single and several right-hand
// sides): workspace alignment, launch grids, work-item counts of a matrix
// orientation, Infinity Cache budget, iteration batching and timing events.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <unordered_map>
#include <utility>

#include "internal.h"

namespace sla {

// Device memory a handle owns comes from a small caching allocator: a
// destroyed handle parks its buffers in a per-device cache (up to kCacheKeep
// bytes), and the next handle reuses a cached buffer of the same or a
// slightly larger size.  Creating and destroying handles every step (as a
// training loop does) then costs no hipMalloc / hipFree after the first
// time; each of those takes tens to hundreds of microseconds and hipFree
// synchronises the device.  A failed hipMalloc empties the cache and retries.
namespace {
constexpr size_t kCacheKeep = 8ull << 30;
struct BufCache {
  std::mutex mu;
  std::multimap<size_t, void*> idle[64];      // size -> buffer, per device
  std::unordered_map<void*, std::pair<int, size_t>> live;  // buffer -> device, size
  size_t held[64] = {};
};
BufCache& cache() {
  static BufCache c;
  return c;
}
void drop_idle(BufCache& c, int dev) {
  for (auto& kv : c.idle[dev]) (void)hipFree(kv.second);
  c.idle[dev].clear();
  c.held[dev] = 0;
}
}  // namespace

hipError_t buf_alloc(void** p, size_t bytes) {
  bytes = std::max<size_t>(bytes, 256);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  BufCache& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  auto it = c.idle[dev].lower_bound(bytes);
  if (it != c.idle[dev].end() && it->first <= bytes + bytes / 4) {
    *p = it->second;
    c.live[*p] = {dev, it->first};
    c.held[dev] -= it->first;
    c.idle[dev].erase(it);
    return hipSuccess;
  }
  e = hipMalloc(p, bytes);
  if (e == hipErrorOutOfMemory && !c.idle[dev].empty()) {
    (void)hipGetLastError();
    drop_idle(c, dev);
    e = hipMalloc(p, bytes);
  }
  if (e == hipSuccess) c.live[*p] = {dev, bytes};
  return e;
}

void buf_free(void* p) {
  if (!p) return;
  BufCache& c = cache();
  std::lock_guard<std::mutex> lk(c.mu);
  auto it = c.live.find(p);
  if (it == c.live.end()) return;
  const int dev = it->second.first;
  const size_t bytes = it->second.second;
  c.live.erase(it);
  if (c.held[dev] + bytes > kCacheKeep) {
    (void)hipFree(p);
    return;
  }
  c.idle[dev].insert({bytes, p});
  c.held[dev] += bytes;
}

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

// Bytes one one-right-hand-side product streams from the matrix side of a
// CSR orientation: the SELL-64 copy in the form the products read (values
// and per-entry column words, or values, one offset per slot and one mask
// byte per row in the slice-offset form), else the CSR arrays.
size_t stream_bytes(const sla_mat& m, const MatView& v) {
  const size_t es = m.dtype == SLA_F64 ? 8 : 4;
  if (m.bs != 1 || !v.sell) return matrix_bytes(m);
  const size_t slots = (size_t)v.sell_slots, ns = (size_t)v.nslices;
  const size_t cols = v.so ? slots / 16 + ns * 64 : slots * (v.sd ? 2 : 4);
  return slots * es + cols + 4 * (ns + 1);
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
