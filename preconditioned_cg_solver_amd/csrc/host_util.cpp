// Host helpers shared by the PCG drivers (single and several right-hand
// sides): workspace alignment, launch grids, work-item counts of a matrix
// orientation, Infinity Cache budget, iteration batching and timing events.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstdlib>
#include <map>
#include <mutex>
#include <new>
#include <unordered_map>
#include <utility>
#include <vector>

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

// Polling records: a solve copies its 16-byte exit flag into pinned host
// memory once per batch of iterations and waits on an event; each running
// solve holds a record of its own, so solves on different streams or threads
// proceed independently.  Records return to a per-device pool and are reused.
namespace {
struct PollPool {
  std::mutex mu;
  std::vector<PollSlot*> idle[64];
};
PollPool& poll_pool() {
  static PollPool p;
  return p;
}
int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  return dev;
}
}  // namespace

sla_status poll_create(PollSlot** out) {
  *out = nullptr;
  PollSlot* p = new (std::nothrow) PollSlot();
  if (!p) {
    set_error("host allocation failed");
    return SLA_ERR_OOM;
  }
  p->device = current_device();
  if (hipHostMalloc(&p->host, kPollBytes, hipHostMallocDefault) != hipSuccess) {
    (void)hipGetLastError();
    delete p;
    set_error("hipHostMalloc of a polling record failed");
    return SLA_ERR_OOM;
  }
  if (hipHostGetDevicePointer(&p->dev, p->host, 0) != hipSuccess || !p->dev) {
    (void)hipGetLastError();
    (void)hipHostFree(p->host);
    delete p;
    set_error("hipHostGetDevicePointer of a polling record failed");
    return SLA_ERR_HIP;
  }
  for (auto& e : p->ev) {
    const hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableTiming);
    if (r != hipSuccess) {
      for (auto& f : p->ev)
        if (f) (void)hipEventDestroy(f);
      (void)hipHostFree(p->host);
      delete p;
      return hip_fail(r, "hipEventCreateWithFlags");
    }
  }
  *out = p;
  return SLA_OK;
}

sla_status poll_acquire(PollSlot** out) {
  const int dev = current_device();
  PollPool& pp = poll_pool();
  {
    std::lock_guard<std::mutex> lk(pp.mu);
    if (!pp.idle[dev].empty()) {
      *out = pp.idle[dev].back();
      pp.idle[dev].pop_back();
      return SLA_OK;
    }
  }
  return poll_create(out);
}

void poll_release(PollSlot* p) {
  if (!p) return;
  PollPool& pp = poll_pool();
  std::lock_guard<std::mutex> lk(pp.mu);
  pp.idle[p->device >= 0 && p->device < 64 ? p->device : 0].push_back(p);
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

// Grid of a product that reads no partials: one work item per workgroup, up
// to kWideGrid times the resident capacity, a multiple of 8.
int wide_grid(int ntiles) {
  int g = std::min(std::max(ntiles, 1), kWideGrid * max_grid());
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

// Iterations per host-polled batch.  Two batches are queued at a time and
// the device decides when to stop, so after the converging iteration up to
// about two batches of launches still run (each returns at once but costs
// its dispatch: a few microseconds for a grid over every CU).  A batch of
// about 0.8 ms keeps the device busy while the host waits on the previous
// batch and queues the next one, and bounds that tail on short solves of big
// matrices (the elasticity system converges in a few dozen iterations of
// ~0.25 ms).  `iter_us` is the caller's estimate of one iteration;
// SLA_BATCH_ITERS overrides.
int batch_iters(double iter_us) {
  static const int env = [] {
    const char* e = getenv("SLA_BATCH_ITERS");
    return e ? std::max(1, std::min(atoi(e), 4096)) : 0;
  }();
  if (env > 0) return env;
  const double b = std::ceil(800.0 / std::max(iter_us, 1.0));
  return (int)std::max(2.0, std::min(b, 16.0));
}

// Waits until the batch ending at iteration kend has filled its polling
// record and copies the record to *out.  The host spins on the mapped
// record: no event, whose barrier packet would stall the queue at every
// batch.  If the stream drains without the record (a launch failed), the
// device's done flag is read instead and reported as done.
hipError_t wait_poll(const SolverState* rec, int kend, hipStream_t s, const int* dev_done,
                     SolverState* out) {
  const volatile SolverState* r = rec;
  for (unsigned spins = 1; r->exit_iter != kend; ++spins) {
    if ((spins & 4095) == 0) {
      const hipError_t q = hipStreamQuery(s);
      if (q == hipErrorNotReady) continue;
      __atomic_thread_fence(__ATOMIC_ACQUIRE);
      if (r->exit_iter == kend) break;
      if (q != hipSuccess) return q;
      int done = 0;
      const hipError_t e = hipMemcpy(&done, dev_done, sizeof(int), hipMemcpyDeviceToHost);
      out->done = 1;  // nothing left to wait for
      out->exit_iter = kend;
      return e;
    }
    __builtin_ia32_pause();
  }
  __atomic_thread_fence(__ATOMIC_ACQUIRE);
  out->done = r->done;
  out->exit_iter = r->exit_iter;
  out->rr = r->rr;
  out->bb = r->bb;
  return hipSuccess;
}

// Rough duration of one iteration over A and G with k right-hand sides
// (us): the value and index streams of A, G and G^T once and ten vector
// passes of n entries per column at 5 TB/s, plus 3 us per kernel launch.
// Only the batch size depends on it.
double iteration_estimate_us(const sla_mat& A, const sla_mat& G, int elem_bytes, int k,
                             int launches) {
  auto stream = [&](const sla_mat& m) {
    return (double)m.nnz() * elem_bytes + (double)m.nnzb * 4.0;
  };
  const double bytes = stream(A) + 2.0 * stream(G) + 10.0 * (double)A.n() * elem_bytes * k;
  return bytes / 5.0e6 + 3.0 * launches;
}

}  // namespace sla
