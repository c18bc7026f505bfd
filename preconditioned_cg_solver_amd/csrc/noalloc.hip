// PCG solve that allocates nothing: the workspace of sla_pcg_solve comes from
// a fixed device array of this library instead of the caller, for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` is a file-scope __device__ array: every device the
// library runs on holds its own copy (kScratchBytes) until the process
// ends.  On the host its name stands for no device address, so the address
// is resolved once per device by sla_init() (hipGetSymbolAddress, with that
// device current) and only that pointer is handed to kernels and memsets.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "internal.h"

namespace sla {
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct NoAllocDevice {
  std::mutex mu;            // serialises the solves on this device (they share scratch)
  void* ptr = nullptr;      // device address of scratch on this device
  PollSlot* slot = nullptr; // polling record reserved at sla_init
  bool ready = false;
};
NoAllocDevice g_na[64];
std::mutex g_na_init_mu;

int current_device_or(int fallback) {
  int dev = fallback;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  return dev;
}

}  // namespace
}  // namespace sla

using namespace sla;

extern "C" {

sla_status sla_init(void) {
  const int dev = current_device_or(0);
  if (dev < 0 || dev >= 64) {
    set_error("no usable current HIP device");
    return SLA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lk(g_na_init_mu);
  NoAllocDevice& d = g_na[dev];
  if (d.ready) return SLA_OK;
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
  if (ptr == nullptr) {
    set_error("hipGetSymbolAddress(scratch) returned NULL");
    return SLA_ERR_HIP;
  }
  PollSlot* slot = nullptr;
  const sla_status st = poll_create(&slot);
  if (st != SLA_OK) return st;
  (void)device_info();  // launch grids of this device, resolved once here
  d.ptr = ptr;
  d.slot = slot;
  d.ready = true;
  return SLA_OK;
}

sla_status sla_pcg_solve_noalloc(sla_mat_t A, sla_mat_t G, double eps, const void* d_b,
                                 void* d_x, double rtol, int32_t maxit, void* stream,
                                 sla_solve_info* info) {
  sla_status st = check_solve_args(A, G, eps, d_b, d_x, rtol, maxit, nullptr, 0, 0, false);
  if (st != SLA_OK) return st;
  const int dev = current_device_or(-1);
  if (dev < 0 || dev >= 64 || !g_na[dev].ready) {
    set_error("sla_init() has not been called on the current device");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->device != dev || G->device != dev) {
    set_error("A and G must belong to the current device");
    return SLA_ERR_INVALID_ARG;
  }
  // the solve runs in A's own row order (the locality ordering would build
  // permuted copies), so it needs exactly the base workspace
  const size_t need = workspace_base(*A);
  if (need > kScratchBytes) {
    set_error("system needs " + std::to_string(need) + " bytes of solver workspace; the "
              "no-allocation scratch holds " + std::to_string(kScratchBytes) +
              " (use sla_pcg_solve with a caller workspace)");
    return SLA_ERR_INVALID_ARG;
  }
  NoAllocDevice& d = g_na[dev];
  std::lock_guard<std::mutex> lk(d.mu);
  return sla::pcg_solve(*A, *G, eps, d_b, d_x, rtol, maxit, d.ptr, kScratchBytes,
                        (hipStream_t)stream, info, nullptr, nullptr, 0, d.slot, true);
}

}  // extern "C"
