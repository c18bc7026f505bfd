// Optional tracing, switched on by SLA_TRACE=1 (read once per process):
//  - roctx ranges around the library's phases (handle set-up, locality
//    ordering, solves, adjoint solves, pattern gradient), which
//    rocprofv3 --marker-trace records next to the kernels.  The roctx
//    library is opened at run time, so the library does not link against
//    the profiler and runs unchanged where it is absent;
//  - one line per solve on stderr: the call, n, iterations, relative
//    residual, status and the call's wall time (solves are synchronous).
#include <dlfcn.h>

#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "internal.h"

namespace sla {
namespace {

struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};

bool env_on() {
  const char* e = getenv("SLA_TRACE");
  return e && e[0] == '1';
}

const Roctx& roctx() {
  static Roctx r;
  static std::once_flag once;
  std::call_once(once, [] {
    if (!env_on()) return;
    for (const char* lib : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so",
                            "libroctx64.so.4", "libroctx64.so"}) {
      void* h = dlopen(lib, RTLD_NOW | RTLD_LOCAL);
      if (!h) continue;
      auto push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
      auto pop = (int (*)())dlsym(h, "roctxRangePop");
      if (push && pop) {
        r.push = push;
        r.pop = pop;
        return;
      }
      dlclose(h);
    }
  });
  return r;
}

}  // namespace

bool trace_on() {
  static const bool on = env_on();
  return on;
}

TraceRange::TraceRange(const char* name) : on_(trace_on()), t0_(0.0) {
  if (!on_) return;
  if (const Roctx& r = roctx(); r.push) r.push(name);
  t0_ = std::chrono::duration<double, std::milli>(
            std::chrono::steady_clock::now().time_since_epoch())
            .count();
}

TraceRange::~TraceRange() {
  if (!on_) return;
  if (const Roctx& r = roctx(); r.pop) r.pop();
}

double TraceRange::elapsed_ms() const {
  if (!on_) return 0.0;
  return std::chrono::duration<double, std::milli>(
             std::chrono::steady_clock::now().time_since_epoch())
             .count() -
         t0_;
}

void trace_solve(const TraceRange& r, const char* what, int64_t n, const sla_solve_info* info,
                 sla_status st) {
  if (!trace_on()) return;
  if (info)
    fprintf(stderr,
            "[sla] %s n=%lld iterations=%d converged=%d rel_residual=%.3e status=%s %.3f ms\n",
            what, (long long)n, info->iterations, info->converged, info->rel_residual,
            sla_status_string(st), r.elapsed_ms());
  else
    fprintf(stderr, "[sla] %s n=%lld status=%s %.3f ms\n", what, (long long)n,
            sla_status_string(st), r.elapsed_ms());
}

}  // namespace sla
