// C ABI of the gfx950 PCG library: handle management, argument checks and
// error reporting around the kernels in setup.hip and solver.hip.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <new>
#include <string>

#include "internal.h"

namespace sla {

int occupancy_grid(int cus);  // solver.hip

namespace {
thread_local std::string g_last_error;

enum OwnedSlot {
  O_TILES_F = 0,
  O_TILES_T = 1,
  O_LPART_F = 2,
  O_LCNT_F = 3,
  O_LPART_T = 4,
  O_LCNT_T = 5,
  O_TRP = 6,
  O_TCI = 7,
  O_TV = 8,
  O_SELL_F = 9,   // 9, 10, 11: values, columns, slice offsets
  O_SELL_T = 12,  // 12, 13, 14
  O_ORD_RP = 15,  // arrays of a permuted copy (15, 16, 17)
  O_PERM = 18,
  O_IPERM = 19,
  O_SOFS_F = 20,  // slice offsets and row masks (20, 21; 22, 23)
  O_SOFS_T = 22
};

std::mutex g_dev_mu;
DeviceInfo g_dev[64];
bool g_dev_ready[64];

// Returns a handle's buffers to the cache; callers have synchronised the
// device (destroy) or the creation stream (a failed create) first, so no
// queued work can still use them.
void free_owned(sla_mat* m) {
  for (void*& p : m->owned) {
    buf_free(p);
    p = nullptr;
  }
  free_colblocks(m);
}

// Waits for the asynchronous calls queued on a handle (its use events) and
// releases the events.
void wait_uses(sla_mat* m) {
  std::lock_guard<std::mutex> lk(m->use_mu);
  for (auto& u : m->uses) {
    (void)hipEventSynchronize(u.e);
    (void)hipEventDestroy(u.e);
  }
  m->uses.clear();
}

// Frees a handle, its permuted copy and their buffers once the work queued
// on them has finished.
void destroy_handle(sla_mat* m) {
  if (m->ord) destroy_handle(m->ord);
  wait_uses(m);
  free_owned(m);
  delete m;
}

sla_status alloc_long_scratch(sla_mat* m, MatView& v, int part_slot, int cnt_slot,
                              hipStream_t s) {
  const size_t np = (size_t)std::max(1, v.n_long_part);
  const size_t nc = (size_t)std::max(1, v.nlong_rows);
  SLA_HIP(buf_alloc(&m->owned[part_slot], np * sizeof(double)));
  SLA_HIP(buf_alloc(&m->owned[cnt_slot], nc * sizeof(int)));
  SLA_HIP(hipMemsetAsync(m->owned[cnt_slot], 0, nc * sizeof(int), s));
  return SLA_OK;
}

// Sliced copies (SELL-64, BSR sliced ELL) are built unless SLA_SELL=0 at
// handle creation (then CSR products use the LDS-tile engine and BSR the
// block-row engine).
bool sell_enabled() {
  const char* e = getenv("SLA_SELL");
  return !(e && e[0] == '0');
}

bool check(bool ok, const char* msg) {
  if (!ok) set_error(msg);
  return ok;
}

// Whether solves with m as A run on the locality ordering: SLA_ORDER=0 never,
// =1 for every CSR matrix outside the SELL layout, otherwise (auto) when such
// a matrix has at least kOrderMinRows rows and at least half of
// kOrderSamples evenly spaced stored entries lie more than kOrderNear rows
// from the diagonal (gathers with no locality for the ordering to lose).
sla_status decide_order(sla_mat* m, hipStream_t s) {
  m->ord_want = false;
  if (m->bs != 1 || m->fwd.sell || m->nbr == 0 || m->nnzb == 0) return SLA_OK;
  const char* e = getenv("SLA_ORDER");
  if (e && e[0] == '0') return SLA_OK;
  if (e && e[0] == '1') {
    m->ord_want = true;
    return SLA_OK;
  }
  if (m->nbr < kOrderMinRows) return SLA_OK;
  const int samples = (int)std::min<int64_t>(m->nnzb, kOrderSamples);
  int far = 0;
  sla_status st = count_far_entries(*m, samples, kOrderNear, &far, s);
  if (st != SLA_OK) return st;
  m->ord_want = 2 * (int64_t)far >= samples;
  return SLA_OK;
}

sla_status create_common(sla_mat_t* out, int64_t nbr, int64_t nnzb, int32_t bs, const int32_t* rp,
                         const int32_t* ci, const void* v, sla_dtype dtype, uint32_t flags,
                         void* stream, bool ordering = true) {
  if (!check(out != nullptr, "out is NULL")) return SLA_ERR_INVALID_ARG;
  *out = nullptr;
  if (!check(nbr >= 0 && nnzb >= 0, "negative size")) return SLA_ERR_INVALID_ARG;
  if (!check(dtype == SLA_F64 || dtype == SLA_F32, "unknown dtype")) return SLA_ERR_INVALID_ARG;
  if (bs != 1 && bs != 3) {
    set_error("only block sizes 1 (CSR) and 3 (3x3 BSR) are supported");
    return SLA_ERR_UNSUPPORTED;
  }
  if (nbr * bs >= (int64_t)INT32_MAX || nnzb * bs * bs >= (int64_t)INT32_MAX) {
    set_error("sizes must fit int32 indices (n and nnz < 2^31)");
    return SLA_ERR_UNSUPPORTED;
  }
  if (!check(rp != nullptr, "row_ptr is NULL")) return SLA_ERR_INVALID_ARG;
  if (!check(nnzb == 0 || (ci != nullptr && v != nullptr), "col_idx or vals is NULL"))
    return SLA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  int hb[2] = {-1, -1};
  SLA_HIP(hipMemcpyAsync(&hb[0], rp, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&hb[1], rp + nbr, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  if (hb[0] != 0 || hb[1] != (int)nnzb) {
    char msg[128];
    snprintf(msg, sizeof msg, "row_ptr[0] = %d, row_ptr[n] = %d, expected 0 and %lld", hb[0],
             hb[1], (long long)nnzb);
    set_error(msg);
    return SLA_ERR_INVALID_ARG;
  }
  sla_mat* m = new (std::nothrow) sla_mat();
  if (!m) {
    set_error("host allocation failed");
    return SLA_ERR_OOM;
  }
  m->nbr = nbr;
  m->bs = bs;
  m->nnzb = nnzb;
  m->dtype = dtype;
  (void)hipGetDevice(&m->device);
  m->fwd.rp = rp;
  m->fwd.ci = ci;
  m->fwd.v = v;
  sla_status st = SLA_OK;
  if (flags & SLA_VALIDATE) st = validate_structure(*m, s);
  if (st == SLA_OK && bs == 1) st = build_tiling(rp, nbr, m->fwd, &m->owned[O_TILES_F], s);
  if (st == SLA_OK && bs == 1 && sell_enabled())
    st = build_sell(m->fwd, nbr, nnzb, dtype, &m->owned[O_SELL_F], &m->owned[O_SOFS_F], s);
  if (st == SLA_OK && bs == 3 && sell_enabled())
    st = build_bsell(m->fwd, nbr, nnzb, dtype, &m->owned[O_SELL_F], s);
  if (st == SLA_OK && bs == 3) st = max_row_length(rp, nbr, &m->fwd.max_row, s);
  if (st == SLA_OK) st = alloc_long_scratch(m, m->fwd, O_LPART_F, O_LCNT_F, s);
  if (st == SLA_OK && ordering) st = decide_order(m, s);
  m->cb_want = ordering && colblocks_wanted(*m);
  if (st == SLA_OK && (flags & SLA_BUILD_TRANSPOSE)) {
    int32_t *trp = nullptr, *tci = nullptr;
    void* tv = nullptr;
    st = build_transpose(*m, &trp, &tci, &tv, s);
    m->owned[O_TRP] = trp;
    m->owned[O_TCI] = tci;
    m->owned[O_TV] = tv;
    if (st == SLA_OK) {
      m->has_t = true;
      m->tr.rp = trp;
      m->tr.ci = tci;
      m->tr.v = tv;
      if (bs == 1) st = build_tiling(trp, nbr, m->tr, &m->owned[O_TILES_T], s);
      if (st == SLA_OK && bs == 1 && sell_enabled())
        st = build_sell(m->tr, nbr, nnzb, dtype, &m->owned[O_SELL_T], &m->owned[O_SOFS_T], s);
      if (st == SLA_OK && bs == 3 && sell_enabled())
        st = build_bsell(m->tr, nbr, nnzb, dtype, &m->owned[O_SELL_T], s);
      if (st == SLA_OK) st = alloc_long_scratch(m, m->tr, O_LPART_T, O_LCNT_T, s);
    }
  }
  if (st == SLA_OK) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) st = hip_fail(e, "hipStreamSynchronize");
  }
  if (st != SLA_OK) {
    (void)hipStreamSynchronize(s);
    free_owned(m);
    delete m;
    return st;
  }
  *out = m;
  return SLA_OK;
}

// P M P^T as a handle of its own that owns its arrays (transpose built when
// asked).  P is given by perm / iperm.
sla_status make_permuted(const sla_mat& src, const int32_t* perm, const int32_t* iperm,
                         bool transpose, sla_mat** out, hipStream_t s) {
  int32_t *rp = nullptr, *ci = nullptr;
  void* v = nullptr;
  sla_status st = build_permuted(src, perm, iperm, &rp, &ci, &v, s);
  if (st == SLA_OK)
    st = create_common(out, src.nbr, src.nnzb, 1, rp, ci, v, (sla_dtype)src.dtype,
                       transpose ? SLA_BUILD_TRANSPOSE : 0, s, false);
  if (st != SLA_OK) {
    (void)hipStreamSynchronize(s);
    buf_free(rp);
    buf_free(ci);
    buf_free(v);
    return st;
  }
  (*out)->owned[O_ORD_RP] = rp;
  (*out)->owned[O_ORD_RP + 1] = ci;
  (*out)->owned[O_ORD_RP + 2] = v;
  // the solves' products on the ordering run on column blocks
  return src.cb_want ? build_colblocks(*out, s) : SLA_OK;
}

std::mutex g_order_mu;
uint64_t g_order_serial = 0;

// Builds, at the first solve that needs them, A's ordering with P A P^T and
// P G P^T for that ordering (rebuilt when G was last used with another A).
// *use = false when A's solves do not reorder.
sla_status ensure_order(sla_mat* A, sla_mat* G, hipStream_t s, bool* use) {
  *use = false;
  if (!A->ord_want || A == G || A->n() == 0) return SLA_OK;
  std::lock_guard<std::mutex> lk(g_order_mu);
  sla_status st = SLA_OK;
  TraceRange tr("locality ordering");
  if (!A->perm) {
    int32_t *perm = nullptr, *iperm = nullptr;
    st = build_order(*A, &perm, &iperm, s);
    if (st != SLA_OK) {
      (void)hipStreamSynchronize(s);
      buf_free(perm);
      buf_free(iperm);
      return st;
    }
    A->owned[O_PERM] = perm;
    A->owned[O_IPERM] = iperm;
    A->perm = perm;
    A->iperm = iperm;
  }
  if (!A->ord) {
    if ((st = make_permuted(*A, A->perm, A->iperm, false, &A->ord, s)) != SLA_OK) return st;
    A->ord_id = ++g_order_serial;
  }
  if (!G->ord || G->ord_id != A->ord_id) {
    if (G->ord) {
      // the copy is used only by solves, which return when their work is done
      destroy_handle(G->ord);
      G->ord = nullptr;
    }
    if ((st = make_permuted(*G, A->perm, A->iperm, true, &G->ord, s)) != SLA_OK) return st;
    G->ord_id = A->ord_id;
  }
  *use = true;
  return SLA_OK;
}

// One-right-hand-side solve, on A's locality ordering when it has one: b
// enters as P b, the solve runs on P A P^T and P G P^T, and x = P^T x~.
// The permuted b and x sit after the base workspace.
sla_status solve_any(sla_mat* A, sla_mat* G, double eps, const void* b, void* x, double rtol,
                     int32_t maxit, void* work, size_t work_bytes, hipStream_t s,
                     sla_solve_info* info, double* ha = nullptr, double* hb = nullptr,
                     int32_t hl = 0) {
  bool use = false;
  sla_status st = ensure_order(A, G, s, &use);
  if (st != SLA_OK) return st;
  if (!use)
    return sla::pcg_solve(*A, *G, eps, b, x, rtol, maxit, work, work_bytes, s, info, ha, hb, hl);
  const size_t base = workspace_base(*A);
  const size_t vb = align_up((size_t)A->n() * (A->dtype == SLA_F64 ? 8 : 4));
  void* pb = (char*)work + base;
  void* px = (char*)work + base + vb;
  if ((st = permute_rows(A->perm, b, pb, A->n(), 1, A->dtype, true, s)) != SLA_OK) return st;
  if ((st = permute_rows(A->perm, nullptr, px, A->n(), 1, A->dtype, true, s)) != SLA_OK) return st;
  st = sla::pcg_solve(*A->ord, *G->ord, eps, pb, px, rtol, maxit, work, base, s, info, ha, hb,
                      hl);
  if (st == SLA_ERR_HIP || st == SLA_ERR_OOM || st == SLA_ERR_INVALID_ARG ||
      st == SLA_ERR_UNSUPPORTED)
    return st;
  sla_status pst = permute_rows(A->perm, px, x, A->n(), 1, A->dtype, false, s);
  if (pst != SLA_OK) return pst;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return st;
}

// Several right-hand sides, on A's locality ordering when it has one: the
// n x k blocks are permuted by rows (P B in, X = P^T Y out), after the base
// workspace.
sla_status solve_multi_any(sla_mat* A, sla_mat* G, double eps, const void* b, void* x, int32_t k,
                           double rtol, int32_t maxit, void* work, hipStream_t s,
                           sla_solve_info* info, sla_status* cst) {
  bool use = false;
  sla_status st = ensure_order(A, G, s, &use);
  if (st != SLA_OK) return st;
  if (!use) return sla::pcg_solve_multi(*A, *G, eps, b, x, k, rtol, maxit, work, s, info, cst);
  const size_t base = workspace_base_multi(*A, k);
  const size_t vb = align_up((size_t)A->n() * (size_t)k * (A->dtype == SLA_F64 ? 8 : 4));
  void* pb = (char*)work + base;
  void* px = (char*)work + base + vb;
  if ((st = permute_rows(A->perm, b, pb, A->n(), k, A->dtype, true, s)) != SLA_OK) return st;
  if ((st = permute_rows(A->perm, nullptr, px, A->n(), k, A->dtype, true, s)) != SLA_OK) return st;
  st = sla::pcg_solve_multi(*A->ord, *G->ord, eps, pb, px, k, rtol, maxit, work, s, info, cst);
  if (st == SLA_ERR_HIP || st == SLA_ERR_OOM || st == SLA_ERR_INVALID_ARG ||
      st == SLA_ERR_UNSUPPORTED)
    return st;
  sla_status pst = permute_rows(A->perm, px, x, A->n(), k, A->dtype, false, s);
  if (pst != SLA_OK) return pst;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return st;
}

sla_status check_solve(sla_mat_t A, sla_mat_t G, double eps, const void* b, const void* x,
                       double rtol, int32_t maxit, const void* work, size_t work_bytes,
                       int32_t k = 0) {
  return check_solve_args(A, G, eps, b, x, rtol, maxit, work, work_bytes, k, true);
}

// [p, p + pb) and [q, q + qb) overlap
bool overlaps(const void* p, size_t pb, const void* q, size_t qb) {
  const uintptr_t a = (uintptr_t)p, c = (uintptr_t)q;
  return pb > 0 && qb > 0 && a < c + qb && c < a + pb;
}

// The adjoint's output lambda (= dL/db) must not share memory with x, which
// the pattern gradient reads after the solve, or with the workspace; the
// gradient must not share memory with lambda or x.
sla_status check_adjoint_outputs(const sla_mat& A, int k, const void* x, const void* grad_b,
                                 const void* grad_vals, const void* work, size_t work_bytes) {
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  const size_t vb = (size_t)A.n() * (size_t)k * es, gb = (size_t)A.nnz() * es;
  if (!check(!overlaps(grad_b, vb, x, vb), "grad_b must not overlap x")) return SLA_ERR_INVALID_ARG;
  if (!check(!overlaps(grad_b, vb, work, work_bytes), "grad_b must not overlap the workspace"))
    return SLA_ERR_INVALID_ARG;
  if (!check(!overlaps(grad_vals, gb, x, vb) && !overlaps(grad_vals, gb, grad_b, vb),
             "grad_vals must not overlap x or grad_b"))
    return SLA_ERR_INVALID_ARG;
  return SLA_OK;
}

}  // namespace

// k = 0: one right-hand side; k >= 1: the multi-RHS solver's workspace.
sla_status check_solve_args(const sla_mat* A, const sla_mat* G, double eps, const void* b,
                            const void* x, double rtol, int32_t maxit, const void* work,
                            size_t work_bytes, int32_t k, bool need_work) {
  if (!check(A && G, "matrix handle is NULL")) return SLA_ERR_INVALID_ARG;
  if (!check(A->nbr == G->nbr && A->bs == G->bs && A->dtype == G->dtype,
             "A and G differ in size, block size or dtype"))
    return SLA_ERR_INVALID_ARG;
  if (!check(G->has_t, "G was created without SLA_BUILD_TRANSPOSE")) return SLA_ERR_INVALID_ARG;
  if (!check(std::isfinite(eps) && eps >= 0.0, "eps must be finite and >= 0"))
    return SLA_ERR_INVALID_ARG;
  if (!check(std::isfinite(rtol) && rtol >= 0.0, "rtol must be finite and >= 0"))
    return SLA_ERR_INVALID_ARG;
  if (!check(maxit >= 0, "maxit must be >= 0")) return SLA_ERR_INVALID_ARG;
  if (A->n() == 0) return SLA_OK;
  if (!check(b && x, "vector pointer is NULL")) return SLA_ERR_INVALID_ARG;
  if (!check(b != x, "x must not alias b")) return SLA_ERR_INVALID_ARG;
  if (k > 0) {
    if (need_work && !check(work != nullptr && work_bytes >= workspace_bytes_multi(*A, k),
                            "workspace too small"))
      return SLA_ERR_INVALID_ARG;
    return SLA_OK;
  }
  if (need_work &&
      !check(work != nullptr && work_bytes >= workspace_bytes(*A), "workspace too small"))
    return SLA_ERR_INVALID_ARG;
  // the workspace's long-row scratch is sized from A's entry count
  const int64_t rows = long_rows_bound(*A), parts = long_part_bound(*A);
  if (!check(G->fwd.nlong_rows <= rows && G->tr.nlong_rows <= rows &&
                 G->fwd.n_long_part <= parts && G->tr.n_long_part <= parts,
             "G has more long rows than the workspace sized for A provides"))
    return SLA_ERR_INVALID_ARG;
  return SLA_OK;
}

sla_status use_begin(const sla_mat& m, hipStream_t s, bool scratch) {
  if (!scratch) return SLA_OK;
  std::lock_guard<std::mutex> lk(m.use_mu);
  for (const auto& u : m.uses)
    if (u.scratch && u.s != s) SLA_HIP(hipStreamWaitEvent(s, u.e, 0));
  return SLA_OK;
}

sla_status use_end(const sla_mat& m, hipStream_t s, bool scratch) {
  std::lock_guard<std::mutex> lk(m.use_mu);
  sla_mat::Use* u = nullptr;
  for (auto& v : m.uses)
    if (v.s == s) u = &v;
  if (!u) {
    hipEvent_t e = nullptr;
    SLA_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    m.uses.push_back({s, e, false});
    u = &m.uses.back();
  }
  u->scratch = u->scratch || scratch;
  SLA_HIP(hipEventRecord(u->e, s));
  return SLA_OK;
}

// Runs an asynchronous call on handle m (and m2, if given) between the use
// log's begin and end: the call waits for m's own long-row scratch on other
// streams when it uses it, and records the stream's event on both handles.
template <typename F>
sla_status async_call(const sla_mat& m, const sla_mat* m2, hipStream_t s, bool scratch, F&& f) {
  sla_status st = use_begin(m, s, scratch);
  if (st != SLA_OK) return st;
  st = f();
  if (st != SLA_OK) return st;
  st = use_end(m, s, scratch);
  if (st == SLA_OK && m2 && m2 != &m) st = use_end(*m2, s, false);
  return st;
}

void set_error(const std::string& msg) { g_last_error = msg; }

sla_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return e == hipErrorOutOfMemory ? SLA_ERR_OOM : SLA_ERR_HIP;
}

const DeviceInfo& device_info() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (!g_dev_ready[dev]) {
    DeviceInfo d;
    (void)hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (d.cus <= 0) d.cus = 256;
    d.max_grid = occupancy_grid(d.cus);
    if (const char* e = getenv("SLA_GRID")) {
      const int g = atoi(e);
      if (g >= 8) d.max_grid = g & ~7;
    }
    g_dev[dev] = d;
    g_dev_ready[dev] = true;
  }
  return g_dev[dev];
}

}  // namespace sla

using namespace sla;

extern "C" {

sla_status sla_csr_create(sla_mat_t* out, int64_t n, int64_t nnz, const int32_t* d_row_ptr,
                          const int32_t* d_col_idx, const void* d_vals, sla_dtype dtype,
                          uint32_t flags, void* stream) {
  TraceRange tr("sla_csr_create");
  const sla_status st = create_common(out, n, nnz, 1, d_row_ptr, d_col_idx, d_vals, dtype, flags,
                                      stream);
  trace_solve(tr, "sla_csr_create", n, nullptr, st);
  return st;
}

sla_status sla_bsr_create(sla_mat_t* out, int64_t n_block_rows, int64_t nnzb, int32_t block_dim,
                          const int32_t* d_brow_ptr, const int32_t* d_bcol_idx,
                          const void* d_bvals, sla_dtype dtype, uint32_t flags, void* stream) {
  TraceRange tr("sla_bsr_create");
  const sla_status st = create_common(out, n_block_rows, nnzb, block_dim, d_brow_ptr, d_bcol_idx,
                                      d_bvals, dtype, flags, stream);
  trace_solve(tr, "sla_bsr_create", n_block_rows * block_dim, nullptr, st);
  return st;
}

sla_status sla_mat_destroy(sla_mat_t m) {
  if (!m) return SLA_OK;
  // waits for the handle's queued asynchronous calls (their events) before
  // its buffers go back to the cache; solves and creation have already
  // finished when they return
  destroy_handle(m);
  return SLA_OK;
}

sla_status sla_mat_info(sla_mat_t m, int64_t* n, int64_t* nnz, int32_t* block_dim,
                        int32_t* dtype) {
  if (!m) {
    set_error("matrix handle is NULL");
    return SLA_ERR_INVALID_ARG;
  }
  if (n) *n = m->n();
  if (nnz) *nnz = m->nnz();
  if (block_dim) *block_dim = m->bs;
  if (dtype) *dtype = m->dtype;
  return SLA_OK;
}

sla_status sla_mat_transpose_arrays(sla_mat_t m, const int32_t** d_row_ptr,
                                    const int32_t** d_col_idx, const void** d_vals) {
  if (!m || !m->has_t) {
    set_error("handle has no transpose (create with SLA_BUILD_TRANSPOSE)");
    return SLA_ERR_INVALID_ARG;
  }
  if (d_row_ptr) *d_row_ptr = m->tr.rp;
  if (d_col_idx) *d_col_idx = m->tr.ci;
  if (d_vals) *d_vals = m->tr.v;
  return SLA_OK;
}

sla_status sla_mat_tiling(sla_mat_t m, int32_t transpose, int64_t* n_tiles, int64_t* n_long) {
  if (!m || (transpose && !m->has_t)) {
    set_error("bad handle or no transpose");
    return SLA_ERR_INVALID_ARG;
  }
  const MatView& v = transpose ? m->tr : m->fwd;
  if (n_tiles) *n_tiles = m->bs == 1 ? v.ntiles : (m->nbr + kBsrTileRows - 1) / kBsrTileRows;
  if (n_long) *n_long = v.nlong;
  return SLA_OK;
}

sla_status sla_mat_reordered(sla_mat_t m, int32_t* reordered) {
  if (!m || !reordered) {
    set_error("NULL argument");
    return SLA_ERR_INVALID_ARG;
  }
  *reordered = m->ord_want ? 1 : 0;
  return SLA_OK;
}

sla_status sla_spmv(sla_mat_t A, const void* d_x, void* d_y, void* stream) {
  if (!A) {
    set_error("matrix handle is NULL");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->n() > 0 && (!d_x || !d_y || d_x == d_y)) {
    set_error("x and y must be distinct non-NULL device vectors");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, nullptr, s, A->fwd.nlong > 0,
                    [&] { return sla::spmv(*A, false, d_x, d_y, s); });
}

sla_status sla_spmv_t(sla_mat_t A, const void* d_x, void* d_y, void* stream) {
  if (!A || !A->has_t) {
    set_error("handle has no transpose (create with SLA_BUILD_TRANSPOSE)");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->n() > 0 && (!d_x || !d_y || d_x == d_y)) {
    set_error("x and y must be distinct non-NULL device vectors");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, nullptr, s, A->tr.nlong > 0,
                    [&] { return sla::spmv(*A, true, d_x, d_y, s); });
}

sla_status sla_pcg_workspace_size(sla_mat_t A, size_t* bytes) {
  if (!A || !bytes) {
    set_error("NULL argument");
    return SLA_ERR_INVALID_ARG;
  }
  *bytes = workspace_bytes(*A);
  return SLA_OK;
}

sla_status sla_precond_apply(sla_mat_t G, double eps, const void* d_r, void* d_z, void* d_work,
                             size_t work_bytes, void* stream) {
  if (!G || !G->has_t) {
    set_error("G must be created with SLA_BUILD_TRANSPOSE");
    return SLA_ERR_INVALID_ARG;
  }
  if (!(std::isfinite(eps) && eps >= 0.0)) {
    set_error("eps must be finite and >= 0");
    return SLA_ERR_INVALID_ARG;
  }
  if (G->n() > 0 && (!d_r || !d_z || d_r == d_z || !d_work || work_bytes < workspace_base(*G))) {
    set_error("bad vector or workspace argument");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*G, nullptr, s, false, [&] {
    return sla::precond_apply(*G, eps, d_r, d_z, d_work, work_bytes, s);
  });
}

sla_status sla_pcg_solve(sla_mat_t A, sla_mat_t G, double eps, const void* d_b, void* d_x,
                         double rtol, int32_t maxit, void* d_work, size_t work_bytes, void* stream,
                         sla_solve_info* info) {
  sla_status st = check_solve(A, G, eps, d_b, d_x, rtol, maxit, d_work, work_bytes);
  if (st != SLA_OK) return st;
  TraceRange tr("sla_pcg_solve");
  st = solve_any(A, G, eps, d_b, d_x, rtol, maxit, d_work, work_bytes, (hipStream_t)stream, info);
  trace_solve(tr, "sla_pcg_solve", A->n(), info, st);
  return st;
}

sla_status sla_pcg_solve_history(sla_mat_t A, sla_mat_t G, double eps, const void* d_b, void* d_x,
                                 double rtol, int32_t maxit, void* d_work, size_t work_bytes,
                                 double* d_alpha, double* d_beta, int32_t hist_len, void* stream,
                                 sla_solve_info* info) {
  sla_status st = check_solve(A, G, eps, d_b, d_x, rtol, maxit, d_work, work_bytes);
  if (st != SLA_OK) return st;
  if (hist_len < 0 || (hist_len > 0 && (!d_alpha || !d_beta))) {
    set_error("history buffers must hold hist_len doubles each");
    return SLA_ERR_INVALID_ARG;
  }
  return solve_any(A, G, eps, d_b, d_x, rtol, maxit, d_work, work_bytes, (hipStream_t)stream,
                   info, d_alpha, d_beta, hist_len);
}

sla_status sla_pcg_adjoint(sla_mat_t A, sla_mat_t G, double eps, const void* d_x,
                           const void* d_grad_x, void* d_grad_b, void* d_grad_vals, double rtol,
                           int32_t maxit, void* d_work, size_t work_bytes, void* stream,
                           sla_solve_info* info) {
  sla_status st = check_solve(A, G, eps, d_grad_x, d_grad_b, rtol, maxit, d_work, work_bytes);
  if (st != SLA_OK) return st;
  if (A->n() > 0 && (!d_x || (A->nnzb > 0 && !d_grad_vals))) {
    set_error("x or grad_vals is NULL");
    return SLA_ERR_INVALID_ARG;
  }
  if ((st = check_adjoint_outputs(*A, 1, d_x, d_grad_b, d_grad_vals, d_work, work_bytes)) !=
      SLA_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  TraceRange tr("sla_pcg_adjoint");
  st = solve_any(A, G, eps, d_grad_x, d_grad_b, rtol, maxit, d_work, work_bytes, s, info);
  if (st < 0) {
    trace_solve(tr, "sla_pcg_adjoint", A->n(), info, st);
    return st;
  }
  sla_status gs;
  {
    TraceRange tg("sla_pattern_grad");
    gs = sla::pattern_grad(*A, d_grad_b, d_x, d_grad_vals, s);
  }
  if (gs != SLA_OK) return gs;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  trace_solve(tr, "sla_pcg_adjoint", A->n(), info, st);
  return st;
}

sla_status sla_spmm(sla_mat_t A, const void* d_x, void* d_y, int32_t k, void* stream) {
  if (!A || k < 0) {
    set_error("matrix handle is NULL or k < 0");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->n() > 0 && k > 0 && (!d_x || !d_y || d_x == d_y)) {
    set_error("X and Y must be distinct non-NULL device arrays");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, nullptr, s, false, [&] { return sla::spmm(*A, false, d_x, d_y, k, s); });
}

sla_status sla_spmm_t(sla_mat_t A, const void* d_x, void* d_y, int32_t k, void* stream) {
  if (!A || !A->has_t || k < 0) {
    set_error("handle is NULL, has no transpose (create with SLA_BUILD_TRANSPOSE) or k < 0");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->n() > 0 && k > 0 && (!d_x || !d_y || d_x == d_y)) {
    set_error("X and Y must be distinct non-NULL device arrays");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, nullptr, s, false, [&] { return sla::spmm(*A, true, d_x, d_y, k, s); });
}

sla_status sla_pcg_workspace_size_multi(sla_mat_t A, int32_t k, size_t* bytes) {
  if (!A || !bytes || k < 1) {
    set_error("NULL argument or k < 1");
    return SLA_ERR_INVALID_ARG;
  }
  *bytes = workspace_bytes_multi(*A, k);
  return SLA_OK;
}

sla_status sla_pcg_solve_multi(sla_mat_t A, sla_mat_t G, double eps, const void* d_b, void* d_x,
                               int32_t k, double rtol, int32_t maxit, void* d_work,
                               size_t work_bytes, void* stream, sla_solve_info* info,
                               sla_status* col_status) {
  if (k < 1) {
    set_error("k must be >= 1");
    return SLA_ERR_INVALID_ARG;
  }
  sla_status st = check_solve(A, G, eps, d_b, d_x, rtol, maxit, d_work, work_bytes, k);
  if (st != SLA_OK) return st;
  TraceRange tr("sla_pcg_solve_multi");
  st = solve_multi_any(A, G, eps, d_b, d_x, k, rtol, maxit, d_work, (hipStream_t)stream, info,
                       col_status);
  trace_solve(tr, "sla_pcg_solve_multi", A->n() * k, nullptr, st);
  return st;
}

sla_status sla_pcg_adjoint_multi(sla_mat_t A, sla_mat_t G, double eps, const void* d_x,
                                 const void* d_grad_x, void* d_grad_b, void* d_grad_vals,
                                 int32_t k, double rtol, int32_t maxit, void* d_work,
                                 size_t work_bytes, void* stream, sla_solve_info* info,
                                 sla_status* col_status) {
  if (k < 1) {
    set_error("k must be >= 1");
    return SLA_ERR_INVALID_ARG;
  }
  sla_status st = check_solve(A, G, eps, d_grad_x, d_grad_b, rtol, maxit, d_work, work_bytes, k);
  if (st != SLA_OK) return st;
  if (A->n() > 0 && (!d_x || (A->nnzb > 0 && !d_grad_vals))) {
    set_error("x or grad_vals is NULL");
    return SLA_ERR_INVALID_ARG;
  }
  if ((st = check_adjoint_outputs(*A, k, d_x, d_grad_b, d_grad_vals, d_work, work_bytes)) !=
      SLA_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  st = solve_multi_any(A, G, eps, d_grad_x, d_grad_b, k, rtol, maxit, d_work, s, info,
                       col_status);
  if (st < 0) return st;
  sla_status gs = sla::pattern_grad_multi(*A, d_grad_b, d_x, k, d_grad_vals, s);
  if (gs != SLA_OK) return gs;
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  return st;
}

sla_status sla_lanczos_extremes(const double* h_alpha, const double* h_beta, int32_t k,
                                double* lmin, double* lmax) {
  if (k < 1 || !h_alpha || (k > 1 && !h_beta) || !lmin || !lmax) {
    set_error("need k >= 1 and non-NULL alpha[k], beta[k-1], lmin, lmax");
    return SLA_ERR_INVALID_ARG;
  }
  return sla::lanczos_extremes(h_alpha, h_beta, k, lmin, lmax);
}

sla_status sla_sai_loss(sla_mat_t A, sla_mat_t G, double eps, const void* d_probes,
                        int32_t nprobe, double scale, void* d_work, size_t work_bytes,
                        double* d_out, void* stream) {
  if (!A || !G || !G->has_t) {
    set_error("A and G must be non-NULL and G created with SLA_BUILD_TRANSPOSE");
    return SLA_ERR_INVALID_ARG;
  }
  if (G->n() != A->n() || G->bs != A->bs || G->dtype != A->dtype) {
    set_error("A and G must have the same size, block size and dtype");
    return SLA_ERR_INVALID_ARG;
  }
  if (!(std::isfinite(eps) && eps >= 0.0) || !(std::isfinite(scale) && scale > 0.0) ||
      nprobe < 0) {
    set_error("need finite eps >= 0, finite scale > 0 and nprobe >= 0");
    return SLA_ERR_INVALID_ARG;
  }
  const size_t need = std::max(sla::workspace_bytes(*A), sla::workspace_bytes(*G));
  if (nprobe > 0 && (!d_out || (A->n() > 0 && !d_probes) || !d_work || work_bytes < need)) {
    set_error("bad probe, output or workspace argument");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, G, s, false, [&] {
    return sla::sai_loss(*A, *G, eps, d_probes, nprobe, scale, d_work, d_out, s);
  });
}

sla_status sla_pattern_grad(sla_mat_t A, const void* d_lambda, const void* d_x,
                            void* d_grad_vals, void* stream) {
  if (!A) {
    set_error("matrix handle is NULL");
    return SLA_ERR_INVALID_ARG;
  }
  if (A->nnzb > 0 && (!d_lambda || !d_x || !d_grad_vals)) {
    set_error("NULL vector");
    return SLA_ERR_INVALID_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  return async_call(*A, nullptr, s, false,
                    [&] { return sla::pattern_grad(*A, d_lambda, d_x, d_grad_vals, s); });
}

const char* sla_status_string(sla_status st) {
  switch (st) {
    case SLA_OK: return "SLA_OK";
    case SLA_NOT_CONVERGED: return "SLA_NOT_CONVERGED";
    case SLA_ERR_INVALID_ARG: return "SLA_ERR_INVALID_ARG";
    case SLA_ERR_UNSUPPORTED: return "SLA_ERR_UNSUPPORTED";
    case SLA_ERR_BREAKDOWN: return "SLA_ERR_BREAKDOWN";
    case SLA_ERR_NONFINITE: return "SLA_ERR_NONFINITE";
    case SLA_ERR_HIP: return "SLA_ERR_HIP";
    case SLA_ERR_OOM: return "SLA_ERR_OOM";
  }
  return "unknown status";
}

const char* sla_last_error(void) { return g_last_error.c_str(); }

sla_status sla_set_profiling(int32_t enable) {
  prof_enable(enable);
  return SLA_OK;
}

sla_status sla_set_profiling_stride(int32_t every) {
  if (every < 1) {
    set_error("every must be >= 1");
    return SLA_ERR_INVALID_ARG;
  }
  prof_every(every);
  return SLA_OK;
}

sla_status sla_get_profile(int32_t kernel_class, int64_t* launches, double* total_ms) {
  if (kernel_class < 0 || kernel_class > 3) {
    set_error("kernel_class must be 0..3");
    return SLA_ERR_INVALID_ARG;
  }
  prof_get(kernel_class, launches, total_ms);
  return SLA_OK;
}

sla_status sla_reset_profile(void) {
  prof_reset();
  return SLA_OK;
}

}  // extern "C"
