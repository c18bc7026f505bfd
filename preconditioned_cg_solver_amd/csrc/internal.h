// Internal declarations of the gfx950 PCG library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <string>
#include <vector>

#include "bounds.h"
#include "planner.h"
#include "sla.h"

namespace sla {

// Workgroup size of every row-parallel kernel: four wave64 wavefronts.
constexpr int kWG = 256;
constexpr int kWaves = kWG / 64;
// CSR tiles: at most kTileRows consecutive rows whose nonzeros (<= kLdsCap)
// are staged in LDS; rows with more than kLdsCap nonzeros are split into
// kLongChunk-sized chunks processed by separate workgroups.
constexpr int kTileRows = 256;
constexpr int kLdsCap = 2048;
constexpr int kLongChunk = 4096;
// Locality ordering of the solves (CSR matrices outside the SELL layout
// with at least kOrderMinRows rows whose sampled entries lie mostly more
// than kOrderNear rows from the diagonal): rows sorted by decreasing length
// (lengths capped at kOrderKeyMax for the sort) and dealt over eight row
// segments; see build_order.
constexpr int kOrderKeyBits = 16;
constexpr int kOrderKeyMax = (1 << kOrderKeyBits) - 1;
constexpr int kOrderMinRows = 1 << 17;
constexpr int kOrderNear = 1 << 15;
constexpr int kOrderSamples = 1 << 16;
// Sliced ELLPACK with one wavefront per slice (SELL-64): used for a CSR
// orientation whose rows are short and of even length (at most
// kSellMaxWidth nonzeros per row, padding at most kSellMaxPadPct percent).
constexpr int kSlice = 64;
constexpr int kSellMaxWidth = 32;
constexpr int kSellMaxPadPct = 25;
// SELL columns are stored as int16 offsets from the row when every
// |col - row| fits; kPad16 marks padding slots.
constexpr int kPad16 = -32768;
// Padding slots allocated past the last slice (covers the widest batch).
constexpr int kSellTail = 16 * kSlice;
// Slice-offset form of SELL-64 (banded matrices with a repeating pattern,
// e.g. stencils): every slice lists the distinct column offsets of its rows
// (at most kOfsMax, ascending) and slot j of the slice holds offset j for
// every row; a one-byte mask per row marks the slots the row has.  The
// per-entry column words are then read only by the one-workgroup solver.
constexpr int kOfsMax = 8;
// Halo of the windowed slice-offset engine: slot offsets within +-kWinHalo
// rows are read from the workgroup's LDS window of the gathered vector.
constexpr int kWinHalo = 128;
// Capacity of the MI355X last-level Infinity Cache (MALL).
constexpr size_t kMallBytes = (size_t)256 << 20;
// Sliced ELLPACK for 3x3 BSR: kBSlice block rows per wavefront slice (lane
// l = 3 i + c takes block row 21 s + i and block component c; lane 63 idles).
// A slot (one block of each of the slice's 21 block rows) keeps kBSlotVals
// values, three block rows r of 64 entries (63 used, entry (r, c) of block i
// at 64 r + 21 c + i), and kBSlotCols column entries (21 used), so every
// load of a block row of a slot, and of a slot's columns, covers whole
// 128-byte lines and shares none with the next load.
constexpr int kBSlice = 21;
constexpr int kBSellMaxWidth = 64;
constexpr int kBSlotVals = 192;
constexpr int kBSlotCols = 32;
// Padding slots allocated past the last slice (covers the widest batch).
constexpr int kBSellTail = 16;
// BSR(3x3) engine: kBsrLanes lanes per block row, kWG / kBsrLanes block rows
// per tile.
constexpr int kBsrLanes = 32;
constexpr int kBsrTileRows = kWG / kBsrLanes;
// Ring sizes of the per-iteration scalars kept on the device.
constexpr int kRing = 4;
// Index of entry (r, c) of local block row li of slot q in the BSR
// sliced-ELL value array.
__host__ __device__ inline size_t bsell_val(int q, int r, int c, int li) {
  return (size_t)q * kBSlotVals + (size_t)(64 * r + 21 * c + li);
}

// Right-hand sides advanced together by one pass of the multi-RHS solver.
constexpr int kMaxRhs = 8;
// A pass of 8 columns over a SELL matrix whose stored entries reach further
// than kFarRows rows from the diagonal runs as two passes of 4: the 64-byte
// rows gathered at both far ends, 2 x kFarRows rows apart, then no longer
// stay in an XCD's 4 MB L2 beside the rows in flight.
constexpr int kFarRows = 8192;

// Tile descriptor (CSR engine).
//   kind 0: rows [a, b) staged through LDS, 2^c lanes per row; their
//           nonzeros are [d, d + pad[0]).
//   kind 1: a chunk of one long row: row a, nonzeros [b, c) of the matrix,
//           its partial sum goes to long_part[d]; pad[0] = long-row index,
//           pad[1] = chunks of the row, pad[2] = the row's first partial
//           slot.  The chunk that finishes last (integer ticket) sums the
//           row's partials in chunk order and runs the row epilogue.
enum TileKind { kTileLds = 0, kTileLong = 1 };
struct Tile {
  int a, b, c, d;
  int kind;
  int pad[3];
};

// Device-resident solver state (lives in the caller's workspace).
struct SolverState {
  int done;        // set once an exit condition is met
  int exit_kind;   // ExitKind
  int exit_iter;   // iteration index at which the exit was taken
  int dbg_bad;     // debug builds: gathered columns found out of range
  double rr;       // last ||r||^2
  double bb;       // ||b||^2
  double rho[kRing];    // rho_k = r_k . z_k at slot k % kRing
  double alpha[kRing];  // alpha_k at slot k % kRing
  double sigma;         // last p.Ap
  double pad1;
};

enum ExitKind {
  EX_NONE = 0,
  EX_CONV = 1,          // ||r_k|| <= rtol ||b|| at the G step of iteration k
  EX_MAXIT = 2,         // k == maxit without convergence
  EX_BREAK_SIGMA = 3,   // p.Ap <= 0 or non-finite at the G^T step of iteration k
  EX_BREAK_RHO = 4,     // rho_{k-1} <= 0 or non-finite at the A step of iteration k
  EX_BREAK_RR = 5,      // ||r_k||^2 non-finite
  EX_NONFINITE_B = 6,   // ||b||^2 non-finite
  EX_BZERO = 7,         // b == 0
  EX_MAXIT0 = 8         // maxit == 0, b != 0
};

// One orientation (A or A^T) of a matrix on the device.
struct MatView {
  const int32_t* rp = nullptr;
  const int32_t* ci = nullptr;
  const void* v = nullptr;
  const Tile* tiles = nullptr;   // CSR only
  int ntiles = 0;                // CSR: descriptor count; BSR: block-row tiles
  int nlong = 0;                 // long-row chunks among the tiles
  int nlong_rows = 0;            // rows split into chunks
  int n_long_part = 0;           // partial slots needed by the long-row chunks
  int max_row = -1;              // longest row in blocks (BSR; -1 = not computed)
  int max_dist = -1;             // largest |col - row| (CSR in the SELL layout; -1 = unknown)
  const int* long_rows = nullptr;  // row index of each of the nlong_rows long rows (CSR)
  // SELL-64 copy (owned), built once when the rows qualify: slice s holds
  // rows [64 s, 64 s + 64); slot j of its row 64 s + l sits at
  // soff[s] + 64 j + l; padding slots have column -1 and value 0.
  // For 3x3 BSR the same fields hold the block form: slice s holds block
  // rows [21 s, 21 s + 21) in slots soff[s] .. soff[s + 1] - 1 (soff counts
  // slots); in slot q, local block row i has its block column at
  // kBSlotCols q + i (sc absolute, -1 padding; or sd as block column minus
  // block row, kPad16 padding) and its entry (r, c) at bsell_val(q, r, c, i).
  const void* sv = nullptr;
  const int32_t* sc = nullptr;   // absolute columns, or
  const int16_t* sd = nullptr;   // column - row offsets (preferred when they fit)
  const int32_t* soff = nullptr;
  int nslices = 0;
  int sell_w = 0;                // widest slice (slots per row)
  int64_t sell_slots = 0;        // stored slots (x 64 values; BSR: block slots)
  bool sell = false;
  // Slice-offset form (CSR, null when the rows do not qualify): the column
  // offset of slot j of slice s is so[soff[s] / 64 + j]; bit j of sm[row]
  // is set when the row has that slot (the same slots hold the same values
  // and int16 offsets in sv and sd, padding elsewhere).
  const int32_t* so = nullptr;
  const uint8_t* sm = nullptr;
};

// Column-block copy of a CSR operator (random-graph matrices on their
// locality ordering): its entries split by column into kColBlocks blocks of
// equal column ranges, each a CSR matrix over all rows with the LDS-tile
// layout.  A product runs block b on the workgroups b, b + kColBlocks, ...
// (round-robin dispatch puts them on XCD b), so block b gathers only from
// its eighth of the vector, which that XCD's L2 can hold; the eight
// per-block results of a row are then added in block order.
constexpr int kColBlocks = 8;
struct ColBlockSet {
  MatView blk[kColBlocks];
  int lrow_off[kColBlocks];   // block's long rows in the shared ticket array
  int lpart_off[kColBlocks];  // block's chunk partials in the shared array
};
struct ColBlocks {
  ColBlockSet fwd, tr;
  bool has_tr = false;
  std::vector<void*> owned;
};

}  // namespace sla

struct sla_mat {
  int64_t nbr = 0;     // block rows (= rows for CSR)
  int32_t bs = 1;      // block size
  int64_t nnzb = 0;    // stored blocks (= nonzeros for CSR)
  int32_t dtype = SLA_F64;
  int device = 0;
  sla::MatView fwd;
  bool has_t = false;
  sla::MatView tr;
  // column-block copies (built with the locality ordering's copies when
  // cb_want, decided at creation)
  sla::ColBlocks* cb = nullptr;
  bool cb_want = false;
  // owned device memory: tiles, long-row scratch, the transpose arrays and,
  // for the copies below, the permuted arrays and the permutation
  void* owned[24] = {};
  // Locality ordering used by the solves with this handle as A (decided at
  // creation, built at the first solve): perm maps a row of P A P^T to A's
  // row, iperm the other way; ord is P A P^T, or for a G handle P G P^T of
  // the A ordering numbered ord_id.
  bool ord_want = false;
  const int32_t* perm = nullptr;
  const int32_t* iperm = nullptr;
  sla_mat* ord = nullptr;
  uint64_t ord_id = 0;
  // Asynchronous calls on the handle (products, preconditioner apply,
  // pattern gradient, SAI loss) record an event on their stream after their
  // launches; sla_mat_destroy waits on these instead of the whole device.
  // `scratch` marks streams whose last call used the handle's own long-row
  // scratch (the standalone products): a later call on another stream that
  // uses it waits for that event first.
  struct Use {
    hipStream_t s;
    hipEvent_t e;
    bool scratch;
  };
  mutable std::mutex use_mu;
  mutable std::vector<Use> uses;
  int64_t n() const { return nbr * bs; }
  int64_t nnz() const { return nnzb * bs * bs; }
};

namespace sla {

// Error plumbing (api.cpp).
void set_error(const std::string& msg);
sla_status hip_fail(hipError_t e, const char* what);

#define SLA_HIP(call)                                        \
  do {                                                       \
    hipError_t e_ = (call);                                  \
    if (e_ != hipSuccess) return ::sla::hip_fail(e_, #call); \
  } while (0)

// Device properties cached per device (api.cpp).
struct DeviceInfo {
  int cus = 0;
  int max_grid = 0;      // resident workgroups of the step kernels
};
const DeviceInfo& device_info();
int occupancy_grid(int cus);

// Setup (setup.hip).
sla_status build_tiling(const int32_t* d_rp, int64_t n, MatView& view, void** owned_tiles,
                        hipStream_t s);
// Column-block copies of m's forward view (and of its transpose when m has
// one); SLA_COLBLK=0 leaves m->cb null.
sla_status build_colblocks(sla_mat* m, hipStream_t s);
void free_colblocks(sla_mat* m);
bool colblocks_wanted(const sla_mat& A);
sla_status build_transpose(const sla_mat& m, int32_t** t_rp, int32_t** t_ci, void** t_v,
                           hipStream_t s);
sla_status validate_structure(const sla_mat& m, hipStream_t s);
sla_status max_row_length(const int32_t* d_rp, int64_t nbr, int* out, hipStream_t s);
sla_status build_sell(MatView& view, int64_t n, int64_t nnz, int32_t dtype, void** owned3,
                      void** owned_ofs2, hipStream_t s);
sla_status build_bsell(MatView& view, int64_t nbr, int64_t nnzb, int32_t dtype, void** owned3,
                       hipStream_t s);
sla_status count_far_entries(const sla_mat& m, int samples, int near, int* far, hipStream_t s);
sla_status build_order(const sla_mat& m, int32_t** perm, int32_t** iperm, hipStream_t s);
sla_status build_permuted(const sla_mat& m, const int32_t* perm, const int32_t* iperm,
                          int32_t** rp, int32_t** ci, void** v, hipStream_t s);
// Rows of n x cols row-major arrays.  into: dst row j = src row perm[j];
// otherwise dst row perm[j] = src row j; src == NULL zeroes dst.
sla_status permute_rows(const int32_t* perm, const void* src, void* dst, int64_t n, int cols,
                        int32_t dtype, bool into, hipStream_t s);

// Long-row scratch of a product: per-chunk partial sums and one integer
// ticket per long row (the chunk that takes the last ticket sums the row and
// resets its ticket to 0).  The standalone products use the handle's own
// (long_scratch_of); the solves, the preconditioner apply and the SAI loss
// carve theirs from the caller's workspace, so calls on different streams
// never share tickets.
struct LongScratch {
  double* part;
  int* cnt;
};
LongScratch long_scratch_of(const sla_mat& m, bool transpose);
// Bounds on the long rows and chunks of any matrix with at most A's stored
// entries (the workspace sizes its long-row scratch by them).
int64_t long_rows_bound(const sla_mat& A);
int64_t long_part_bound(const sla_mat& A);

// Event log of a handle's asynchronous calls (api.cpp): use_begin before
// enqueueing work on s (waits for the handle's scratch on other streams
// when `scratch`), use_end after it (records the stream's event).
sla_status use_begin(const sla_mat& m, hipStream_t s, bool scratch);
sla_status use_end(const sla_mat& m, hipStream_t s, bool scratch);

// Pinned host records a running solve polls (host_util.cpp): kPollBytes of
// pinned memory and three events.  poll_acquire takes one from a pool
// (allocating when every pooled slot is in use); poll_create makes a slot
// outside the pool.
constexpr size_t kPollBytes = 4096;
struct PollSlot {
  void* host = nullptr;
  void* dev = nullptr;  // the same pinned record as the device addresses it
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  int device = -1;
};
sla_status poll_create(PollSlot** out);
sla_status poll_acquire(PollSlot** out);
void poll_release(PollSlot* p);
// Holds a pooled slot for the lifetime of a solve.
struct PollLease {
  PollSlot* p = nullptr;
  PollLease() = default;
  PollLease(const PollLease&) = delete;
  PollLease& operator=(const PollLease&) = delete;
  ~PollLease() {
    if (p) poll_release(p);
  }
};

// Solver (solver.hip).  workspace_bytes = workspace_base plus, for an A the
// solves reorder, the two permuted vectors (b and x) after it.
size_t workspace_base(const sla_mat& A);
size_t workspace_bytes(const sla_mat& A);
// y = A x (or A^T x) with the given long-row scratch (NULL: the handle's).
sla_status spmv(const sla_mat& A, bool transpose, const void* x, void* y, hipStream_t s,
                const LongScratch* ls = nullptr);
sla_status precond_apply(const sla_mat& G, double eps, const void* r, void* z, void* work,
                         size_t work_bytes, hipStream_t s);
// slot: the polling record to use (NULL: one from the pool); quiet: record
// no profiling events (the no-allocation entry point).
sla_status pcg_solve(const sla_mat& A, const sla_mat& G, double eps, const void* b, void* x,
                     double rtol, int32_t maxit, void* work, size_t work_bytes, hipStream_t s,
                     sla_solve_info* info, double* hist_a = nullptr, double* hist_b = nullptr,
                     int32_t hist_len = 0, PollSlot* slot = nullptr, bool quiet = false);
sla_status pattern_grad(const sla_mat& A, const void* lam, const void* x, void* grad,
                        hipStream_t s);
sla_status sai_loss(const sla_mat& A, const sla_mat& G, double eps, const void* probes,
                    int32_t nprobe, double scale, void* work, double* out, hipStream_t s);
// Argument checks shared by the solve entry points (api.cpp): k = 0 for one
// right-hand side, k >= 1 for the multi-RHS workspace; need_work = false
// skips the workspace check (the no-allocation entry point).
sla_status check_solve_args(const sla_mat* A, const sla_mat* G, double eps, const void* b,
                            const void* x, double rtol, int32_t maxit, const void* work,
                            size_t work_bytes, int32_t k, bool need_work);

// Small systems solved in one workgroup per right-hand side (solver.hip).
bool small_applies(const sla_mat& A, const sla_mat& G);
size_t small_states_bytes(int k);
sla_status small_solve_batch(const sla_mat& A, const sla_mat& G, double eps, const void* b,
                             void* x, int k, double rtol, int maxit, void* states,
                             hipStream_t s, sla_solve_info* info, sla_status* cst);

// Several right-hand sides (multi.hip); the same split as workspace_bytes,
// with the permuted blocks n x k.
size_t workspace_base_multi(const sla_mat& A, int k);
size_t workspace_bytes_multi(const sla_mat& A, int k);
sla_status spmm(const sla_mat& A, bool transpose, const void* x, void* y, int k, hipStream_t s);
sla_status pcg_solve_multi(const sla_mat& A, const sla_mat& G, double eps, const void* b, void* x,
                           int k, double rtol, int maxit, void* work, hipStream_t s,
                           sla_solve_info* info, sla_status* cst);
sla_status pattern_grad_multi(const sla_mat& A, const void* lam, const void* x, int k, void* grad,
                              hipStream_t s);

// Host helpers (host_util.cpp).
// Device buffers owned by handles, from the library's caching allocator
// (buf_free only after every queued use of the buffer has completed).
hipError_t buf_alloc(void** p, size_t bytes);
void buf_free(void* p);
size_t align_up(size_t v);
int max_grid();
// Separate iteration form on BSR: products on up to kWideGrid x the
// resident grid.
constexpr int kWideGrid = 4;
int wide_grid(int ntiles);
int step_grid(int ntiles);
int view_tiles(const sla_mat& m, const MatView& v);
size_t matrix_bytes(const sla_mat& m);
size_t stream_bytes(const sla_mat& m, const MatView& v);
size_t mall_budget();
hipEvent_t timing_event();
int batch_iters(double iter_us);
// Tracing (trace.cpp, SLA_TRACE=1): a roctx range for the lifetime of a
// TraceRange, and one stderr line per solve.
bool trace_on();
class TraceRange {
 public:
  explicit TraceRange(const char* name);
  ~TraceRange();
  double elapsed_ms() const;

 private:
  bool on_;
  double t0_;
};
void trace_solve(const TraceRange& r, const char* what, int64_t n, const sla_solve_info* info,
                 sla_status st);
hipError_t wait_poll(const SolverState* rec, int kend, hipStream_t s, const int* dev_done,
                     SolverState* out);
double iteration_estimate_us(const sla_mat& A, const sla_mat& G, int elem_bytes, int k,
                             int launches);

// Spectrum of the Lanczos tridiagonal (spectrum.cpp, host only).
sla_status lanczos_extremes(const double* alpha, const double* beta, int32_t k, double* lmin,
                            double* lmax);

// Profiling (solver.hip).
void prof_enable(int mask);
void prof_every(int every);
void prof_get(int cls, int64_t* launches, double* ms);
void prof_reset();

}  // namespace sla
