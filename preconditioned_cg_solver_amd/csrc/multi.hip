// Several right-hand sides sharing one A and one G: K PCG solves advanced in
// lock step so that every product streams its matrix once for all K columns.
//
// Vectors are row-major n x K blocks: entry i of column c sits at i * ld + c,
// so a gathered column index j brings in K contiguous values (one 16-64 byte
// load) for the one matrix value read.  Every column keeps its own scalars
// (alpha, beta, rho, ||r||) and its own exit: a column that converges or
// breaks down is frozen (its x no longer changes) while the others go on, and
// the solve ends when every column has exited.  Each column's arithmetic is
// the single-right-hand-side iteration's, so column c gives the result of an
// independent solve for b_c (the solves share only the operators).
//
// One iteration k is three kernels, as for one right-hand side:
//   A step   Q = A P_k with P_k = Z + beta P_{k-1} formed on the fly (stored
//            for owned rows) and partials of sigma_c = p_c . q_c;
//   G^T step T = G^T R_k with R_k = R_{k-1} - alpha Q formed on the fly
//            (stored), X += alpha P_k on owned rows, partials of ||r_c||^2;
//   G step   Z = G T + eps R_k, partials of rho_c = r_c . z_c.
// (With one right-hand side the x update rides in the next A step; here it
// is applied in the G^T step, so a column that exits leaves x final.)
//
// Method: "Learning Sparse Approximate Inverse Preconditioners for CG Solvers
// on GPUs" (Approach) for M^-1 = G G^T + eps I; several same-pattern systems
// solved together is the batched use of "torch-sla" (Significance, batched
// solves); adjoint gradients add over the solves because A is shared
// ("torch-sla", Technical Summary, Methodology 2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "device_util.h"
#include "internal.h"

namespace sla {
namespace {

struct MState {
  int done;  // every column has exited
  int pad[3];
  int exit_kind[kMaxRhs];
  int exit_iter[kMaxRhs];
  double bb[kMaxRhs];
  double rr[kMaxRhs];
  double rho[kRing][kMaxRhs];
  double alpha[kRing][kMaxRhs];
};

enum MMode {
  MM_PLAIN = 0,  // Y = M X
  MM_A1 = 1,     // A step of iteration 1 (P_1 = Z_0)
  MM_A = 2,      // A step of iteration k >= 2
  MM_GT = 3,     // G^T step of iteration k >= 1
  MM_G0 = 4,     // G step of the start-up (checks ||b_c||)
  MM_G = 5,      // G step of iteration k >= 1 (checks convergence)
  MM_AU = 6,     // separate form: Q = A P_k on a stored P_k, sigma partials
  MM_GTU = 7     // separate form: T = G^T R_k on a stored R_k
};

template <typename T>
struct MArgs {
  const int32_t* rp;
  const int32_t* ci;
  const T* v;
  const T* sv;
  const int32_t* sc;
  const int16_t* sd;
  const int32_t* soff;
  int nslices;
  const int32_t* so;  // slice-offset form: offset of each slot (null: per-entry words)
  const uint8_t* sm;  // slice-offset form: slots present in each row
  const Tile* tiles;  // CSR row tiles (tile engine)
  int ntiles;
  int nbr;
  int n;
  const int* long_rows;  // CSR rows longer than a tile (one workgroup each)
  int nlong;
  int ld;        // row stride of the gathered / owned vectors
  const T* in0;  // gathered: X, Z (A step), R_{k-1} (G^T step), T (G step)
  const T* in1;  // gathered second operand: P_{k-1} (A step), Q (G^T step)
  T* own;        // owned-row output: P_k, R_k
  T* y;          // product output
  const T* rv;   // R_k (G step)
  const T* pv;   // P_k (G^T step)
  T* xv;         // solution columns, row stride ldx
  int ldx;
  double eps;
  const double* pin;  // producer partials, [npin][K]
  int npin;
  double* pout;  // this kernel's partials, [gridDim.x][K]
  MState* st;
  // G step of a batch's last iteration: the host-mapped polling record it
  // fills (done, iteration, the largest ||r_c||^2 / ||b_c||^2 of the
  // columns still iterating, 1); null otherwise
  SolverState* poll;
  int k;
  int maxit;
  double rtol;
};

template <typename T, int K>
struct MCoef {
  T c[K];   // gather coefficient (beta, -alpha or 0)
  T c2[K];  // alpha for the x update
  bool act[K];
};

template <int K>
__device__ __forceinline__ void block_sum_k(double (&v)[K], double* red) {
#pragma unroll
  for (int c = 0; c < K; ++c) v[c] = wave_sum(v[c]);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int c = 0; c < K; ++c) red[(threadIdx.x >> 6) * K + c] = v[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < K; ++c) {
    double s = red[c];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) s += red[q * K + c];
    v[c] = s;
  }
}

// This thread's share of K interleaved sums of partials (before the
// workgroup sum).
template <int K>
__device__ __forceinline__ void partial_share_k(const double* __restrict__ p, int np,
                                                double (&out)[K]) {
#pragma unroll
  for (int c = 0; c < K; ++c) out[c] = 0.0;
  // in index order per thread; the loads of 16 / K strides (at least one)
  // are issued together, and past the end a thread adds 0.0
  constexpr int S = K >= 16 ? 1 : 16 / K;
  for (int i = threadIdx.x; i < np; i += S * kWG) {
    double v[S][K];
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < K; ++c)
        v[u][c] = i + u * kWG < np ? p[(size_t)(i + u * kWG) * K + c] : 0.0;
#pragma unroll
    for (int u = 0; u < S; ++u)
#pragma unroll
      for (int c = 0; c < K; ++c) out[c] += v[u][c];
  }
}

__device__ __forceinline__ void col_exit(MState* st, int c, int kind, int k) {
  st->exit_kind[c] = kind;
  st->exit_iter[c] = k;
}

// Kernel start: the done check, then every workgroup sums the producer's
// partials in the same order and takes the same per-column decisions; the
// lead thread records them.  Returns false when the kernel has no work.
template <typename T, int MODE, int K>
__device__ __forceinline__ bool mprologue(const MArgs<T>& a, MCoef<T, K>& cf, double* red,
                                          int* s_flag) {
#pragma unroll
  for (int c = 0; c < K; ++c) {
    cf.c[c] = T(0);
    cf.c2[c] = T(0);
    cf.act[c] = true;
  }
  if constexpr (MODE == MM_PLAIN) {
    return true;
  } else {
    constexpr bool SUMS = MODE != MM_AU && MODE != MM_GTU;
    const int k = a.k;
    // Every load the decisions need is issued before the first wait: this
    // thread's share of the partials, each column's exit kind and state
    // scalar (written by earlier kernels) and the done flag: one memory
    // round trip rather than three in a row.  Unused when the solve is done.
    double s[K];
    int ek[K];
    double s0[K];
#pragma unroll
    for (int c = 0; c < K; ++c) {
      s[c] = 0.0;
      ek[c] = EX_NONE;
      s0[c] = 0.0;
    }
    if constexpr (SUMS) {
      partial_share_k<K>(a.pin, a.npin, s);
      if constexpr (MODE != MM_G0) {
#pragma unroll
        for (int c = 0; c < K; ++c) {
          ek[c] = a.st->exit_kind[c];
          if constexpr (MODE == MM_A) s0[c] = a.st->rho[(k - 2) % kRing][c];
          else if constexpr (MODE == MM_GT) s0[c] = a.st->rho[(k - 1) % kRing][c];
          else if constexpr (MODE == MM_G) s0[c] = a.st->bb[c];
        }
      }
    }
    if (threadIdx.x == 0)
      *s_flag = __hip_atomic_load(&a.st->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
    if (*s_flag) {
      if constexpr (MODE == MM_G) {
        if (a.poll && lead) post_poll(a.poll, 1, a.k, 0.0, 0.0);
      }
      return false;
    }
    if constexpr (!SUMS) return true;
    block_sum_k<K>(s, red);
    int live = 0;
#pragma unroll
    for (int c = 0; c < K; ++c) {
      bool act;
      if constexpr (MODE == MM_G0) {
        const double bb = s[c];
        int ex = EX_NONE;
        if (!isfinite(bb)) ex = EX_NONFINITE_B;
        else if (bb == 0.0) ex = EX_BZERO;
        else if (a.maxit == 0) ex = EX_MAXIT0;
        if (lead) {
          a.st->bb[c] = bb;
          a.st->rr[c] = bb;
          if (ex != EX_NONE) col_exit(a.st, c, ex, 0);
        }
        act = ex == EX_NONE;
      } else {
        act = ek[c] == EX_NONE;
        if (act) {
          if constexpr (MODE == MM_A1 || MODE == MM_A) {
            const double rho = s[c];  // rho_{k-1}
            if (!(rho > 0.0) || !isfinite(rho)) {
              if (lead) col_exit(a.st, c, EX_BREAK_RHO, k);
              act = false;
            } else {
              if (lead) a.st->rho[(k - 1) % kRing][c] = rho;
              if constexpr (MODE == MM_A) cf.c[c] = T(rho / s0[c]);
            }
          } else if constexpr (MODE == MM_GT) {
            const double sigma = s[c];
            if (!(sigma > 0.0) || !isfinite(sigma)) {
              if (lead) col_exit(a.st, c, EX_BREAK_SIGMA, k);
              act = false;
            } else {
              const double alpha = s0[c] / sigma;
              if (lead) a.st->alpha[k % kRing][c] = alpha;
              cf.c[c] = T(-alpha);
              cf.c2[c] = T(alpha);
            }
          } else {  // MM_G
            const double rr = s[c];
            const double rnorm = sqrt(rr), bnorm = sqrt(s0[c]);
            int ex = EX_NONE;
            if (!isfinite(rnorm)) ex = EX_BREAK_RR;
            else if (rnorm <= a.rtol * bnorm) ex = EX_CONV;
            else if (k == a.maxit) ex = EX_MAXIT;
            if (lead) {
              a.st->rr[c] = rr;
              if (ex != EX_NONE) col_exit(a.st, c, ex, k);
            }
            act = ex == EX_NONE;
          }
        }
      }
      cf.act[c] = act;
      live += act ? 1 : 0;
    }
    if constexpr (MODE == MM_G) {
      if (a.poll && lead) {
        double worst = 0.0;
#pragma unroll
        for (int c = 0; c < K; ++c)
          if (cf.act[c] && a.st->bb[c] > 0.0) worst = fmax(worst, s[c] / a.st->bb[c]);
        post_poll(a.poll, live == 0, k, worst, 1.0);
      }
    }
    if (live == 0) {
      if (lead) a.st->done = 1;
      return false;
    }
    return true;
  }
}

// Gathered value of column c at vector row j.
template <typename T, int MODE, int K>
__device__ __forceinline__ T mgat(const MArgs<T>& a, size_t base, int c, const MCoef<T, K>& cf) {
  if constexpr (MODE == MM_A || MODE == MM_GT) return fma(cf.c[c], a.in1[base + c], a.in0[base + c]);
  else return a.in0[base + c];
}

template <typename T, int K>
struct MOwn {
  T a[K], b[K], p[K], x[K];
};

template <typename T, int MODE, int K>
__device__ __forceinline__ void mown_load(const MArgs<T>& a, int i, MOwn<T, K>& o) {
  const size_t r = (size_t)i * a.ld;
#pragma unroll
  for (int c = 0; c < K; ++c) {
    if constexpr (MODE == MM_A1 || MODE == MM_AU) {
      o.a[c] = a.in0[r + c];
    } else if constexpr (MODE == MM_A) {
      o.a[c] = a.in1[r + c];
      o.b[c] = a.in0[r + c];
    } else if constexpr (MODE == MM_GT) {
      o.a[c] = a.in1[r + c];
      o.b[c] = a.in0[r + c];
      o.p[c] = a.pv[r + c];
      o.x[c] = a.xv[(size_t)i * a.ldx + c];
    } else if constexpr (MODE == MM_G0 || MODE == MM_G) {
      o.a[c] = a.rv[r + c];
    }
  }
}

// Row epilogue: stores and the row's contributions to the K dot products.
template <typename T, int MODE, int K>
__device__ __forceinline__ void mepi(const MArgs<T>& a, int i, const T (&acc)[K],
                                     const MCoef<T, K>& cf, const MOwn<T, K>& o,
                                     double (&dot)[K]) {
  const size_t r = (size_t)i * a.ld;
#pragma unroll
  for (int c = 0; c < K; ++c) {
    if constexpr (MODE == MM_PLAIN || MODE == MM_GTU) {
      a.y[r + c] = acc[c];
    } else if constexpr (MODE == MM_AU) {
      a.y[r + c] = acc[c];
      dot[c] += (double)o.a[c] * (double)acc[c];
    } else if constexpr (MODE == MM_A1 || MODE == MM_A) {
      const T pn = MODE == MM_A1 ? o.a[c] : fma(cf.c[c], o.a[c], o.b[c]);
      a.own[r + c] = pn;
      a.y[r + c] = acc[c];
      dot[c] += (double)pn * (double)acc[c];
    } else if constexpr (MODE == MM_GT) {
      const T rn = fma(cf.c[c], o.a[c], o.b[c]);
      a.own[r + c] = rn;
      a.y[r + c] = acc[c];
      if (cf.act[c]) a.xv[(size_t)i * a.ldx + c] = fma(cf.c2[c], o.p[c], o.x[c]);
      dot[c] += (double)rn * (double)rn;
    } else {
      const T zv = fma(T(a.eps), o.a[c], acc[c]);
      a.y[r + c] = zv;
      dot[c] += (double)o.a[c] * (double)zv;
    }
  }
}

template <typename T, int MODE, int K>
__device__ __forceinline__ void mfinish(const MArgs<T>& a, double (&dot)[K], double* red) {
  if constexpr (MODE != MM_PLAIN && MODE != MM_GTU) {
    block_sum_k<K>(dot, red);
    if (threadIdx.x < K) {
      double v = dot[0];
#pragma unroll
      for (int c = 1; c < K; ++c)
        if ((int)threadIdx.x == c) v = dot[c];
      a.pout[(size_t)blockIdx.x * K + threadIdx.x] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// SELL-64 engine (CSR whose rows qualified for the sliced layout): one
// wavefront per slice of 64 rows, lane l owns row 64 s + l, every value and
// column word of a wavefront is one contiguous access; each slot gathers the
// K entries of its column.
// ---------------------------------------------------------------------------

// One batch of U slots of a slice: values and decoded columns (-1 for
// padding).  Loads past the slice end stay inside the arrays' padding tail.
// OFS: the slice-offset form, one offset per slot instead of a column word
// per entry.
template <typename T, bool I16, int U, bool OFS>
__device__ __forceinline__ void msell_batch(const MArgs<T>& a, int off, int lane, int j,
                                            T (&v)[U], int (&raw)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = off + (j + u) * kSlice + lane;
    v[u] = ld_stream<true>(a.sv + idx);
    if constexpr (OFS) raw[u] = ld_stream<true>(a.so + off / kSlice + j + u);
    else if constexpr (I16) raw[u] = ld_stream<true>(a.sd + idx);
    else raw[u] = ld_stream<true>(a.sc + idx);
  }
}

template <typename T, int MODE, int K, bool I16, int U, bool OFS>
__global__ __launch_bounds__(kWG) void msell_step(MArgs<T> a) {
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  const int lane = threadIdx.x & (kSlice - 1), wv = threadIdx.x / kSlice;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  // Software pipeline over the wave's batches (slice by slice, U slots at a
  // time): the matrix data of the next batch -- possibly the next slice's
  // first -- is loaded while the current batch's gathers are in flight.
  auto slice_of = [&](int t, int& off, int& w) {
    const int sl = t * kWaves + wv;
    off = 0;
    w = -1;  // no such slice
    if (t < t1 && sl < a.nslices) {
      off = a.soff[sl];
      w = (a.soff[sl + 1] - off) / kSlice;
    }
  };
  int t = t0, off, w;
  slice_of(t, off, w);
  while (t < t1 && w < 0) {
    t += step;
    slice_of(t, off, w);
  }
  T cv[U];
  int cr[U];
  if (w >= 0) msell_batch<T, I16, U, OFS>(a, off, lane, 0, cv, cr);
  MCoef<T, K> cf;
  if (!mprologue<T, MODE, K>(a, cf, s_red, &s_flag)) return;
  double dot[K];
#pragma unroll
  for (int c = 0; c < K; ++c) dot[c] = 0.0;
  int j = 0;
  int row = (t * kWaves + wv) * kSlice + lane;
  MOwn<T, K> o;
  if (w >= 0) mown_load<T, MODE, K>(a, row < a.n ? row : 0, o);
  int msk = 0;  // slice-offset form: the row's present slots
  if constexpr (OFS)
    if (w >= 0) msk = a.sm[(t * kWaves + wv) * kSlice + lane];
  T acc[K];
#pragma unroll
  for (int c = 0; c < K; ++c) acc[c] = T(0);
  while (w >= 0) {
    // position of the next batch
    int nt = t, nj = j + U, noff = off, nw = w;
    if (nj >= w) {
      nj = 0;
      do {
        nt += step;
        slice_of(nt, noff, nw);
      } while (nt < t1 && nw < 0);
    }
    // gathers of the current batch
    T g[U][K];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int col;
      if constexpr (OFS) col = (j + u < w && ((msk >> (j + u)) & 1)) ? row + cr[u] : -1;
      else if constexpr (I16) col = (j + u < w && cr[u] != kPad16) ? row + cr[u] : -1;
      else col = j + u < w ? cr[u] : -1;
      ok[u] = col >= 0;
      const size_t base = (size_t)(ok[u] ? col : 0) * a.ld;
#pragma unroll
      for (int c = 0; c < K; ++c) g[u][c] = mgat<T, MODE, K>(a, base, c, cf);
    }
    // matrix data of the next batch
    T nv[U];
    int nr[U];
    if (nw >= 0) msell_batch<T, I16, U, OFS>(a, noff, lane, nj, nv, nr);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const T vu = ok[u] ? cv[u] : T(0);
#pragma unroll
      for (int c = 0; c < K; ++c) acc[c] = fma(vu, ok[u] ? g[u][c] : T(0), acc[c]);
    }
    if (nj == 0) {
      if (row < a.n) mepi<T, MODE, K>(a, row, acc, cf, o, dot);
#pragma unroll
      for (int c = 0; c < K; ++c) acc[c] = T(0);
      row = (nt * kWaves + wv) * kSlice + lane;
      if (nw >= 0) mown_load<T, MODE, K>(a, row < a.n ? row : 0, o);
      if constexpr (OFS)
        if (nw >= 0) msk = a.sm[(nt * kWaves + wv) * kSlice + lane];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cv[u] = nv[u];
      cr[u] = nr[u];
    }
    t = nt;
    j = nj;
    off = noff;
    w = nw;
  }
  mfinish<T, MODE, K>(a, dot, s_red);
}

// ---------------------------------------------------------------------------
// Sliced-ELL engine for 3x3 BSR: one wavefront per slice of 21 block rows;
// lane l = 3 i + c takes block row i and block component c.  Per slot it
// reads column c of each block (slot layout: bsell_val) and gathers the K
// contiguous entries of row c of the block column only, keeping the three
// row partials of every right-hand side; after the slice the three lanes of
// a block row add their partials in component order and lane 3 i + r runs
// the epilogue of scalar row 3 (21 s + i) + r.
// ---------------------------------------------------------------------------

template <typename T, int MODE, int K, bool I16, int U>
__global__ __launch_bounds__(kWG) void mbsell_step(MArgs<T> a) {
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // lane 63 mirrors lane 60 (block row 20, component 0) and stores nothing
  const int li = min(lane / 3, kBSlice - 1), c = lane - 3 * (lane / 3);
  const bool lane_live = lane < 3 * kBSlice;
  const int src_prev = 3 * li + (c + 2) % 3, src_next = 3 * li + (c + 1) % 3;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  MCoef<T, K> cf;
  if (!mprologue<T, MODE, K>(a, cf, s_red, &s_flag)) return;
  double dot[K];
#pragma unroll
  for (int k = 0; k < K; ++k) dot[k] = 0.0;
  for (int t = t0; t < t1; t += step) {
    const int sl = t * kWaves + wv;
    if (sl >= a.nslices) continue;
    const int off = a.soff[sl], w = a.soff[sl + 1] - off;
    const int brow = sl * kBSlice + li;
    const bool live = lane_live && brow < a.nbr;
    const int row = 3 * brow + c;
    MOwn<T, K> o;
    mown_load<T, MODE, K>(a, live ? row : 0, o);
    T acc[3][K];
#pragma unroll
    for (int r = 0; r < 3; ++r)
#pragma unroll
      for (int k = 0; k < K; ++k) acc[r][k] = T(0);
    for (int j = 0; j < w; j += U) {
      T bv[U][3];
      int bc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // loads past the slice end stay inside the arrays' padding tail
        const int q = off + j + u;
        const size_t ci = (size_t)q * kBSlotCols + li;
        const int raw = I16 ? (int)ld_stream<true>(a.sd + ci) : ld_stream<true>(a.sc + ci);
        bc[u] = j + u >= w ? -1 : I16 ? (raw == kPad16 ? -1 : brow + raw) : raw;
#pragma unroll
        for (int r = 0; r < 3; ++r) bv[u][r] = ld_stream<true>(a.sv + bsell_val(q, r, c, li));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = bc[u] >= 0;
        const size_t base = (size_t)(ok ? 3 * bc[u] + c : 0) * a.ld;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const T g = ok ? mgat<T, MODE, K>(a, base, k, cf) : T(0);
#pragma unroll
          for (int r = 0; r < 3; ++r) acc[r][k] = fma(ok ? bv[u][r] : T(0), g, acc[r][k]);
        }
      }
    }
    // row c of this block row, per right-hand side: own partial plus those of
    // components c - 1 and c + 1 (mod 3), added in component order
    T y[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const T own = c == 0 ? acc[0][k] : (c == 1 ? acc[1][k] : acc[2][k]);
      const T for_next = c == 0 ? acc[1][k] : (c == 1 ? acc[2][k] : acc[0][k]);
      const T for_prev = c == 0 ? acc[2][k] : (c == 1 ? acc[0][k] : acc[1][k]);
      const T from_prev = __shfl(for_next, src_prev, 64);
      const T from_next = __shfl(for_prev, src_next, 64);
      y[k] = c == 0 ? (own + from_next) + from_prev
           : c == 1 ? (from_prev + own) + from_next
                    : (from_next + from_prev) + own;
    }
    if (live) mepi<T, MODE, K>(a, row, y, cf, o, dot);
  }
  mfinish<T, MODE, K>(a, dot, s_red);
}

// ---------------------------------------------------------------------------
// Tile engine for CSR without the sliced layout: the row tiles of the
// one-column engine (at most 256 rows and kLdsCap nonzeros, 2^lg lanes per
// row), staged through LDS with the next tile's matrix data loaded into
// registers while the current tile gathers.  The lanes of a row stride over
// its entries (for K <= 4 in batches of two, whose K-wide gathers are in
// flight together) with K partial sums each, summed across the row's lanes.  Long-row chunks
// are skipped: rows longer than kLdsCap are taken by a whole workgroup each
// (lanes stride over the entries, then a fixed-order workgroup sum), so a
// hub row does not serialise.
// ---------------------------------------------------------------------------

template <typename T, int MODE, int K, bool NT>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4)))
void mtile_step(MArgs<T> a) {
  __shared__ T s_val[kLdsCap];
  __shared__ int s_col[kLdsCap];
  __shared__ int s_rp[kTileRows + 1];
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  MCoef<T, K> cf;
  if (!mprologue<T, MODE, K>(a, cf, s_red, &s_flag)) return;
  double dot[K];
#pragma unroll
  for (int c = 0; c < K; ++c) dot[c] = 0.0;
  const int tid = threadIdx.x;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  TileRegs<T> R;
  Tile nxt;
  if (t0 < t1) {
    nxt = a.tiles[t0];
    if (nxt.kind == kTileLds) tile_load<NT>(a, nxt, R);
  }
  for (int t = t0; t < t1; t += step) {
    const Tile d = nxt;
    if (d.kind == kTileLds) tile_commit(d, R, s_val, s_col, s_rp);
    if (t + step < t1) {
      nxt = a.tiles[t + step];
      if (nxt.kind == kTileLds) tile_load<NT>(a, nxt, R);
    }
    if (d.kind != kTileLds) continue;
    __syncthreads();
    const int nr = d.b - d.a, lg = d.c, kb = d.d;
    const int L = 1 << lg, g = tid >> lg, sub = tid & (L - 1);
    const bool in = g < nr;
    const int i = d.a + (in ? g : 0);
    MOwn<T, K> o;
    if (in && sub == 0) mown_load<T, MODE, K>(a, i, o);
    T acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) acc[c] = T(0);
    if (in) {
      // entries per batch: two for K <= 4, one for K = 8 (register budget)
      constexpr int EB = K >= 8 ? 1 : 2;
      const int e1 = s_rp[g + 1] - kb;
      for (int e = s_rp[g] - kb + sub; e < e1; e += EB * L) {
        T vb[EB], xb[EB][K];
#pragma unroll
        for (int u = 0; u < EB; ++u) {
          const bool ok = e + u * L < e1;
          const int ee = ok ? e + u * L : e;
          vb[u] = ok ? s_val[ee] : T(0);
          const size_t base = (size_t)s_col[ee] * a.ld;
#pragma unroll
          for (int c = 0; c < K; ++c) xb[u][c] = mgat<T, MODE, K>(a, base, c, cf);
        }
#pragma unroll
        for (int u = 0; u < EB; ++u)
#pragma unroll
          for (int c = 0; c < K; ++c) acc[c] = fma(vb[u], xb[u][c], acc[c]);
      }
    }
    for (int off = L >> 1; off >= 1; off >>= 1) {
#pragma unroll
      for (int c = 0; c < K; ++c) acc[c] += __shfl_xor(acc[c], off, 64);
    }
    if (in && sub == 0) mepi<T, MODE, K>(a, i, acc, cf, o, dot);
    __syncthreads();
  }
  for (int q = blockIdx.x; q < a.nlong; q += gridDim.x) {
    const int i = a.long_rows[q];
    const int e0 = a.rp[i], e1 = a.rp[i + 1];
    T acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) acc[c] = T(0);
    for (int e = e0 + tid; e < e1; e += kWG) {
      const T vu = a.v[e];
      const size_t base = (size_t)a.ci[e] * a.ld;
#pragma unroll
      for (int c = 0; c < K; ++c) acc[c] = fma(vu, mgat<T, MODE, K>(a, base, c, cf), acc[c]);
    }
    double sum[K];
#pragma unroll
    for (int c = 0; c < K; ++c) sum[c] = (double)acc[c];
    block_sum_k<K>(sum, s_red);
    if (tid == 0) {
      MOwn<T, K> o;
      mown_load<T, MODE, K>(a, i, o);
      T tot[K];
#pragma unroll
      for (int c = 0; c < K; ++c) tot[c] = T(sum[c]);
      mepi<T, MODE, K>(a, i, tot, cf, o, dot);
    }
  }
  mfinish<T, MODE, K>(a, dot, s_red);
}

// ---------------------------------------------------------------------------
// Row engine for 3x3 BSR without the sliced layout: one lane per scalar
// row walks its block row's entries in storage order.
// ---------------------------------------------------------------------------

template <typename T, int MODE, int K>
__global__ __launch_bounds__(kWG) void mrow_step(MArgs<T> a) {
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  MCoef<T, K> cf;
  if (!mprologue<T, MODE, K>(a, cf, s_red, &s_flag)) return;
  double dot[K];
#pragma unroll
  for (int c = 0; c < K; ++c) dot[c] = 0.0;
  for (int i = blockIdx.x * kWG + threadIdx.x; i < a.n; i += gridDim.x * kWG) {
    MOwn<T, K> o;
    mown_load<T, MODE, K>(a, i, o);
    T acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) acc[c] = T(0);
    const int I = i / 3, r = i - 3 * I;
    const int e0 = a.rp[I], e1 = a.rp[I + 1];
    for (int e = e0; e < e1; ++e) {
      const int J = a.ci[e];
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const T vu = a.v[(size_t)e * 9 + 3 * r + q];
        const size_t base = (size_t)(3 * J + q) * a.ld;
#pragma unroll
        for (int c = 0; c < K; ++c) acc[c] = fma(vu, mgat<T, MODE, K>(a, base, c, cf), acc[c]);
      }
    }
    mepi<T, MODE, K>(a, i, acc, cf, o, dot);
  }
  mfinish<T, MODE, K>(a, dot, s_red);
}

// Separate form of the iteration (single-gather products, vector updates
// in streaming passes).  The n x K blocks are walked as flat arrays, two
// consecutive entries per thread and step (one 16-byte access per operand);
// the grid-wide step is a multiple of K, so a thread always meets the same
// two columns.  P_k = Z + beta P_{k-1} after the rho check ...
template <typename T, int MODE, int K>
__global__ __launch_bounds__(kWG) void mvec_p(MArgs<T> a) {
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  MCoef<T, K> cf;
  if (!mprologue<T, MODE, K>(a, cf, s_red, &s_flag)) return;
  constexpr int E = K >= 2 ? 2 : 1;
  const size_t total = (size_t)a.n * K;
  const size_t stride = (size_t)gridDim.x * kWG * E;
  const size_t first = ((size_t)blockIdx.x * kWG + threadIdx.x) * E;
  const int c0 = (int)(first % K);
  T beta[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    beta[e] = cf.c[0];
#pragma unroll
    for (int c = 1; c < K; ++c)
      if (c0 + e == c) beta[e] = cf.c[c];
  }
  for (size_t f = first; f < total; f += stride) {
    T z[E], po[E];
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = a.in0[f + e];
    if constexpr (MODE == MM_A) {
#pragma unroll
      for (int e = 0; e < E; ++e) po[e] = a.in1[f + e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if constexpr (MODE == MM_A1) a.own[f + e] = z[e];
      else a.own[f + e] = fma(beta[e], po[e], z[e]);
    }
  }
}

// ... and R_k = R_{k-1} - alpha Q, X += alpha P_k with ||r_k||^2 partials
// after the sigma check (the G^T step's prologue).
template <typename T, int K>
__global__ __launch_bounds__(kWG) void mvec_r(MArgs<T> a) {
  __shared__ double s_red[kWaves * K];
  __shared__ int s_flag;
  MCoef<T, K> cf;
  if (!mprologue<T, MM_GT, K>(a, cf, s_red, &s_flag)) return;
  constexpr int E = K >= 2 ? 2 : 1;
  const size_t total = (size_t)a.n * K;
  const size_t stride = (size_t)gridDim.x * kWG * E;
  const size_t first = ((size_t)blockIdx.x * kWG + threadIdx.x) * E;
  const int c0 = (int)(first % K);
  T nal[E], al[E];
  bool act[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    nal[e] = cf.c[0];
    al[e] = cf.c2[0];
    act[e] = cf.act[0];
#pragma unroll
    for (int c = 1; c < K; ++c)
      if (c0 + e == c) {
        nal[e] = cf.c[c];
        al[e] = cf.c2[c];
        act[e] = cf.act[c];
      }
  }
  double d[E];
#pragma unroll
  for (int e = 0; e < E; ++e) d[e] = 0.0;
  for (size_t f = first; f < total; f += stride) {
    const size_t i = f / K;
    const size_t fx = i * a.ldx + c0;
    T ro[E], q[E], pk[E], xo[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ro[e] = a.in0[f + e];
#pragma unroll
    for (int e = 0; e < E; ++e) q[e] = a.in1[f + e];
#pragma unroll
    for (int e = 0; e < E; ++e) pk[e] = a.pv[f + e];
#pragma unroll
    for (int e = 0; e < E; ++e) xo[e] = a.xv[fx + e];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const T rn = fma(nal[e], q[e], ro[e]);
      a.own[f + e] = rn;
      d[e] += (double)rn * (double)rn;
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (act[e]) a.xv[fx + e] = fma(al[e], pk[e], xo[e]);
  }
  double dot[K];
#pragma unroll
  for (int c = 0; c < K; ++c) {
    dot[c] = 0.0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (c0 + e == c) dot[c] = d[e];
  }
  mfinish<T, MM_GT, K>(a, dot, s_red);
}

// Columns of a pass: the n x kw block src into columns [0, kw) of the n x ld
// array dst (which points at the pass's first column).
template <typename T>
__global__ __launch_bounds__(kWG) void mcopy_cols(const T* __restrict__ src, int kw,
                                                  T* __restrict__ dst, int ld, int n) {
  const size_t m = (size_t)n * kw;
  for (size_t f = blockIdx.x * (size_t)kWG + threadIdx.x; f < m; f += (size_t)gridDim.x * kWG) {
    const size_t i = f / kw;
    dst[i * ld + (f - i * kw)] = src[f];
  }
}

// Start-up: R_0 = B (columns c0 .. c0 + K - 1 of the caller's n x ldb array),
// X = 0 on the same columns, partials of ||b_c||^2.
template <typename T, int K>
__global__ __launch_bounds__(kWG) void minit(const T* __restrict__ b, int ldb, T* __restrict__ r0,
                                             T* __restrict__ x, int ldx, int n,
                                             double* __restrict__ pout) {
  __shared__ double s_red[kWaves * K];
  double dot[K];
#pragma unroll
  for (int c = 0; c < K; ++c) dot[c] = 0.0;
  for (int i = blockIdx.x * kWG + threadIdx.x; i < n; i += gridDim.x * kWG) {
#pragma unroll
    for (int c = 0; c < K; ++c) {
      const T v = b[(size_t)i * ldb + c];
      r0[(size_t)i * K + c] = v;
      x[(size_t)i * ldx + c] = T(0);
      dot[c] += (double)v * (double)v;
    }
  }
  block_sum_k<K>(dot, s_red);
  if (threadIdx.x < K) {
    double v = dot[0];
#pragma unroll
    for (int c = 1; c < K; ++c)
      if ((int)threadIdx.x == c) v = dot[c];
    pout[(size_t)blockIdx.x * K + threadIdx.x] = v;
  }
}

// dL/dA over k solves: g[e] = -sum_c lambda_c[row(e)] x_c[col(e)], the sum
// taken over c = 0 .. k-1 in order (products rounded before the subtraction).
// One wavefront per block row; its lanes stride over the row's scalars.
template <typename T>
__global__ __launch_bounds__(kWG) void mgrad(const int32_t* __restrict__ rp,
                                             const int32_t* __restrict__ ci, int nbr, int bs,
                                             const T* __restrict__ lam,
                                             const T* __restrict__ x, int k,
                                             T* __restrict__ g) {
  const int lane = threadIdx.x & 63;
  const int bb = bs * bs;
  for (int I = blockIdx.x * kWaves + (threadIdx.x >> 6); I < nbr; I += gridDim.x * kWaves) {
    const int e0 = rp[I] * bb, e1 = rp[I + 1] * bb;
    for (int e = e0 + lane; e < e1; e += 64) {
      const int kb = e / bb, w = e - kb * bb;
      const int r = w / bs, cc = w - r * bs;
      const size_t li = (size_t)(I * bs + r) * k, xi = (size_t)(ci[kb] * bs + cc) * k;
      T s = T(0);
      for (int c = 0; c < k; ++c) {
#pragma clang fp contract(off)
        s = s - lam[li + c] * x[xi + c];
      }
      g[e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

template <typename T>
void fill_mat(MArgs<T>& a, const sla_mat& m, const MatView& v) {
  a.rp = v.rp;
  a.ci = v.ci;
  a.v = (const T*)v.v;
  a.nbr = (int)m.nbr;
  a.n = (int)m.n();
  a.long_rows = m.bs == 1 ? v.long_rows : nullptr;
  a.nlong = m.bs == 1 && v.long_rows ? v.nlong_rows : 0;
  if (v.sell) {
    a.sv = (const T*)v.sv;
    a.sc = v.sd ? nullptr : v.sc;
    a.sd = v.sd;
    a.soff = v.soff;
    a.nslices = v.nslices;
    a.so = v.so;
    a.sm = v.sm;
    a.ntiles = (v.nslices + kWaves - 1) / kWaves;
  } else if (m.bs == 1) {
    a.tiles = v.tiles;
    a.ntiles = v.ntiles;
  } else {
    a.ntiles = 0;
  }
}

template <typename T, int MODE, int K>
hipError_t mlaunch(const sla_mat& m, const MatView& v, const MArgs<T>& a, int grid,
                   hipStream_t s) {
  const dim3 g(grid), b(kWG);
  // slots per load batch (measured on 3D Poisson 128^3 and 2D heat 512^2:
  // 8 and 6 slots at K = 4, 3 and 4 at K = 8 gave no consistent gain)
  constexpr int U = K >= 8 ? 2 : 4;
  if (m.bs == 1 && v.sell) {
    if (v.so) hipLaunchKernelGGL((msell_step<T, MODE, K, true, U, true>), g, b, 0, s, a);
    else if (v.sd) hipLaunchKernelGGL((msell_step<T, MODE, K, true, U, false>), g, b, 0, s, a);
    else hipLaunchKernelGGL((msell_step<T, MODE, K, false, U, false>), g, b, 0, s, a);
  } else if (m.bs == 3 && v.sell) {
    // one gathered block row per lane and slot: K entries per slot, batches
    // of UB slots keep the three row partials per column within registers
    constexpr int UB = K >= 4 ? 1 : 2;
    if (v.sd) hipLaunchKernelGGL((mbsell_step<T, MODE, K, true, UB>), g, b, 0, s, a);
    else hipLaunchKernelGGL((mbsell_step<T, MODE, K, false, UB>), g, b, 0, s, a);
  } else if (m.bs == 1) {
    if (matrix_bytes(m) > mall_budget())
      hipLaunchKernelGGL((mtile_step<T, MODE, K, true>), g, b, 0, s, a);
    else
      hipLaunchKernelGGL((mtile_step<T, MODE, K, false>), g, b, 0, s, a);
  } else {
    hipLaunchKernelGGL((mrow_step<T, MODE, K>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

int mgrid(const sla_mat& m) {
  const int rows = (int)std::min<int64_t>(m.n(), (int64_t)1 << 30);
  int g = std::max(view_tiles(m, m.fwd), (rows + kWG - 1) / kWG);
  if (m.has_t) g = std::max(g, view_tiles(m, m.tr));
  return step_grid(g);
}

// Grid of the lock-step solve's kernels.  With a sliced CSR A, half the
// resident capacity (two workgroups per CU): fewer slices in flight per XCD
// keep the gathered K-wide rows of the products' operands in its L2
// (3D Poisson 128^3, 4 columns: 275 us per lock-step iteration against
// 286 us with four per CU; 2D heat 512^2: 48 against 50 us, 8 columns 86
// against 99 us).  Other layouts keep the resident grid (3x3 BSR with 4
// columns ran 35% slower at half).
int solve_grid(const sla_mat& A, const sla_mat& G) {
  int g = std::max(mgrid(A), mgrid(G));
  if (A.bs == 1 && A.fwd.sell && g >= 16) g = std::max(8, std::min(g, max_grid() / 2) & ~7);
  return g;
}

// Iteration form: products with p and r formed inside their gathers
// (fused) or single-gather products with the p and r updates in streaming
// passes (separate, the default: with K columns the fused form's two
// gathered vectors per nonzero overflow L2).  SLA_MFUSION=fused|unfused.
bool mfused() {
  const char* e = getenv("SLA_MFUSION");
  return e && !strcmp(e, "fused");
}

// Columns handled per pass: the largest of 8, 4, 2, 1 that fits k, with
// passes of 4 instead of 8 on a SELL matrix reaching further than kFarRows
// from its diagonal (3D Poisson 128^3 on the half grid: 600 us per
// 8-column lock-step iteration against 2 x 275 us for two passes of 4, and
// 620 us on the resident grid; 2D heat 512^2, whose rows reach 512 rows
// out, keeps passes of 8).
// SLA_MCHUNK=1|2|4|8 replaces the rule by a fixed cap (read once per
// process: the workspace size depends on it).
int chunk_cap() {
  static const int cap = [] {
    const char* e = getenv("SLA_MCHUNK");
    const int v = e ? atoi(e) : 0;
    return v == 1 || v == 2 || v == 4 || v == 8 ? v : 0;
  }();
  return cap;
}

int chunk_width(const sla_mat& A, int k) {
  const int cap = chunk_cap();
  const bool far = A.bs == 1 && A.fwd.sell && A.fwd.max_dist > kFarRows;
  const int lim = cap ? cap : far ? 4 : 8;
  if (k >= 8 && lim >= 8) return 8;
  if (k >= 4 && lim >= 4) return 4;
  return k >= 2 && lim >= 2 ? 2 : 1;
}

struct MWork {
  MState* st;
  double* psig;
  double* prr;
  double* prho;
  void* vec[7];  // P0 P1 R0 R1 Q T Z, n x K each
  void* xblk;    // the pass's X, n x K (only when k is cut into several passes)
};

MWork mcarve(const sla_mat& A, int kw, bool xblk, void* work) {
  MWork w;
  char* p = (char*)work;
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  w.st = (MState*)p;
  p += align_up(sizeof(MState));
  const size_t ps = align_up((size_t)max_grid() * kMaxRhs * sizeof(double));
  w.psig = (double*)p;
  p += ps;
  w.prr = (double*)p;
  p += ps;
  w.prho = (double*)p;
  p += ps;
  for (int i = 0; i < 7; ++i) {
    w.vec[i] = p;
    p += align_up((size_t)A.n() * kw * es);
  }
  w.xblk = xblk ? p : nullptr;
  return w;
}

static_assert(4 * sizeof(MState) <= kPollBytes, "polling record too small");

// One pass of K columns: b and x point at the pass's first column of the
// caller's n x ld arrays.
template <typename T, int K>
sla_status mpcg_pass(const sla_mat& A, const sla_mat& G, double eps, const T* b, int ldb, T* x,
                     int ldx, double rtol, int maxit, const MWork& w, hipStream_t s,
                     sla_solve_info* info, sla_status* cst) {
  const int n = (int)A.n();
  T *P[2] = {(T*)w.vec[0], (T*)w.vec[1]}, *R[2] = {(T*)w.vec[2], (T*)w.vec[3]};
  T *q = (T*)w.vec[4], *t = (T*)w.vec[5], *z = (T*)w.vec[6];
  const int grid = solve_grid(A, G);
  SLA_HIP(hipMemsetAsync(w.st, 0, sizeof(MState), s));

  MArgs<T> aA{}, aT{}, aG{};
  fill_mat(aA, A, A.fwd);
  fill_mat(aT, G, G.tr);
  fill_mat(aG, G, G.fwd);
  for (MArgs<T>* a : {&aA, &aT, &aG}) {
    a->st = w.st;
    a->maxit = maxit;
    a->rtol = rtol;
    a->eps = eps;
    a->ld = K;
    a->xv = x;
    a->ldx = ldx;
    a->npin = grid;
  }
  aA.pin = w.prho;
  aA.pout = w.psig;
  aA.in0 = z;
  aA.y = q;
  aT.pin = w.psig;
  aT.pout = w.prr;
  aT.in1 = q;
  aT.y = t;
  aG.pin = w.prr;
  aG.pout = w.prho;
  aG.in0 = t;
  aG.y = z;

  // separate form: vector passes around single-gather products
  const bool fused = mfused();
  MArgs<T> aV = aA, aR = aT;
  aV.in0 = z;
  aR.in1 = q;

  // start-up: R_0 = B, X = 0, ||b_c||^2; T = G^T R_0; Z_0 = G T + eps R_0
  hipLaunchKernelGGL((minit<T, K>), dim3(grid), dim3(kWG), 0, s, b, ldb, R[0], x, ldx, n, w.prr);
  SLA_HIP(hipGetLastError());
  MArgs<T> a0 = aT;
  a0.in0 = R[0];
  SLA_HIP((mlaunch<T, MM_PLAIN, K>(G, G.tr, a0, grid, s)));
  aG.k = 0;
  aG.rv = R[0];
  SLA_HIP((mlaunch<T, MM_G0, K>(G, G.fwd, aG, grid, s)));

  PollLease lease;
  sla_status pst = poll_acquire(&lease.p);
  if (pst != SLA_OK) return pst;
  // polling records in slots 0..2 (as in the one-column driver), the final
  // state after them
  static_assert(sizeof(SolverState) <= sizeof(MState), "record layout");
  SolverState* rec = (SolverState*)lease.p->host;
  SolverState* drec = (SolverState*)lease.p->dev;
  MState* mhost = (MState*)lease.p->host;
  int pend[3], pend_k[3];
  int npend = 0, pfirst = 0;
  int next_slot = 0;
  BatchPlanner plan_b(batch_iters(iteration_estimate_us(A, G, (int)sizeof(T), K, fused ? 3 : 5)),
                      rtol);
  int k = 1;
  bool finished = false;
  while (!finished) {
    const int want = k <= maxit ? plan_b.next(k) : 0;
    if (k <= maxit && npend < 2 && (want > 0 || npend == 0)) {
      const int kend = std::min(maxit, k + std::max(want, plan_b.restart()) - 1);
      const int ps = next_slot;
      next_slot = (next_slot + 1) % 3;
      ((volatile SolverState*)&rec[ps])->exit_iter = -1;
      for (int kk = k; kk <= kend; ++kk) {
        if (fused) {
          aA.k = kk;
          aA.in1 = P[(kk - 1) & 1];
          aA.own = P[kk & 1];
          if (kk == 1) SLA_HIP((mlaunch<T, MM_A1, K>(A, A.fwd, aA, grid, s)));
          else SLA_HIP((mlaunch<T, MM_A, K>(A, A.fwd, aA, grid, s)));
          aT.k = kk;
          aT.in0 = R[(kk - 1) & 1];
          aT.own = R[kk & 1];
          aT.pv = P[kk & 1];
          SLA_HIP((mlaunch<T, MM_GT, K>(G, G.tr, aT, grid, s)));
        } else {
          // P_k; Q = A P_k; R_k and X; T = G^T R_k -- one gather per product
          aV.k = kk;
          aV.in1 = P[(kk - 1) & 1];
          aV.own = P[kk & 1];
          if (kk == 1)
            hipLaunchKernelGGL((mvec_p<T, MM_A1, K>), dim3(grid), dim3(kWG), 0, s, aV);
          else
            hipLaunchKernelGGL((mvec_p<T, MM_A, K>), dim3(grid), dim3(kWG), 0, s, aV);
          SLA_HIP(hipGetLastError());
          aA.k = kk;
          aA.in0 = P[kk & 1];
          SLA_HIP((mlaunch<T, MM_AU, K>(A, A.fwd, aA, grid, s)));
          aR.k = kk;
          aR.in0 = R[(kk - 1) & 1];
          aR.own = R[kk & 1];
          aR.pv = P[kk & 1];
          hipLaunchKernelGGL((mvec_r<T, K>), dim3(grid), dim3(kWG), 0, s, aR);
          SLA_HIP(hipGetLastError());
          aT.k = kk;
          aT.in0 = R[kk & 1];
          SLA_HIP((mlaunch<T, MM_GTU, K>(G, G.tr, aT, grid, s)));
        }
        aG.k = kk;
        aG.rv = R[kk & 1];
        aG.poll = kk == kend ? drec + ps : nullptr;
        SLA_HIP((mlaunch<T, MM_G, K>(G, G.fwd, aG, grid, s)));
      }
      aG.poll = nullptr;
      pend[(pfirst + npend) % 3] = ps;
      pend_k[(pfirst + npend) % 3] = kend;
      ++npend;
      k = kend + 1;
      continue;
    }
    if (npend > 0) {
      const int ps = pend[pfirst], kb = pend_k[pfirst];
      pfirst = (pfirst + 1) % 3;
      --npend;
      SolverState r{};
      SLA_HIP(wait_poll(&rec[ps], kb, s, &w.st->done, &r));
      if (r.done) finished = true;
      else plan_b.observe(r.exit_iter, r.rr, r.bb);
      continue;
    }
    finished = true;  // k > maxit and nothing queued
  }
  // batches still queued return at once; the stream synchronization below
  // waits for them
  MState* hs = &mhost[3];
  SLA_HIP(hipMemcpyAsync(hs, w.st, sizeof(MState), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  const MState fin = *hs;

  sla_status worst = SLA_OK;
  for (int c = 0; c < K; ++c) {
    sla_status st = SLA_OK;
    int iters = 0, conv = 0;
    const int e = fin.exit_iter[c];
    switch (fin.exit_kind[c]) {
      case EX_CONV: st = SLA_OK; iters = e; conv = 1; break;
      case EX_BZERO: st = SLA_OK; iters = 0; conv = 1; break;
      case EX_MAXIT: st = SLA_NOT_CONVERGED; iters = e; break;
      case EX_MAXIT0: st = SLA_NOT_CONVERGED; iters = 0; break;
      case EX_BREAK_SIGMA: st = SLA_ERR_BREAKDOWN; iters = e - 1; break;
      case EX_BREAK_RHO: st = SLA_ERR_BREAKDOWN; iters = e - 1; break;
      case EX_BREAK_RR: st = SLA_ERR_BREAKDOWN; iters = e; break;
      case EX_NONFINITE_B: st = SLA_ERR_NONFINITE; iters = 0; break;
      default:
        set_error("solver finished without an exit record for a column");
        return SLA_ERR_HIP;
    }
    if (cst) cst[c] = st;
    if (info) {
      info[c].iterations = iters;
      info[c].converged = conv;
      info[c].bnorm = std::sqrt(fin.bb[c]);
      info[c].rel_residual = fin.bb[c] > 0 ? std::sqrt(fin.rr[c]) / std::sqrt(fin.bb[c])
                                           : (fin.exit_kind[c] == EX_BZERO ? 0.0 : 1.0);
      if (fin.exit_kind[c] == EX_MAXIT0) info[c].rel_residual = 1.0;
    }
    if (st < 0 && worst >= 0) worst = st;
    else if (st == SLA_NOT_CONVERGED && worst == SLA_OK) worst = st;
  }
  return worst;
}

template <typename T>
sla_status mpcg_impl(const sla_mat& A, const sla_mat& G, double eps, const T* b, T* x, int k,
                     double rtol, int maxit, void* work, hipStream_t s, sla_solve_info* info,
                     sla_status* cst) {
  const int kw0 = chunk_width(A, k);
  // several passes: each pass keeps its X columns contiguous in the
  // workspace (the per-iteration X update then streams whole rows) and
  // copies them into the caller's n x k array when it ends
  const bool staged = kw0 < k;
  const MWork w = mcarve(A, kw0, staged, work);
  sla_status worst = SLA_OK;
  for (int c0 = 0; c0 < k;) {
    const int kw = chunk_width(A, k - c0);
    sla_status st;
    sla_solve_info* ci = info ? info + c0 : nullptr;
    sla_status* cs = cst ? cst + c0 : nullptr;
    T* xp = staged ? (T*)w.xblk : x + c0;
    const int ldx = staged ? kw : k;
    switch (kw) {
      case 8: st = mpcg_pass<T, 8>(A, G, eps, b + c0, k, xp, ldx, rtol, maxit, w, s, ci, cs); break;
      case 4: st = mpcg_pass<T, 4>(A, G, eps, b + c0, k, xp, ldx, rtol, maxit, w, s, ci, cs); break;
      case 2: st = mpcg_pass<T, 2>(A, G, eps, b + c0, k, xp, ldx, rtol, maxit, w, s, ci, cs); break;
      default: st = mpcg_pass<T, 1>(A, G, eps, b + c0, k, xp, ldx, rtol, maxit, w, s, ci, cs); break;
    }
    if (st == SLA_ERR_HIP || st == SLA_ERR_OOM) return st;
    if (staged) {
      const size_t m = (size_t)A.n() * kw;
      const int g = (int)std::min<size_t>((m + kWG - 1) / kWG, 65536);
      hipLaunchKernelGGL(mcopy_cols<T>, dim3(g), dim3(kWG), 0, s, (const T*)w.xblk, kw, x + c0, k,
                         (int)A.n());
      SLA_HIP(hipGetLastError());
    }
    if (st < 0 && worst >= 0) worst = st;
    else if (st == SLA_NOT_CONVERGED && worst == SLA_OK) worst = st;
    c0 += kw;
  }
  if (staged) SLA_HIP(hipStreamSynchronize(s));
  return worst;
}

template <typename T, int K>
hipError_t spmm_pass(const sla_mat& A, bool transpose, const T* x, T* y, int ld, hipStream_t s) {
  const MatView& v = transpose ? A.tr : A.fwd;
  MArgs<T> a{};
  fill_mat(a, A, v);
  a.ld = ld;
  a.in0 = x;
  a.y = y;
  return mlaunch<T, MM_PLAIN, K>(A, v, a, mgrid(A), s);
}

template <typename T>
sla_status spmm_impl(const sla_mat& A, bool transpose, const T* x, T* y, int k, hipStream_t s) {
  for (int c0 = 0; c0 < k;) {
    const int kw = chunk_width(A, k - c0);
    switch (kw) {
      case 8: SLA_HIP((spmm_pass<T, 8>(A, transpose, x + c0, y + c0, k, s))); break;
      case 4: SLA_HIP((spmm_pass<T, 4>(A, transpose, x + c0, y + c0, k, s))); break;
      case 2: SLA_HIP((spmm_pass<T, 2>(A, transpose, x + c0, y + c0, k, s))); break;
      default: SLA_HIP((spmm_pass<T, 1>(A, transpose, x + c0, y + c0, k, s))); break;
    }
    c0 += kw;
  }
  return SLA_OK;
}

}  // namespace

size_t workspace_base_multi(const sla_mat& A, int k) {
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  const int kw = chunk_width(A, k);
  const size_t lockstep = align_up(sizeof(MState)) +
                          3 * align_up((size_t)max_grid() * kMaxRhs * sizeof(double)) +
                          (kw < k ? 8 : 7) * align_up((size_t)A.n() * kw * es);
  return std::max(lockstep, small_states_bytes(k));
}

size_t workspace_bytes_multi(const sla_mat& A, int k) {
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  return workspace_base_multi(A, k) +
         (A.ord_want ? 2 * align_up((size_t)A.n() * (size_t)k * es) : 0);
}

sla_status spmm(const sla_mat& A, bool transpose, const void* x, void* y, int k, hipStream_t s) {
  if (A.n() == 0 || k == 0) return SLA_OK;
  if (A.dtype == SLA_F64) return spmm_impl<double>(A, transpose, (const double*)x, (double*)y, k, s);
  return spmm_impl<float>(A, transpose, (const float*)x, (float*)y, k, s);
}

sla_status pcg_solve_multi(const sla_mat& A, const sla_mat& G, double eps, const void* b, void* x,
                           int k, double rtol, int maxit, void* work, hipStream_t s,
                           sla_solve_info* info, sla_status* cst) {
  if (A.n() == 0) {
    for (int c = 0; c < k; ++c) {
      if (info) info[c] = sla_solve_info{0, 1, 0.0, 0.0};
      if (cst) cst[c] = SLA_OK;
    }
    return SLA_OK;
  }
  // small systems: one workgroup per column, every column in one launch
  if (small_applies(A, G))
    return small_solve_batch(A, G, eps, b, x, k, rtol, maxit, work, s, info, cst);
  if (A.dtype == SLA_F64)
    return mpcg_impl<double>(A, G, eps, (const double*)b, (double*)x, k, rtol, maxit, work, s,
                             info, cst);
  return mpcg_impl<float>(A, G, eps, (const float*)b, (float*)x, k, rtol, maxit, work, s, info,
                          cst);
}

sla_status pattern_grad_multi(const sla_mat& A, const void* lam, const void* x, int k, void* grad,
                              hipStream_t s) {
  if (A.nnzb == 0) return SLA_OK;
  const int grid = (int)std::min<int64_t>((A.nbr + kWaves - 1) / kWaves, 65536);
  if (A.dtype == SLA_F64)
    hipLaunchKernelGGL(mgrad<double>, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci,
                       (int)A.nbr, (int)A.bs, (const double*)lam, (const double*)x, k,
                       (double*)grad);
  else
    hipLaunchKernelGGL(mgrad<float>, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci, (int)A.nbr,
                       (int)A.bs, (const float*)lam, (const float*)x, k, (float*)grad);
  SLA_HIP(hipGetLastError());
  return SLA_OK;
}

}  // namespace sla
