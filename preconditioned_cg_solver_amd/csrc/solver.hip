// Hot path of the gfx950 PCG library: the three fused product kernels of a
// preconditioned-CG iteration, the finalize step, the adjoint's pattern
// gradient, and the host driver.
//
// Method: CG for sparse SPD A x = b with M^-1 = G G^T + eps I ("Learning
// Sparse Approximate Inverse Preconditioners for CG Solvers on GPUs",
// "Approach": G on A's sparsity, each apply is two sparse products); adjoint
// A^T lambda = dL/dx and dL/dA_ij = -lambda_i x_j on the pattern ("torch-sla",
// Technical Summary, Methodology 2, linear systems).
//
// One iteration k (textbook PCG, stopping on the recursive residual) is
// three kernels, each one pass over one matrix with its vector work fused:
//
//   A step   q = A p_{k-1} with p_{k-1} = z_{k-1} + beta_{k-1} p_{k-2} formed
//            on the fly for every gathered column (double-buffered p) and
//            stored for owned rows, the deferred x_{k-1} = x_{k-2} +
//            alpha_{k-1} p_{k-2}, and partials of sigma = p.q;
//   G^T step t = G^T r_k with r_k = r_{k-1} - alpha_k q formed on the fly
//            (double-buffered r) and stored, and partials of ||r_k||^2;
//   G step   z_k = G t + eps r_k, partials of rho_k = r_k . z_k.
//
// That fused form runs for CSR matrices in the SELL-64 layout.  BSR matrices
// and irregular CSR take the separate form (use_fused): bare products
// q = A p_{k-1} (with p.q) and t = G^T r_k around two streaming passes,
// vec_p_update (p and the deferred x) and vec_r_update (r and ||r||^2),
// so each product gathers one vector.
//
// Each kernel begins by summing the previous kernel's per-workgroup partials
// in a fixed order (so every workgroup derives the same scalar) and the
// convergence / breakdown decisions are taken on the device; the host polls
// a small state record once per batch of iterations.  No floating-point
// atomics are used anywhere, so results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"
#include "device_util.h"

namespace sla {
namespace {

enum Mode {
  M_PLAIN = 0,  // y = M x
  M_A1 = 1,     // A step of iteration 1 (p_0 = z_0)
  M_A = 2,      // A step of iteration k >= 2
  M_GT0 = 3,    // G^T step of the start-up: r_0 = b, x = 0, t = G^T b
  M_GT = 4,     // G^T step of iteration k >= 1
  M_G0 = 5,     // G step of the start-up (checks ||b||)
  M_G = 6,      // G step of iteration k >= 1 (checks convergence)
  M_GZ = 7,     // z = G t + eps r without solver state (precondition apply)
  M_AU = 8,     // unfused A product: q = A p on a stored p, p.q partials
  M_GTU = 9     // unfused G^T product: t = G^T r on a stored r
};

template <typename T>
struct StepArgs {
  const int32_t* rp;
  const int32_t* ci;
  const T* v;
  const Tile* tiles;
  int ntiles;
  int nbr;
  int n;                 // scalar rows (vector length)
  const T* sv;           // SELL-64 copy (null: use the tiles)
  const int32_t* sc;     // absolute columns (-1 = padding), or
  const int16_t* sd;     // column - row offsets (kPad16 = padding)
  const int32_t* soff;
  int nslices;
  int sell_w;            // widest slice (slots per row)
  const int32_t* so;     // slice-offset form: offset of each slot (null: per-entry words)
  const uint8_t* sm;     // slice-offset form: slots present in each row
  double* long_part;
  int* long_cnt;
  const T* in0;   // gathered vector (PLAIN: x, A: z, GT0: b, GT: r_{k-1}, G: t)
  const T* in1;   // second gathered vector (A: p_{k-2}, GT: q)
  T* y;           // product output (PLAIN: y, A: q, GT: t, G: z)
  T* own;         // own-row vector output (A: p_{k-1}, GT: r_k)
  T* xv;          // solution (A: deferred update, GT0: zeroed)
  const T* rv;    // G: r_k
  double eps;
  const double* pin;  // partials summed in the prologue
  int npin;
  double* pout;       // partials written: [gridDim.x] workgroups then long rows
  SolverState* st;
  // G step of a batch's last iteration: the host-mapped polling record it
  // fills (done flag, iteration, ||r||^2, ||b||^2); null otherwise
  SolverState* poll;
  int k;
  int maxit;
  double rtol;
  double* hist_a;  // optional coefficient history: alpha_k at [k-1],
  double* hist_b;  // beta_k = rho_k / rho_{k-1} at [k-1], for k <= hist_len
  int hist_len;
#ifdef SLA_DEBUG
  int dbg_shrink;  // gathered columns must lie below n - dbg_shrink
#endif
};

template <typename T>
struct Coef {
  T c;
  T c2;
};

__device__ __forceinline__ void take_exit(SolverState* st, int kind, int k) {
  st->exit_kind = kind;
  st->exit_iter = k;
  st->done = 1;
}

// ---------------------------------------------------------------------------
// Prologue: scalars of the step and exit decisions.  Returns false when the
// whole workgroup must return (uniformly).
// ---------------------------------------------------------------------------

template <typename T, int MODE>
__device__ __forceinline__ bool prologue(const StepArgs<T>& a, Coef<T>& cf, double* red,
                                         int* s_flag) {
  cf.c = T(0);
  cf.c2 = T(0);
  if constexpr (MODE == M_PLAIN || MODE == M_GZ) {
    return true;
  } else {
    constexpr bool SUMS = MODE != M_AU && MODE != M_GTU && MODE != M_GT0;
    const int k = a.k;
    // Every load the prologue needs is issued before its first wait: this
    // thread's share of the partials, the state scalars written by earlier
    // kernels and the exit flag, so that they cost one memory round trip
    // rather than three in a row.  Loaded but unused when the solve is done.
    double part = 0.0, s0 = 0.0, s1 = 0.0;
    if constexpr (SUMS) part = partial_share(a.pin, a.npin);
    if constexpr (MODE == M_A) {
      s0 = a.st->rho[(k - 2) % kRing];    // rho_{k-2}
      s1 = a.st->alpha[(k - 1) % kRing];  // alpha_{k-1}
    } else if constexpr (MODE == M_GT) {
      s0 = a.st->rho[(k - 1) % kRing];    // rho_{k-1}
    } else if constexpr (MODE == M_G) {
      s0 = a.st->bb;
    }
    if (threadIdx.x == 0) *s_flag = __hip_atomic_load(&a.st->done, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (*s_flag) {
      if constexpr (MODE == M_G) {
        if (a.poll && blockIdx.x == 0 && threadIdx.x == 0) post_poll(a.poll, 1, a.k, 0.0, 0.0);
      }
      return false;
    }
    if constexpr (!SUMS) return true;
    const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
    if constexpr (MODE == M_A1 || MODE == M_A) {
      const double rho = block_sum(part, red);  // rho_{k-1}
      const bool bad = !(rho > 0.0) || !isfinite(rho);
      if (lead) {
        if (bad) take_exit(a.st, EX_BREAK_RHO, k);
        else a.st->rho[(k - 1) % kRing] = rho;
      }
      if (bad) return false;
      if constexpr (MODE == M_A) {
        const double beta = rho / s0;
        cf.c = T(beta);   // beta_{k-1}
        cf.c2 = T(s1);    // alpha_{k-1}
        if (lead && a.hist_b && k - 1 <= a.hist_len) a.hist_b[k - 2] = beta;
      }
      return true;
    } else if constexpr (MODE == M_GT) {
      const double sigma = block_sum(part, red);
      const bool bad = !(sigma > 0.0) || !isfinite(sigma);
      const double alpha = s0 / sigma;
      if (lead) {
        if (bad) {
          take_exit(a.st, EX_BREAK_SIGMA, k);
        } else {
          a.st->alpha[k % kRing] = alpha;
          a.st->sigma = sigma;
          if (a.hist_a && k <= a.hist_len) a.hist_a[k - 1] = alpha;
        }
      }
      if (bad) return false;
      cf.c = T(-alpha);
      return true;
    } else if constexpr (MODE == M_G0) {
      const double bb = block_sum(part, red);
      int ex = EX_NONE;
      if (!isfinite(bb)) ex = EX_NONFINITE_B;
      else if (bb == 0.0) ex = EX_BZERO;
      else if (a.maxit == 0) ex = EX_MAXIT0;
      if (lead) {
        a.st->bb = bb;
        a.st->rr = bb;
        if (ex != EX_NONE) take_exit(a.st, ex, 0);
      }
      return ex == EX_NONE;
    } else {  // M_G
      const double rr = block_sum(part, red);
      const double rnorm = sqrt(rr);
      const double bnorm = sqrt(s0);
      int ex = EX_NONE;
      if (!isfinite(rnorm)) ex = EX_BREAK_RR;
      else if (rnorm <= a.rtol * bnorm) ex = EX_CONV;
      else if (k == a.maxit) ex = EX_MAXIT;
      if (lead) {
        a.st->rr = rr;
        if (ex != EX_NONE) take_exit(a.st, ex, k);
        if (a.poll) post_poll(a.poll, ex != EX_NONE, k, rr, s0);
      }
      return ex == EX_NONE;
    }
  }
}

// Value of the gathered vector at column j.  Debug builds (SLA_DEBUG) check
// j against the vector length (less dbg_shrink, which a test sets from the
// host to force the check on valid input): an offender is counted in the
// solve's state and entry 0 is read instead, and the host turns the count
// into SLA_ERR_INVALID_ARG.
template <typename T, int MODE>
__device__ __forceinline__ T gat(const StepArgs<T>& a, int j, const Coef<T>& cf) {
#ifdef SLA_DEBUG
  if (j < 0 || j >= a.n - a.dbg_shrink) {
    if (a.st) atomicAdd(&a.st->dbg_bad, 1);
    j = 0;
  }
#endif
  if constexpr (MODE == M_A || MODE == M_GT) return fma(cf.c, a.in1[j], a.in0[j]);
  else return a.in0[j];
}

// Row-owned vector entries a row's epilogue needs; they do not depend on the
// row sum, so the SELL engine loads them together with the gathers.
template <typename T>
struct Own {
  T a, b, c;
};
template <typename T, int MODE>
__device__ __forceinline__ Own<T> own_load(const StepArgs<T>& a, int i) {
  Own<T> o{T(0), T(0), T(0)};
  if constexpr (MODE == M_A1 || MODE == M_GT0 || MODE == M_AU) {
    o.a = a.in0[i];
  } else if constexpr (MODE == M_A) {
    o.a = a.in1[i];
    o.b = a.in0[i];
    o.c = a.xv[i];
  } else if constexpr (MODE == M_GT) {
    o.a = a.in1[i];
    o.b = a.in0[i];
  } else if constexpr (MODE == M_G0 || MODE == M_G || MODE == M_GZ) {
    o.a = a.rv[i];
  }
  return o;
}

#ifndef SLA_NTS_MASK
#define SLA_NTS_MASK 3
#endif
// Output stores.  Outputs with no reuse before the next iteration (x and p
// of the A step: bits 1 and 2 of SLA_NTS_MASK; bit 4 would add q, bit 8 the
// result of a plain product) are stored
// non-temporally, so they do not sit dirty in L2 and need no write-back at
// the kernel boundary; outputs the next kernel consumes keep normal stores.
template <int BIT, typename U>
__device__ __forceinline__ void st_out(U* p, U v) {
  if constexpr ((SLA_NTS_MASK & BIT) != 0) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// Row epilogue from preloaded row-owned entries (same arithmetic as epi()).
template <typename T, int MODE>
__device__ __forceinline__ double epi_own(const StepArgs<T>& a, int i, T acc, const Coef<T>& cf,
                                          const Own<T>& o) {
  if constexpr (MODE == M_PLAIN) {
    st_out<8>(a.y + i, acc);
    return 0.0;
  } else if constexpr (MODE == M_GTU) {
    st_out<0>(a.y + i, acc);
    return 0.0;
  } else if constexpr (MODE == M_AU) {
    st_out<0>(a.y + i, acc);
    return (double)o.a * (double)acc;
  } else if constexpr (MODE == M_A1) {
    st_out<2>(a.own + i, o.a);
    st_out<4>(a.y + i, acc);
    return (double)o.a * (double)acc;
  } else if constexpr (MODE == M_A) {
    const T pn = fma(cf.c, o.a, o.b);
    st_out<2>(a.own + i, pn);
    st_out<1>(a.xv + i, fma(cf.c2, o.a, o.c));
    st_out<4>(a.y + i, acc);
    return (double)pn * (double)acc;
  } else if constexpr (MODE == M_GT0) {
    st_out<0>(a.own + i, o.a);
    st_out<1>(a.xv + i, T(0));
    st_out<0>(a.y + i, acc);
    return (double)o.a * (double)o.a;
  } else if constexpr (MODE == M_GT) {
    const T rn = fma(cf.c, o.a, o.b);
    st_out<0>(a.own + i, rn);
    st_out<0>(a.y + i, acc);
    return (double)rn * (double)rn;
  } else {
    const T zv = fma(T(a.eps), o.a, acc);
    st_out<0>(a.y + i, zv);
    return (double)o.a * (double)zv;
  }
}

// Row epilogue: stores and the row's contribution to the fused dot product.
template <typename T, int MODE>
__device__ __forceinline__ double epi(const StepArgs<T>& a, int i, T acc, const Coef<T>& cf) {
  if constexpr (MODE == M_PLAIN || MODE == M_GTU) {
    a.y[i] = acc;
    return 0.0;
  } else if constexpr (MODE == M_AU) {
    a.y[i] = acc;
    return (double)a.in0[i] * (double)acc;
  } else if constexpr (MODE == M_A1) {
    const T pn = a.in0[i];
    a.own[i] = pn;
    a.y[i] = acc;
    return (double)pn * (double)acc;
  } else if constexpr (MODE == M_A) {
    const T po = a.in1[i];
    const T pn = fma(cf.c, po, a.in0[i]);
    a.own[i] = pn;
    a.xv[i] = fma(cf.c2, po, a.xv[i]);
    a.y[i] = acc;
    return (double)pn * (double)acc;
  } else if constexpr (MODE == M_GT0) {
    const T rn = a.in0[i];
    a.own[i] = rn;
    a.xv[i] = T(0);
    a.y[i] = acc;
    return (double)rn * (double)rn;
  } else if constexpr (MODE == M_GT) {
    const T rn = fma(cf.c, a.in1[i], a.in0[i]);
    a.own[i] = rn;
    a.y[i] = acc;
    return (double)rn * (double)rn;
  } else {  // G0, G, GZ
    const T rv = a.rv[i];
    const T zv = fma(T(a.eps), rv, acc);
    a.y[i] = zv;
    return (double)rv * (double)zv;
  }
}

template <typename T>
__device__ __forceinline__ T shfl_xor_t(T v, int m) {
  return __shfl_xor(v, m, 64);
}

#ifndef SLA_ROW_BATCH
#define SLA_ROW_BATCH 4
#endif


// Sum of one row's entries [e0, e1) (stride L) from LDS: batches of
// SLA_ROW_BATCH entries load their values and columns, then issue all the
// gathers, then accumulate in entry order (the order is fixed, so results do
// not depend on the batching).
template <typename T, int MODE>
__device__ __forceinline__ T row_sum_lds(const StepArgs<T>& a, const T* s_val, const int* s_col,
                                         int e0, int e1, int L, const Coef<T>& cf) {
  constexpr int U = SLA_ROW_BATCH;
  T acc = T(0);
  for (int e = e0; e < e1; e += U * L) {
    T vv[U], xx[U];
    int cc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ee = e + u * L;
      const bool in = ee < e1;
      vv[u] = in ? s_val[ee] : T(0);
      cc[u] = in ? s_col[ee] : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) xx[u] = cc[u] >= 0 ? gat<T, MODE>(a, cc[u], cf) : T(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (cc[u] >= 0) acc = fma(vv[u], xx[u], acc);
  }
  return acc;
}

// ---------------------------------------------------------------------------
// CSR engine: tiles staged through LDS (2^c lanes per row) and long-row
// chunks combined by the last finishing chunk (integer ticket).
// ---------------------------------------------------------------------------

static_assert(kTileRows == kWG, "one row pointer per thread when staging a tile");

// Every step kernel must keep kWaves-wide workgroups resident four per CU
// (the grid is sized for that, see occupancy_grid): the plain, preconditioner
// tail and separate G^T forms would otherwise take 130+ VGPRs, fall to three
// waves per SIMD and run a quarter of their workgroups as a second round.
// LDS of the tile engine.
template <typename T>
struct CsrLds {
  T val[kLdsCap];
  int col[kLdsCap];
  int rp[kTileRows + 1];
};

// The tile engine's work for one workgroup: tiles t0, t0 + step, ... < t1
// of the view in `a`; returns the workgroup's share of the step's dot
// product.  `nwg` is the number of workgroups the partials array starts
// with (long rows' dot products follow them).
template <typename T, int MODE, bool NT>
__device__ __forceinline__ double csr_tiles(const StepArgs<T>& a, const Coef<T>& cf, int t0,
                                            int t1, int step, int nwg, CsrLds<T>& L,
                                            double* s_red, int* s_flag) {
  const int tid = threadIdx.x;
  double dot = 0.0;
  TileRegs<T> R;
  Tile nxt;
  if (t0 < t1) {
    nxt = a.tiles[t0];
    if (nxt.kind == kTileLds) tile_load<NT>(a, nxt, R);
  }
  for (int t = t0; t < t1; t += step) {
    const Tile d = nxt;
    if (d.kind == kTileLds) {
      tile_commit(d, R, L.val, L.col, L.rp);
      if (t + step < t1) {
        nxt = a.tiles[t + step];
        if (nxt.kind == kTileLds) tile_load<NT>(a, nxt, R);
      }
      __syncthreads();
      const int r0 = d.a, nr = d.b - d.a, lg = d.c, kb = d.d;
      const int W = 1 << lg, g = tid >> lg, sub = tid & (W - 1);
      T acc = T(0);
      if (g < nr) acc = row_sum_lds<T, MODE>(a, L.val, L.col, L.rp[g] - kb + sub, L.rp[g + 1] - kb,
                                             W, cf);
      for (int off = W >> 1; off >= 1; off >>= 1) acc += shfl_xor_t(acc, off);
      if (g < nr && sub == 0) dot += epi<T, MODE>(a, r0 + g, acc, cf);
      __syncthreads();
    } else {
      // chunk [d.b, d.c) of long row d.a, four loads in flight per thread
      double acc = 0.0;
      for (int k = d.b + tid; k < d.c; k += 4 * kWG) {
        T vv[4], xx[4];
        int cc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int kk = k + u * kWG;
          const bool in = kk < d.c;
          vv[u] = in ? ld_stream<NT>(a.v + kk) : T(0);
          cc[u] = in ? ld_stream<NT>(a.ci + kk) : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) xx[u] = cc[u] >= 0 ? gat<T, MODE>(a, cc[u], cf) : T(0);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (cc[u] >= 0) acc += (double)vv[u] * (double)xx[u];
      }
      const double cs = block_sum(acc, s_red);
      const int lr = d.pad[0], nch = d.pad[1], first = d.pad[2];
      bool finish = false;
      double total = cs;
      if (nch > 1) {
        if (tid == 0) {
          __hip_atomic_store(&a.long_part[d.d], cs, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __threadfence();
          const int ticket = atomicAdd(&a.long_cnt[lr], 1);
          *s_flag = (ticket == nch - 1);
        }
        __syncthreads();
        finish = *s_flag;
        __syncthreads();
        if (finish && tid == 0) {
          __threadfence();
          total = 0.0;
          for (int c = 0; c < nch; ++c)
            total += __hip_atomic_load(&a.long_part[first + c], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
          a.long_cnt[lr] = 0;
        }
      } else {
        finish = true;
      }
      if (finish && tid == 0) {
        const double c = epi<T, MODE>(a, d.a, T(total), cf);
        if (a.pout) a.pout[nwg + lr] = c;
      }
      if (t + step < t1) {
        nxt = a.tiles[t + step];
        if (nxt.kind == kTileLds) tile_load<NT>(a, nxt, R);
      }
    }
  }
  return dot;
}

template <typename T, int MODE, bool NT>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4)))
void csr_step(StepArgs<T> a) {
  __shared__ CsrLds<T> L;
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  const double dot = csr_tiles<T, MODE, NT>(a, cf, t0, t1, step, gridDim.x, L, s_red, &s_flag);
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double s = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
  }
}

// Column-block product (y_b = A_b x for every block b of a ColBlockSet):
// workgroup w takes block w % kColBlocks (round-robin dispatch places the
// workgroups of one block on one XCD) and that block's tiles w /
// kColBlocks, w / kColBlocks + gridDim.x / kColBlocks, ...; the result of
// block b goes to part + b n.  The gathered vector is the plain in0 (the
// separate iteration form's stored p, r or t).  With `st` set the launch
// returns at once after the solve's exit.
template <typename T>
struct BlockArgs {
  StepArgs<T> blk[kColBlocks];
  const SolverState* st;
};
static_assert(sizeof(BlockArgs<double>) <= 4096, "kernel arguments must fit 4 KiB");

template <typename T, bool NT>
__global__ __launch_bounds__(kWG) __attribute__((amdgpu_waves_per_eu(4)))
void csr_blk_step(BlockArgs<T> ba) {
  __shared__ CsrLds<T> L;
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  if (ba.st) {
    if (threadIdx.x == 0)
      s_flag = __hip_atomic_load(&ba.st->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (s_flag) return;
  }
  const int b = blockIdx.x % kColBlocks, nwg = gridDim.x / kColBlocks;
  const StepArgs<T>& a = ba.blk[b];
  const Coef<T> cf{T(0), T(0)};
  (void)csr_tiles<T, M_PLAIN, NT>(a, cf, blockIdx.x / kColBlocks, a.ntiles, nwg, nwg, L, s_red,
                                  &s_flag);
}

// The eight block results of every row (block b's at part + b stride)
// added in block order, then the
// step's own row epilogue (q and p.q; t; z = G t + eps r and r.z; or y).
template <typename T, int MODE>
__global__ __launch_bounds__(kWG) void blk_reduce(StepArgs<T> a, const T* __restrict__ part,
                                                  size_t stride) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  double dot = 0.0;
  for (int i = blockIdx.x * kWG + threadIdx.x; i < a.n; i += gridDim.x * kWG) {
    T v[kColBlocks];
#pragma unroll
    for (int b = 0; b < kColBlocks; ++b) v[b] = part[b * stride + i];
    T acc = v[0];
#pragma unroll
    for (int b = 1; b < kColBlocks; ++b) acc += v[b];
    dot += epi<T, MODE>(a, i, acc, cf);
  }
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double s = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
  }
}

// ---------------------------------------------------------------------------
// SELL-64 engine: one wavefront per slice of 64 rows, lane l owns row
// 64 s + l and reads its slots at soff[s] + 64 j + l, so every value and
// column load of a wavefront is one contiguous 512 / 256 byte access.  No
// LDS and no barrier inside the slice loop: waves advance independently.
// ---------------------------------------------------------------------------

// Raw column word of a slot and its decoding: absolute int32 columns (-1 =
// padding) or int16 offsets from the row (kPad16 = padding).  Loads are
// unconditional (the SELL arrays carry a batch of padding slots past the last
// slice), so a batch issues all its loads back to back; masking happens after.
template <bool NT, bool I16, typename T>
__device__ __forceinline__ int sell_raw(const StepArgs<T>& a, int idx) {
  if constexpr (I16) return ld_stream<NT>(a.sd + idx);
  else return ld_stream<NT>(a.sc + idx);
}
template <bool I16>
__device__ __forceinline__ int sell_decode(int raw, int row, bool in) {
  if constexpr (I16) return (in && raw != kPad16) ? row + raw : -1;
  else return in ? raw : -1;
}

// One batch of U slots starting at slot j of a slice: value, column and
// gathered entry (0 for padding) for every slot.
// OFS: slice-offset form, the slot's offset from the per-slot table and
// the row's mask of present slots (`mask`).
template <typename T, int MODE, bool NT, bool I16, int U, bool OFS>
__device__ __forceinline__ void sell_batch(const StepArgs<T>& a, int off, int lane, int row,
                                           int j, int w, int mask, const Coef<T>& cf,
                                           T (&v)[U], T (&x)[U]) {
  int raw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int idx = off + (j + u) * kSlice + lane;
    v[u] = ld_stream<NT>(a.sv + idx);
    if constexpr (OFS && MODE == M_PLAIN)
      raw[u] = __builtin_amdgcn_readfirstlane(a.so[off / kSlice + j + u]);
    else if constexpr (OFS)  // slice-uniform: kept in a scalar register
      raw[u] = __builtin_amdgcn_readfirstlane(ld_stream<NT>(a.so + off / kSlice + j + u));
    else raw[u] = sell_raw<NT, I16>(a, idx);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int c = OFS ? (((mask >> (j + u)) & 1) ? row + raw[u] : -1)
                      : sell_decode<I16>(raw[u], row, j + u < w);
    const T g = gat<T, MODE>(a, c >= 0 ? c : 0, cf);
    x[u] = c >= 0 ? g : T(0);
    if (c < 0) v[u] = T(0);
  }
}

template <typename T, int MODE, bool NT, bool I16, int U, bool OFS>
__global__ __launch_bounds__(kWG) void sell_step(StepArgs<T> a) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  const int lane = threadIdx.x & (kSlice - 1), wv = threadIdx.x / kSlice;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  // The first batch of slots of the next slice is kept in registers: it is
  // loaded while the current slice does its gathers (and, for the first
  // slice, while the prologue sums the partials).
  T hv[U];
  int hr[U];
  int hoff = 0, hw = 0, hm = 0;
  // SCL: the plain product takes the slice's start, width and slot offsets
  // as wavefront-uniform scalars (one wavefront per slice); measured faster
  // there (SpMV streamed from HBM 88 -> 95% of peak on 3D Poisson 128^3)
  // and slower in the iteration's steps, which keep vector loads.
  constexpr bool SCL = OFS && MODE == M_PLAIN;
  auto uni = [](int v) { return SCL ? __builtin_amdgcn_readfirstlane(v) : v; };
  auto load_head = [&](int sl) {
    sl = uni(sl);
    hoff = 0;
    hw = 0;
    hm = 0;
    if (sl < a.nslices) {
      hoff = uni(a.soff[sl]);
      hw = (uni(a.soff[sl + 1]) - hoff) / kSlice;
      if constexpr (OFS) hm = ld_stream<NT>(a.sm + sl * kSlice + lane);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int idx = hoff + u * kSlice + lane;
      hv[u] = ld_stream<NT>(a.sv + idx);
      if constexpr (SCL) hr[u] = uni(a.so[hoff / kSlice + u]);
      else if constexpr (OFS) hr[u] = ld_stream<NT>(a.so + hoff / kSlice + u);
      else hr[u] = sell_raw<NT, I16>(a, idx);
    }
  };
  if (t0 < t1) load_head(t0 * kWaves + wv);
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  double dot = 0.0;
  for (int t = t0; t < t1; t += step) {
    const int sl = t * kWaves + wv;
    const int off = hoff, w = hw, m = hm;
    T cv[U];
    int cr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cv[u] = hv[u];
      cr[u] = OFS ? __builtin_amdgcn_readfirstlane(hr[u]) : hr[u];
    }
    if (t + step < t1) load_head((t + step) * kWaves + wv);
    if (sl >= a.nslices) continue;
    const int row = sl * kSlice + lane;
    const bool live = row < a.nbr;
    T xx[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = OFS ? (((m >> u) & 1) ? row + cr[u] : -1) : sell_decode<I16>(cr[u], row, u < w);
      const T g = gat<T, MODE>(a, c >= 0 ? c : 0, cf);
      xx[u] = c >= 0 ? g : T(0);
      if (c < 0) cv[u] = T(0);
    }
    const Own<T> o = own_load<T, MODE>(a, live ? row : 0);
    T acc = T(0);
#pragma unroll
    for (int u = 0; u < U; ++u) acc = fma(cv[u], xx[u], acc);
    for (int j = U; j < w; j += U) {
      T vv[U], yy[U];
      sell_batch<T, MODE, NT, I16, U, OFS>(a, off, lane, row, j, w, m, cf, vv, yy);
#pragma unroll
      for (int u = 0; u < U; ++u) acc = fma(vv[u], yy[u], acc);
    }
    if (live) dot += epi_own<T, MODE>(a, row, acc, cf, o);
  }
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double s = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
  }
}

// Slice-offset form with a window in LDS: a workgroup takes kWaves
// consecutive slices (a tile of R = 256 rows) and first writes the gathered
// vector's value (z + beta p_old, r - alpha q, ... as gat() forms it) for
// every row of [the tile's first row - kWinHalo, its last row + kWinHalo]
// into LDS, each row once and with coalesced loads; a slot whose offset lies
// within the halo (the slice-offset form gives every slot one offset for the
// whole slice, so the test is wavefront-uniform) then reads LDS, and only
// the far offsets gather from memory.  On the 3D 7-point stencil that serves
// the offsets 0, +-1 and +-128 of every slice from LDS and leaves the two
// +-16,384 planes to the caches.  The next tile's window entries and each
// wavefront's next slice head (its first U values and offsets, and its row
// masks) are loaded into registers while the current tile computes.  Every
// row adds its slots in the same order and with the same values as
// sell_step, so the results are bit-identical to it.
template <typename T, int MODE, bool NT, int U>
__global__ __launch_bounds__(kWG) void sell_win_step(StepArgs<T> a) {
  constexpr int R = kWaves * kSlice;
  constexpr int WN = R + 2 * kWinHalo;
  constexpr int PER = (WN + kWG - 1) / kWG;
  constexpr bool TWO = MODE == M_A || MODE == M_GT;  // gat() reads in0 and in1
  // A and G^T steps: the tile's own rows take their two operands (z and
  // p_old, r and q) from the window loads, kept in LDS, instead of reading
  // them from memory a second time
  constexpr bool OWNW = MODE == M_A || MODE == M_GT;
  __shared__ T gs[WN];
  __shared__ T gz[OWNW ? R : 1], gq[OWNW ? R : 1];
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  const int lane = threadIdx.x & (kSlice - 1), wv = threadIdx.x / kSlice;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  // next tile: raw window entries and this wavefront's slice head
  T w0[PER], w1[PER];
  T hv[U];
  int hr[U];
  int hoff = 0, hw = 0, hm = 0;
  auto fetch = [&](int t) {
    const int wb = t * R - kWinHalo;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = threadIdx.x + p * kWG, r = wb + i;
      const bool in = i < WN && r >= 0 && r < a.n;
      w0[p] = in ? a.in0[r] : T(0);
      if constexpr (TWO) w1[p] = in ? a.in1[r] : T(0);
    }
    const int sl = t * kWaves + wv;
    hoff = 0;
    hw = 0;
    hm = 0;
    if (sl < a.nslices) {
      hoff = a.soff[sl];
      hw = (a.soff[sl + 1] - hoff) / kSlice;
      hm = ld_stream<NT>(a.sm + sl * kSlice + lane);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      hv[u] = ld_stream<NT>(a.sv + hoff + u * kSlice + lane);
      hr[u] = ld_stream<NT>(a.so + hoff / kSlice + u);
    }
  };
  if (t0 < t1) fetch(t0);
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  double dot = 0.0;
  for (int t = t0; t < t1; t += step) {
    const int wb = t * R - kWinHalo;
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = threadIdx.x + p * kWG;
      if (i < WN) {
        if constexpr (TWO) gs[i] = fma(cf.c, w1[p], w0[p]);
        else gs[i] = w0[p];
        if constexpr (OWNW) {
          const int k = i - kWinHalo;
          if (k >= 0 && k < R) {
            gz[k] = w0[p];
            gq[k] = w1[p];
          }
        }
      }
    }
    const int off = hoff, w = hw, m = hm;
    T cv[U];
    // a slot's offset is the same for every row of the slice: held in a
    // scalar register, the near / far test below is a uniform branch
    int cr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cv[u] = hv[u];
      cr[u] = __builtin_amdgcn_readfirstlane(hr[u]);
    }
    __syncthreads();
    if (t + step < t1) fetch(t + step);
    const int sl = t * kWaves + wv;
    if (sl < a.nslices) {
      const int row = sl * kSlice + lane;
      const bool live = row < a.nbr;
      Own<T> o{T(0), T(0), T(0)};
      if constexpr (OWNW) {
        o.a = gq[threadIdx.x];
        o.b = gz[threadIdx.x];
        if constexpr (MODE == M_A) o.c = a.xv[live ? row : 0];
      } else {
        o = own_load<T, MODE>(a, live ? row : 0);
      }
      T acc = T(0);
      for (int j = 0; j < w; j += U) {
        if (j > 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            cv[u] = ld_stream<NT>(a.sv + off + (j + u) * kSlice + lane);
            cr[u] = __builtin_amdgcn_readfirstlane(ld_stream<NT>(a.so + off / kSlice + j + u));
          }
        }
        T x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const bool ok = (m >> (j + u)) & 1;
          // a row without this slot (padding rows of the last slice
          // included) reads its own window entry or entry 0, never past n
          T g;
          if (cr[u] >= -kWinHalo && cr[u] <= kWinHalo) g = gs[(ok ? row + cr[u] : row) - wb];
          else g = gat<T, MODE>(a, ok ? row + cr[u] : 0, cf);
          x[u] = ok ? g : T(0);
          if (!ok) cv[u] = T(0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = fma(cv[u], x[u], acc);
      }
      if (live) dot += epi_own<T, MODE>(a, row, acc, cf, o);
    }
    __syncthreads();
  }
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double sd = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = sd;
  }
}

// ---------------------------------------------------------------------------
// Sliced-ELL engine for 3x3 BSR: one wavefront per slice of 21 block rows.
// Lane l = 3 i + c takes local block row i and block component c: for every
// block slot it gathers only entry c of the block column (two gathers for
// the A and G^T steps, one otherwise, instead of six or three per lane) and
// reads column c of the block (per block row r one load of 63 values inside
// four aligned 128-byte lines, bsell_val), accumulating the three row
// partials sum_slots v[r][c] x_c.
// After the last slot the three lanes of a block row add their partials for
// row r in component order 0, 1, 2 (two cross-lane reads per slice), and
// lane 3 i + r runs the epilogue of scalar row 3 (21 s + i) + r.  Loads run
// one batch of U slots ahead of the gathers, across slice boundaries.
// ---------------------------------------------------------------------------

template <typename T, int MODE, bool NT, bool I16, int U>
__global__ __launch_bounds__(kWG) void bsell_step(StepArgs<T> a) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // lane 63 mirrors lane 60 (block row 20, component 0) and stores nothing
  const int li = min(lane / 3, kBSlice - 1), c = lane - 3 * (lane / 3);
  const bool lane_live = lane < 3 * kBSlice;
  // lanes holding the same block row's partials, by component distance
  const int src_prev = 3 * li + (c + 2) % 3, src_next = 3 * li + (c + 1) % 3;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  // The wave's batches of U slots form one stream over its slices: the
  // loads of the next batch (possibly the next slice's first) are issued
  // before the current batch gathers, so one batch is always in flight.
  T nv[U][3];
  int nc[U];
  int pre_sl = -1;  // slice whose first batch sits in nv, if any
  auto load_batch = [&](int q0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // loads past the slice end stay inside the arrays' padding tail
      const int q = q0 + u;
      nc[u] = sell_raw<NT, I16>(a, q * kBSlotCols + li);
#pragma unroll
      for (int r = 0; r < 3; ++r) nv[u][r] = ld_stream<NT>(a.sv + bsell_val(q, r, c, li));
    }
  };
  auto slice_of = [&](int t) { return t * kWaves + wv; };
  if (t0 < t1 && slice_of(t0) < a.nslices) {
    const int sl = slice_of(t0), off = a.soff[sl];
    if (a.soff[sl + 1] > off) {
      load_batch(off);
      pre_sl = sl;
    }
  }
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  double dot = 0.0;
  for (int t = t0; t < t1; t += step) {
    const int sl = slice_of(t);
    if (sl >= a.nslices) break;
    const int off = a.soff[sl], w = a.soff[sl + 1] - off;
    const int brow = sl * kBSlice + li;
    const bool live = lane_live && brow < a.nbr;
    const int row = 3 * brow + c;
    const Own<T> o = own_load<T, MODE>(a, live ? row : 0);
    if (w > 0 && pre_sl != sl) load_batch(off);
    // next slice with slots, for the prefetch that crosses the boundary
    const int sl_n = t + step < t1 ? slice_of(t + step) : a.nslices;
    const int off_n = sl_n < a.nslices ? a.soff[sl_n] : 0;
    const bool has_n = sl_n < a.nslices && a.soff[sl_n + 1] > off_n;
    T acc[3] = {T(0), T(0), T(0)};
    for (int j = 0; j < w; j += U) {
      T cv[U][3];
      int cc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cc[u] = nc[u];
#pragma unroll
        for (int r = 0; r < 3; ++r) cv[u][r] = nv[u][r];
      }
      if (j + U < w) {
        load_batch(off + j + U);
      } else if (has_n) {
        load_batch(off_n);
        pre_sl = sl_n;
      }
      T g[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int bc = sell_decode<I16>(cc[u], brow, j + u < w);
        ok[u] = bc >= 0;
        const T x = gat<T, MODE>(a, ok[u] ? 3 * bc + c : 0, cf);
        g[u] = ok[u] ? x : T(0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int r = 0; r < 3; ++r) acc[r] = fma(ok[u] ? cv[u][r] : T(0), g[u], acc[r]);
      }
    }
    // row c of this block row: own partial (component c) plus those of
    // components c - 1 and c + 1 (mod 3), read from the neighbouring lanes,
    // added in component order
    const T own = c == 0 ? acc[0] : (c == 1 ? acc[1] : acc[2]);
    const T for_next = c == 0 ? acc[1] : (c == 1 ? acc[2] : acc[0]);  // row c + 1
    const T for_prev = c == 0 ? acc[2] : (c == 1 ? acc[0] : acc[1]);  // row c - 1
    const T from_prev = __shfl(for_next, src_prev, 64);   // component c - 1
    const T from_next = __shfl(for_prev, src_next, 64);   // component c + 1
    const T y = c == 0 ? (own + from_next) + from_prev
              : c == 1 ? (from_prev + own) + from_next
                       : (from_next + from_prev) + own;
    if (live) dot += epi_own<T, MODE>(a, row, y, cf, o);
  }
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double s = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
  }
}

// ---------------------------------------------------------------------------
// BSR(3x3) engine: kBsrLanes lanes per block row stream the row's blocks
// (9 values each, row-major) contiguously and keep three row accumulators.
// ---------------------------------------------------------------------------

template <typename T, int MODE, bool NT>
__global__ __launch_bounds__(kWG) void bsr3_step(StepArgs<T> a) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  const int g = threadIdx.x / kBsrLanes, sub = threadIdx.x % kBsrLanes;
  double dot = 0.0;
  int t0, t1, step;
  tile_range(a.ntiles, t0, t1, step);
  for (int t = t0; t < t1; t += step) {
    const int I = t * kBsrTileRows + g;
    T acc0 = T(0), acc1 = T(0), acc2 = T(0);
    if (I < a.nbr) {
      const int e0 = ld_stream<NT>(a.rp + I) * 9, e1 = ld_stream<NT>(a.rp + I + 1) * 9;
      // batches of kB values per lane: loads first, then gathers, then the
      // accumulation in value order
      constexpr int kB = 8;
      for (int e = e0 + sub; e < e1; e += kB * kBsrLanes) {
        T vv[kB], xx[kB];
        int rr[kB], cc[kB];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int ee = e + u * kBsrLanes;
          const bool in = ee < e1;
          const int kb = ee / 9;
          const int w = ee - kb * 9;
          rr[u] = in ? w / 3 : -1;
          vv[u] = in ? ld_stream<NT>(a.v + ee) : T(0);
          cc[u] = in ? 3 * ld_stream<NT>(a.ci + kb) + (w - 3 * (w / 3)) : 0;
        }
#pragma unroll
        for (int u = 0; u < kB; ++u) xx[u] = rr[u] >= 0 ? gat<T, MODE>(a, cc[u], cf) : T(0);
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          if (rr[u] == 0) acc0 = fma(vv[u], xx[u], acc0);
          else if (rr[u] == 1) acc1 = fma(vv[u], xx[u], acc1);
          else if (rr[u] == 2) acc2 = fma(vv[u], xx[u], acc2);
        }
      }
    }
#pragma unroll
    for (int off = kBsrLanes / 2; off >= 1; off >>= 1) {
      acc0 += shfl_xor_t(acc0, off);
      acc1 += shfl_xor_t(acc1, off);
      acc2 += shfl_xor_t(acc2, off);
    }
    if (I < a.nbr && sub < 3) {
      const T accr = sub == 0 ? acc0 : (sub == 1 ? acc1 : acc2);
      dot += epi<T, MODE>(a, 3 * I + sub, accr, cf);
    }
  }
  if constexpr (MODE != M_PLAIN && MODE != M_GZ && MODE != M_GTU) {
    const double s = block_sum(dot, s_red);
    if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
  }
}

// ---------------------------------------------------------------------------
// Vector passes of the unfused iteration (matrices whose gathers have no
// locality: forming p and r on the fly would double the random gathers).
// ---------------------------------------------------------------------------

// p_{k-1} = z_{k-1} + beta_{k-1} p_{k-2} and the deferred x update; the
// prologue is the A step's (rho, beta, alpha_{k-1}, breakdown).
template <typename T, int MODE>
__global__ __launch_bounds__(kWG) void vec_p_update(StepArgs<T> a) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  Coef<T> cf;
  if (!prologue<T, MODE>(a, cf, s_red, &s_flag)) return;
  // four grid strides per round (predicated past n), all loads issued
  // before the stores
  const int stride = gridDim.x * kWG;
  for (long long i = blockIdx.x * kWG + threadIdx.x; i < a.n; i += 4LL * stride) {
    T z[4], po[4], xv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long e = i + (long long)u * stride;
      const bool in = e < a.n;
      z[u] = in ? a.in0[e] : T(0);
      if constexpr (MODE != M_A1) {
        po[u] = in ? a.in1[e] : T(0);
        xv[u] = in ? a.xv[e] : T(0);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long e = i + (long long)u * stride;
      if (e >= a.n) break;
      if constexpr (MODE == M_A1) {
        st_out<2>(a.own + e, z[u]);
      } else {
        st_out<2>(a.own + e, fma(cf.c, po[u], z[u]));
        st_out<1>(a.xv + e, fma(cf.c2, po[u], xv[u]));
      }
    }
  }
}

// r_k = r_{k-1} - alpha_k q and ||r_k||^2 partials; the prologue is the G^T
// step's (sigma, alpha_k, breakdown).  Each thread adds its entries in index
// order.
template <typename T>
__global__ __launch_bounds__(kWG) void vec_r_update(StepArgs<T> a) {
  __shared__ double s_red[kWaves];
  __shared__ int s_flag;
  Coef<T> cf;
  if (!prologue<T, M_GT>(a, cf, s_red, &s_flag)) return;
  double dot = 0.0;
  const int stride = gridDim.x * kWG;
  for (long long i = blockIdx.x * kWG + threadIdx.x; i < a.n; i += 4LL * stride) {
    T ro[4], q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long e = i + (long long)u * stride;
      ro[u] = e < a.n ? a.in0[e] : T(0);
      q[u] = e < a.n ? a.in1[e] : T(0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long long e = i + (long long)u * stride;
      if (e >= a.n) break;
      const T rn = fma(cf.c, q[u], ro[u]);
      a.own[e] = rn;
      dot += (double)rn * (double)rn;
    }
  }
  const double s = block_sum(dot, s_red);
  if (threadIdx.x == 0) a.pout[blockIdx.x] = s;
}

// ---------------------------------------------------------------------------
// Finalize: apply the pending x update of the last iteration whose alpha was
// computed (the A step of the next iteration would have applied it).
// ---------------------------------------------------------------------------

template <typename T>
__global__ void finalize_x(const SolverState* __restrict__ st, T* __restrict__ x,
                           const T* __restrict__ p0, const T* __restrict__ p1, int n) {
  const int kind = st->exit_kind, k = st->exit_iter;
  int upd = -1;
  if (kind == EX_CONV || kind == EX_MAXIT || kind == EX_BREAK_RR) upd = k;
  else if (kind == EX_BREAK_RHO && k >= 2) upd = k - 1;
  if (upd < 1) return;
  const T al = T(st->alpha[upd % kRing]);
  const T* p = (upd & 1) ? p1 : p0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    x[i] = fma(al, p[i], x[i]);
}

// ---------------------------------------------------------------------------
// SAI-loss probe term || y / s - w ||^2 with y = A M^-1 w: workgroup partials,
// then one workgroup adds them in index order.
// ---------------------------------------------------------------------------

template <typename T>
__global__ __launch_bounds__(kWG) void sai_partial(const T* __restrict__ y,
                                                   const T* __restrict__ w, double s, int n,
                                                   double* __restrict__ part) {
  __shared__ double s_red[kWaves];
  double acc = 0.0;
  for (int i = blockIdx.x * kWG + threadIdx.x; i < n; i += gridDim.x * kWG) {
    const double d = (double)y[i] / s - (double)w[i];
    acc += d * d;
  }
  const double t = block_sum(acc, s_red);
  if (threadIdx.x == 0) part[blockIdx.x] = t;
}

__global__ __launch_bounds__(kWG) void sai_final(const double* __restrict__ part, int np,
                                                 double* __restrict__ out) {
  __shared__ double s_red[kWaves];
  const double t = sum_partials(part, np, s_red);
  if (threadIdx.x == 0) *out = t;
}

// ---------------------------------------------------------------------------
// Whole solve in one workgroup for small systems (n <= 1024, SELL rows of at
// most kSmallW slots in A, G and G^T): thread i owns row i and keeps its rows
// of A, G and G^T in registers for the whole solve, the three gathered
// vectors (p, r, t) live in LDS, every dot product is a workgroup reduction
// in a fixed order, and the iteration loop runs inside the kernel -- one
// launch per solve instead of three per iteration.  Same recurrences, exit
// rules and records as the multi-kernel solver.
// ---------------------------------------------------------------------------

constexpr int kSmallN = 1024;
constexpr int kSmallW = 8;
constexpr int kSmallWaves = kSmallN / 64;

template <typename T>
struct SmallArgs {
  const T* av;
  const int32_t* ac;
  const int16_t* ad;
  const int32_t* ao;
  const T* gv;
  const int32_t* gc;
  const int16_t* gd;
  const int32_t* go;
  const T* tv;
  const int32_t* tc;
  const int16_t* td;
  const int32_t* to;
  int n;
  double eps;
  const T* b;  // column blockIdx.x of b and x, row stride ld
  T* x;
  int ld;
  double rtol;
  int maxit;
  SolverState* st;  // one record per column
  double* hist_a;
  double* hist_b;
  int hist_len;
};

// Row i of a SELL matrix into registers (value 0 / column 0 for padding).
template <typename T>
__device__ __forceinline__ void small_row(const T* v, const int32_t* c, const int16_t* d,
                                          const int32_t* soff, int i, T (&val)[kSmallW],
                                          int (&col)[kSmallW]) {
  const int sl = i / kSlice, l = i - sl * kSlice;
  const int off = soff[sl], w = (soff[sl + 1] - off) / kSlice;
#pragma unroll
  for (int j = 0; j < kSmallW; ++j) {
    val[j] = T(0);
    col[j] = 0;
    if (j < w) {
      const int idx = off + j * kSlice + l;
      int cc;
      if (d) {
        const int raw = d[idx];
        cc = raw == kPad16 ? -1 : i + raw;
      } else {
        cc = c[idx];
      }
      if (cc >= 0) {
        val[j] = v[idx];
        col[j] = cc;
      }
    }
  }
}

template <typename T>
__device__ __forceinline__ T small_dot_row(const T (&val)[kSmallW], const int (&col)[kSmallW],
                                           const T* vec) {
  T acc = T(0);
#pragma unroll
  for (int j = 0; j < kSmallW; ++j) acc = fma(val[j], vec[col[j]], acc);
  return acc;
}

// Workgroup sums in a fixed order (wave sums, then the waves in order).  The
// reductions alternate between two LDS buffers (red[0..], red[2 kSmallWaves
// ..]), so no barrier is needed before a buffer is written: it was last read
// two reductions earlier, and every thread has passed the barrier of the
// reduction in between since.
__device__ __forceinline__ double small_sum(double v, double* red, int& buf) {
  double* rb = red + buf * 2 * kSmallWaves;
  buf ^= 1;
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) rb[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = rb[0];
#pragma unroll
  for (int q = 1; q < kSmallWaves; ++q) s += rb[q];
  return s;
}

template <typename T>
__global__ __launch_bounds__(kSmallN) void small_pcg(SmallArgs<T> a) {
  __shared__ T s_p[kSmallN], s_r[kSmallN], s_t[kSmallN];
  __shared__ double s_red[4 * kSmallWaves];  // two buffers (small_sum)
  int rbuf = 0;
  const int i = threadIdx.x;
  const bool live = i < a.n;
  T av[kSmallW], gv[kSmallW], tv[kSmallW];
  int ac[kSmallW], gc[kSmallW], tc[kSmallW];
  const int ri = live ? i : 0;
  small_row<T>(a.av, a.ac, a.ad, a.ao, ri, av, ac);
  small_row<T>(a.gv, a.gc, a.gd, a.go, ri, gv, gc);
  small_row<T>(a.tv, a.tc, a.td, a.to, ri, tv, tc);
  if (!live) {
#pragma unroll
    for (int j = 0; j < kSmallW; ++j) av[j] = gv[j] = tv[j] = T(0);
  }
  s_p[i] = T(0);
  s_t[i] = T(0);
  const int col = blockIdx.x;
  const T bi = live ? a.b[(size_t)i * a.ld + col] : T(0);
  T x = T(0), r = bi;
  const bool lead = i == 0;
  int kind = EX_NONE, kexit = 0;
  const double bb = small_sum((double)bi * (double)bi, s_red, rbuf);
  double rr = bb;
  if (!isfinite(bb)) kind = EX_NONFINITE_B;
  else if (bb == 0.0) kind = EX_BZERO;
  else if (a.maxit == 0) kind = EX_MAXIT0;
  const double bnorm = sqrt(bb);
  T z = T(0), p = T(0);
  double rho = 0.0;
  if (kind == EX_NONE) {
    // z_0 = G (G^T r_0) + eps r_0, rho_0
    s_r[i] = r;
    __syncthreads();
    s_t[i] = small_dot_row(tv, tc, s_r);
    __syncthreads();
    z = fma(T(a.eps), r, small_dot_row(gv, gc, s_t));
    rho = small_sum((double)r * (double)z, s_red, rbuf);
    if (!(rho > 0.0) || !isfinite(rho)) {
      kind = EX_BREAK_RHO;
      kexit = 1;
    }
    p = z;
  }
  for (int k = 1; kind == EX_NONE && k <= a.maxit; ++k) {
    s_p[i] = p;
    __syncthreads();
    const T q = small_dot_row(av, ac, s_p);
    const double sigma = small_sum((double)p * (double)q, s_red, rbuf);
    if (!(sigma > 0.0) || !isfinite(sigma)) {
      kind = EX_BREAK_SIGMA;
      kexit = k;
      break;
    }
    const double alpha = rho / sigma;
    if (lead && a.hist_a && k <= a.hist_len) a.hist_a[k - 1] = alpha;
    x = fma(T(alpha), p, x);
    r = fma(T(-alpha), q, r);
    rr = small_sum((double)r * (double)r, s_red, rbuf);
    const double rnorm = sqrt(rr);
    if (!isfinite(rnorm)) kind = EX_BREAK_RR;
    else if (rnorm <= a.rtol * bnorm) kind = EX_CONV;
    else if (k == a.maxit) kind = EX_MAXIT;
    if (kind != EX_NONE) {
      kexit = k;
      break;
    }
    s_r[i] = r;
    __syncthreads();
    s_t[i] = small_dot_row(tv, tc, s_r);
    __syncthreads();
    z = fma(T(a.eps), r, small_dot_row(gv, gc, s_t));
    const double rho_new = small_sum((double)r * (double)z, s_red, rbuf);
    if (!(rho_new > 0.0) || !isfinite(rho_new)) {
      kind = EX_BREAK_RHO;
      kexit = k + 1;
      break;
    }
    const double beta = rho_new / rho;
    if (lead && a.hist_b && k <= a.hist_len) a.hist_b[k - 1] = beta;
    rho = rho_new;
    p = fma(T(beta), p, z);
  }
  if (live) a.x[(size_t)i * a.ld + col] = x;
  if (lead) {
    SolverState* st = a.st + col;
    st->exit_kind = kind;
    st->exit_iter = kexit;
    st->bb = bb;
    st->rr = rr;
    st->done = 1;
  }
}

// ---------------------------------------------------------------------------
// Adjoint pattern gradient: g[k] = -lambda_row(k) * x_col(k).
// ---------------------------------------------------------------------------

// dL/dA in A's storage order, stored non-temporally (not read again here).
template <typename T>
__global__ __launch_bounds__(kWG) void csr_grad(const int32_t* __restrict__ rp,
                                                const int32_t* __restrict__ ci,
                                                const Tile* __restrict__ tiles, int ntiles,
                                                const T* __restrict__ lam, const T* __restrict__ x,
                                                T* __restrict__ g) {
  __shared__ int s_rp[kTileRows + 1];
  __shared__ int s_row[kLdsCap];  // local row of every entry of the tile
  const int tid = threadIdx.x;
  int t0, t1, step;
  tile_range(ntiles, t0, t1, step);
  for (int t = t0; t < t1; t += step) {
    const Tile d = tiles[t];
    if (d.kind == kTileLds) {
      // entries in storage order, one per thread and round; the row of each
      // comes from LDS markers written by the row's own thread
      const int r0 = d.a, nr = d.b - d.a;
      for (int i = tid; i <= nr; i += kWG) s_rp[i] = rp[r0 + i];
      __syncthreads();
      const int kb = s_rp[0], ke = s_rp[nr];
      if (tid < nr)
        for (int e = s_rp[tid]; e < s_rp[tid + 1]; ++e) s_row[e - kb] = tid;
      __syncthreads();
#pragma unroll 4
      for (int k = kb + tid; k < ke; k += kWG)
        __builtin_nontemporal_store(-(lam[r0 + s_row[k - kb]] * x[ci[k]]), g + k);
      __syncthreads();
    } else {
      const T l = lam[d.a];
#pragma unroll 4
      for (int k = d.b + tid; k < d.c; k += kWG) __builtin_nontemporal_store(-(l * x[ci[k]]), g + k);
    }
  }
}

// BSR: a tile of kBsrTileRows block rows owns one contiguous range of the
// gradient (9 entries per block, storage order).  Each thread forms the three
// entries of one block row r of one block (-lambda_{3I+r} times the block
// column's three x entries: one column load, three contiguous gathers) into
// LDS, then the workgroup streams the tile's range out with 16-byte
// non-temporal stores from the 128-byte line boundary below the range (each
// wavefront's store covers whole lines), the odd entries at either end
// alone.  The output is written once and never read here, and a gradient
// larger than the Infinity Cache would otherwise cycle through it.
// (Elasticity 64^3 x 3, 494 MB written, on the per-tile grid: 108 us; with
// the stores starting at the tile's first entry 116 us, with plain stores
// 188 us, with one scalar entry per thread and round, computing its block
// from the entry index, 162 us; a fill of the same size takes 80 us.)
constexpr int kGradMaxBlocks = 27;  // blocks per block row the LDS tile holds
template <typename T, int TR>
__global__ __launch_bounds__(kWG) void bsr3_grad(const int32_t* __restrict__ rp,
                                                 const int32_t* __restrict__ ci, int nbr,
                                                 int ntiles, const T* __restrict__ lam,
                                                 const T* __restrict__ x, T* __restrict__ g) {
  using V2 = T __attribute__((ext_vector_type(2)));
  constexpr int kMax = 9 * kGradMaxBlocks * TR + 128 / (int)sizeof(T);
  // (block, row) items per thread: all of a tile's loads are issued together
  constexpr int QU = (3 * kGradMaxBlocks * TR + kWG - 1) / kWG;
  __shared__ T s_g[kMax];
  int t0, t1, step;
  tile_range(ntiles, t0, t1, step);
  int rr[TR + 1];
  auto load_rows = [&](int t, int (&d)[TR + 1]) {
#pragma unroll
    for (int j = 0; j <= TR; ++j) d[j] = rp[min(t * TR + j, nbr)];
  };
  if (t0 < t1) load_rows(t0, rr);
  for (int t = t0; t < t1; t += step) {
    const int I0 = t * TR;
    const int b0 = rr[0], b1 = rr[TR];
    // (Entry indices fit int: the handle limits 9 nnzb below 2^31.)  The
    // stores start at the 128-byte line below the tile's first entry, so
    // that each wavefront's 16-byte-per-lane store covers whole lines.
    const int e0 = 9 * b0, e1 = 9 * b1, ea = e0 & ~(128 / (int)sizeof(T) - 1);
    // the host sends tiles with more blocks than the LDS holds to the
    // streaming kernel below
    const int nq = 3 * (b1 - b0);
    int kbv[QU], rv[QU], jv[QU];
    T lv[QU];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int q = (int)threadIdx.x + u * kWG;
      kbv[u] = b0 + q / 3;
      rv[u] = q - 3 * (q / 3);
      if (q < nq) {
        int li = 0;
#pragma unroll
        for (int j = 1; j < TR; ++j) li += kbv[u] >= rr[j] ? 1 : 0;
        lv[u] = lam[3 * (I0 + li) + rv[u]];
        jv[u] = ci[kbv[u]];
      }
    }
    // the next tile's row pointers stay in flight through this tile
    int rn[TR + 1];
    if (t + step < t1) load_rows(t + step, rn);
    T xv[QU][3];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      if ((int)threadIdx.x + u * kWG < nq) {
#pragma unroll
        for (int c = 0; c < 3; ++c) xv[u][c] = x[3 * jv[u] + c];
      }
    }
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      if ((int)threadIdx.x + u * kWG < nq) {
        T* d = s_g + (9 * kbv[u] + 3 * rv[u] - ea);
#pragma unroll
        for (int c = 0; c < 3; ++c) d[c] = -(lv[u] * xv[u][c]);
      }
    }
    __syncthreads();
    for (int e = ea + 2 * (int)threadIdx.x; e < e1; e += 2 * kWG) {
      if (e >= e0 && e + 1 < e1) {
        V2 v;
        v.x = s_g[e - ea];
        v.y = s_g[e - ea + 1];
        __builtin_nontemporal_store(v, (V2*)(g + e));
      } else {
        if (e >= e0 && e < e1) __builtin_nontemporal_store(s_g[e - ea], g + e);
        if (e + 1 >= e0 && e + 1 < e1) __builtin_nontemporal_store(s_g[e - ea + 1], g + e + 1);
      }
    }
    __syncthreads();
    if (t + step < t1) {
#pragma unroll
      for (int j = 0; j <= TR; ++j) rr[j] = rn[j];
    }
  }
}

// The same product for BSR tiles of any width, one scalar entry per thread
// and round (used when some block row holds more than kGradMaxBlocks blocks).
template <typename T>
__global__ __launch_bounds__(kWG) void bsr3_grad_wide(const int32_t* __restrict__ rp,
                                                      const int32_t* __restrict__ ci, int nbr,
                                                      int ntiles, const T* __restrict__ lam,
                                                      const T* __restrict__ x,
                                                      T* __restrict__ g) {
  constexpr int B = 4;
  int t0, t1, step;
  tile_range(ntiles, t0, t1, step);
  for (int t = t0; t < t1; t += step) {
    const int I0 = t * kBsrTileRows;
    int rr[kBsrTileRows + 1];
#pragma unroll
    for (int j = 0; j <= kBsrTileRows; ++j) rr[j] = rp[min(I0 + j, nbr)];
    const int e0 = 9 * rr[0], e1 = 9 * rr[kBsrTileRows];
    for (int e = e0 + (int)threadIdx.x; e < e1; e += B * kWG) {
      T prod[B];
#pragma unroll
      for (int u = 0; u < B; ++u) {
        const int eu = min(e + u * kWG, e1 - 1);  // in bounds; stored only if < e1
        const int kb = eu / 9;
        const int w = eu - kb * 9;
        int li = 0;
#pragma unroll
        for (int j = 1; j < kBsrTileRows; ++j) li += kb >= rr[j] ? 1 : 0;
        const int r = w / 3;
        const int c = w - 3 * r;
        prod[u] = lam[3 * (I0 + li) + r] * x[3 * ci[kb] + c];
      }
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (e + u * kWG < e1) __builtin_nontemporal_store(-prod[u], g + e + u * kWG);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------


#ifdef SLA_DEBUG
// Debug builds: SLA_DEBUG_SHRINK=k makes the gather check reject the last k
// columns too (valid input), so tests can reach the error path safely.
int debug_shrink() {
  const char* e = getenv("SLA_DEBUG_SHRINK");
  return e ? std::max(0, atoi(e)) : 0;
}
#endif

template <typename T>
void fill_matrix(StepArgs<T>& a, const sla_mat& m, const MatView& v, double* long_part,
                 int* long_cnt) {
  a.rp = v.rp;
  a.ci = v.ci;
  a.v = (const T*)v.v;
  a.tiles = v.tiles;
  a.ntiles = view_tiles(m, v);
  a.n = (int)m.n();
  if (v.sell) {
    a.sv = (const T*)v.sv;
    a.sc = v.sd ? nullptr : v.sc;
    a.sd = v.sd;
    a.soff = v.soff;
    a.nslices = v.nslices;
    a.sell_w = v.sell_w;
    a.so = v.so;
    a.sm = v.sm;
  }
  a.nbr = (int)m.nbr;
  a.long_part = long_part;
  a.long_cnt = long_cnt;
#ifdef SLA_DEBUG
  a.dbg_shrink = debug_shrink();
#endif
}

// The windowed slice-offset engine (sell_win_step): SLA_WIN=1 (default) for
// the A steps, 2 for every step of the iteration, 0 never (read once per
// solve).
int win_level() {
  const char* e = getenv("SLA_WIN");
  return e ? atoi(e) : 1;
}
bool win_applies(int mode, int level) {
  if (mode == M_PLAIN || level <= 0) return false;
  return level >= 2 || mode == M_A || mode == M_A1 || mode == M_AU;
}

template <typename T, int MODE>
hipError_t launch_step(const sla_mat& m, const StepArgs<T>& a, int grid, hipStream_t s,
                       bool nt, int win = 0) {
  if (m.bs == 1 && (a.sd || a.sc)) {
    // batch of slots per load round: the slice width rounded up to 4 or 8
    const bool wide = a.sell_w > 4;
    const dim3 g(grid), b(kWG);
    if (a.so && win_applies(MODE, win)) {
      if (nt && wide) hipLaunchKernelGGL((sell_win_step<T, MODE, true, 8>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((sell_win_step<T, MODE, true, 4>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((sell_win_step<T, MODE, false, 8>), g, b, 0, s, a);
      else hipLaunchKernelGGL((sell_win_step<T, MODE, false, 4>), g, b, 0, s, a);
    } else if (a.so) {
      if (nt && wide) hipLaunchKernelGGL((sell_step<T, MODE, true, true, 8, true>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((sell_step<T, MODE, true, true, 4, true>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((sell_step<T, MODE, false, true, 8, true>), g, b, 0, s, a);
      else hipLaunchKernelGGL((sell_step<T, MODE, false, true, 4, true>), g, b, 0, s, a);
    } else if (a.sd) {
      if (nt && wide) hipLaunchKernelGGL((sell_step<T, MODE, true, true, 8, false>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((sell_step<T, MODE, true, true, 4, false>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((sell_step<T, MODE, false, true, 8, false>), g, b, 0, s, a);
      else hipLaunchKernelGGL((sell_step<T, MODE, false, true, 4, false>), g, b, 0, s, a);
    } else {
      if (nt && wide) hipLaunchKernelGGL((sell_step<T, MODE, true, false, 8, false>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((sell_step<T, MODE, true, false, 4, false>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((sell_step<T, MODE, false, false, 8, false>), g, b, 0, s, a);
      else hipLaunchKernelGGL((sell_step<T, MODE, false, false, 4, false>), g, b, 0, s, a);
    }
  } else if (m.bs == 1) {
    if (nt) hipLaunchKernelGGL((csr_step<T, MODE, true>), dim3(grid), dim3(kWG), 0, s, a);
    else hipLaunchKernelGGL((csr_step<T, MODE, false>), dim3(grid), dim3(kWG), 0, s, a);
  } else if (a.sc || a.sd) {
    // block slots per load round: 3 for wide block rows, else 2 (fewer
    // registers, more waves in flight, and no partial last round on the
    // 27-slot rows of the 27-point block stencil and the 14-slot rows of its
    // block triangles; 2, 3, 4 and 6 measured there)
    const dim3 g(grid), b(kWG);
    const bool wide = a.sell_w > 16;
    if (a.sd) {
      if (nt && wide) hipLaunchKernelGGL((bsell_step<T, MODE, true, true, 3>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((bsell_step<T, MODE, true, true, 2>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((bsell_step<T, MODE, false, true, 3>), g, b, 0, s, a);
      else hipLaunchKernelGGL((bsell_step<T, MODE, false, true, 2>), g, b, 0, s, a);
    } else {
      if (nt && wide) hipLaunchKernelGGL((bsell_step<T, MODE, true, false, 3>), g, b, 0, s, a);
      else if (nt) hipLaunchKernelGGL((bsell_step<T, MODE, true, false, 2>), g, b, 0, s, a);
      else if (wide) hipLaunchKernelGGL((bsell_step<T, MODE, false, false, 3>), g, b, 0, s, a);
      else hipLaunchKernelGGL((bsell_step<T, MODE, false, false, 2>), g, b, 0, s, a);
    }
  } else {
    if (nt) hipLaunchKernelGGL((bsr3_step<T, MODE, true>), dim3(grid), dim3(kWG), 0, s, a);
    else hipLaunchKernelGGL((bsr3_step<T, MODE, false>), dim3(grid), dim3(kWG), 0, s, a);
  }
  return hipGetLastError();
}

// Infinity Cache (MALL) residency plan for one solve.  Every iteration
// streams A, G^T and G once; the MI355X's 256 MB MALL can hold one operator
// across iterations if the others do not allocate in it.  Keep A resident
// when its streams (values, columns, row pointers) fit the budget, else keep
// nothing resident; the remaining operators are streamed non-temporally.
// When everything fits, nothing is streamed non-temporally.
struct MallPlan {
  bool nt_a, nt_g, nt_t;  // A, G and G^T streams non-temporal
};
MallPlan mall_plan(const sla_mat& A, const sla_mat& G) {
  const size_t a = matrix_bytes(A), g = matrix_bytes(G);
  const size_t vecs = 8 * (size_t)A.n() * (A.dtype == SLA_F64 ? 8 : 4);
  const size_t budget = mall_budget();
  const char* pol = getenv("SLA_MALL_POLICY");
  if (pol) {
    if (!strcmp(pol, "none")) return {true, true, true};
    if (!strcmp(pol, "all")) return {false, false, false};
    if (!strcmp(pol, "A")) return {false, true, true};
    if (!strcmp(pol, "G")) return {true, false, false};
    if (!strcmp(pol, "AG")) return {false, false, true};
    if (!strcmp(pol, "AT")) return {false, true, false};
  }
  if (a + 2 * g + vecs <= budget) return {false, false, false};
  // G and G^T rather than A when their streams are the larger share and fit
  // the 256 MB Infinity Cache beside the six vectors an iteration touches
  // (16 MB left for partials, solver state and the rest)
  const size_t sa = stream_bytes(A, A.fwd), sg = stream_bytes(G, G.fwd) + stream_bytes(G, G.tr);
  const size_t live = 6 * (size_t)A.n() * (A.dtype == SLA_F64 ? 8 : 4);
  if (A.bs == 1 && sg >= sa && sg + live <= kMallBytes - ((size_t)16 << 20))
    return {true, false, false};
  if (a <= budget) return {false, true, true};
  return {true, true, true};
}

// ----- profiling -----
struct ProfClass {
  int64_t launches = 0;
  double ms = 0.0;
};
std::mutex g_prof_mu;
std::atomic<int> g_prof_mask{0};
std::atomic<int> g_prof_every{1};  // events on iterations k with k % every == 0
ProfClass g_prof[4];
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_spmv_pending;  // standalone SpMV timings

struct EventPair {
  hipEvent_t a, b;
  int cls;
  int k;
};

struct Recorder {
  int mask = 0;
  int every = 1;
  hipStream_t s = nullptr;
  std::vector<EventPair> ev;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  hipEvent_t get() {
    if (used == pool.size()) {
      hipEvent_t e = timing_event();
      if (!e) return nullptr;
      pool.push_back(e);
    }
    return pool[used++];
  }
  // Events around the launch of iteration k's class-cls kernel, if that
  // class is profiled and k is a multiple of the sampling stride.
  hipEvent_t begin(int cls, int k) {
    if (!(mask & (1 << cls)) || k % every != 0) return nullptr;
    hipEvent_t e = get();
    if (e) (void)hipEventRecord(e, s);
    return e;
  }
  void end(hipEvent_t a, int cls, int k) {
    if (!a) return;
    hipEvent_t e = get();
    if (!e) return;
    (void)hipEventRecord(e, s);
    ev.push_back({a, e, cls, k});
  }
  // Accumulate the launches that did work: every launch with k <= last_a for
  // the A / G^T classes, k < last_g (or the start-up k = 0) for the G class.
  void flush(int iters_a, int iters_g) {
    if (ev.empty()) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& p : ev) {
      bool real = false;
      if (p.cls == 0 || p.cls == 1) real = p.k <= iters_a;
      else if (p.cls == 2) real = p.k < iters_g || p.k == 0;
      else real = true;
      if (!real) continue;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
        g_prof[p.cls].launches += 1;
        g_prof[p.cls].ms += ms;
      }
    }
    ev.clear();
  }
  ~Recorder() {
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};

static_assert(4 * sizeof(SolverState) <= kPollBytes, "polling record too small");

struct Work {
  SolverState* st;
  int* lcnt;      // long-row tickets (zeroed with the state)
  double* lpart;  // long-row chunk partials
  double* psig;
  double* prr;
  double* prho;
  void* vec[7];  // P0 P1 R0 R1 q t z
  void* cbpart;  // column-block results of one product (kColBlocks n-vectors), or null
};

size_t partial_slots(const sla_mat& A) {
  return (size_t)kWideGrid * max_grid() + (size_t)long_rows_bound(A);
}

// Bytes from the start of the workspace that must be zero when a solve or
// a preconditioner apply starts: the state and the long-row tickets.
size_t zeroed_bytes(const sla_mat& A) {
  return align_up(sizeof(SolverState)) + align_up((size_t)long_rows_bound(A) * sizeof(int));
}

// Column-block results of one product: kColBlocks n-vectors, reserved for a
// handle whose solves run on column blocks (decided at creation, so the
// original handle and its ordered copy agree on the layout).
size_t colblock_bytes(const sla_mat& A) {
  if (A.bs != 1 || !((A.ord_want && A.cb_want) || A.cb)) return 0;
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  return (size_t)kColBlocks * align_up((size_t)A.n() * es);
}

// Workspace layout: state, long-row tickets, long-row partials, the three
// reduction partial arrays, seven n-vectors, column-block results.
Work carve(const sla_mat& A, void* work) {
  Work w;
  char* p = (char*)work;
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  const size_t n = (size_t)A.n();
  w.st = (SolverState*)p;
  p += align_up(sizeof(SolverState));
  w.lcnt = (int*)p;
  p += align_up((size_t)long_rows_bound(A) * sizeof(int));
  w.lpart = (double*)p;
  p += align_up((size_t)long_part_bound(A) * sizeof(double));
  const size_t ps = align_up(partial_slots(A) * sizeof(double));
  w.psig = (double*)p;
  p += ps;
  w.prr = (double*)p;
  p += ps;
  w.prho = (double*)p;
  p += ps;
  for (int i = 0; i < 7; ++i) {
    w.vec[i] = p;
    p += align_up(n * es);
  }
  w.cbpart = colblock_bytes(A) ? (void*)p : nullptr;
  return w;
}

// Status and record of a finished solve from its exit kind and iteration.
sla_status exit_status(const SolverState& fin, sla_solve_info* info, int* iters_out) {
  sla_status st = SLA_OK;
  int iters = 0, conv = 0;
  switch (fin.exit_kind) {
    case EX_CONV: st = SLA_OK; iters = fin.exit_iter; conv = 1; break;
    case EX_BZERO: st = SLA_OK; iters = 0; conv = 1; break;
    case EX_MAXIT: st = SLA_NOT_CONVERGED; iters = fin.exit_iter; break;
    case EX_MAXIT0: st = SLA_NOT_CONVERGED; iters = 0; break;
    case EX_BREAK_SIGMA: st = SLA_ERR_BREAKDOWN; iters = fin.exit_iter - 1; break;
    case EX_BREAK_RHO: st = SLA_ERR_BREAKDOWN; iters = fin.exit_iter - 1; break;
    case EX_BREAK_RR: st = SLA_ERR_BREAKDOWN; iters = fin.exit_iter; break;
    case EX_NONFINITE_B: st = SLA_ERR_NONFINITE; iters = 0; break;
    default:
      set_error("solver finished without an exit record");
      return SLA_ERR_HIP;
  }
  if (st == SLA_ERR_BREAKDOWN) set_error("PCG breakdown (p.Ap <= 0, r.z <= 0 or non-finite residual)");
  if (st == SLA_ERR_NONFINITE) set_error("right-hand side is not finite");
  if (info) {
    info->iterations = iters;
    info->converged = conv;
    info->bnorm = std::sqrt(fin.bb);
    info->rel_residual = fin.bb > 0 ? std::sqrt(fin.rr) / std::sqrt(fin.bb)
                                    : (fin.exit_kind == EX_BZERO ? 0.0 : 1.0);
    if (fin.exit_kind == EX_MAXIT0) info->rel_residual = 1.0;
  }
  if (iters_out) *iters_out = iters;
  return st;
}

template <typename T>
hipError_t launch_blk(const BlockArgs<T>& ba, int grid, hipStream_t s, bool nt) {
  if (nt) hipLaunchKernelGGL((csr_blk_step<T, true>), dim3(grid), dim3(kWG), 0, s, ba);
  else hipLaunchKernelGGL((csr_blk_step<T, false>), dim3(grid), dim3(kWG), 0, s, ba);
  return hipGetLastError();
}

// Fused iteration (p and r formed inside the products' gathers) when A is a
// CSR matrix in the SELL-64 layout (short, even, banded rows: its gathers
// have locality and its one gather per slot costs little next to the value
// stream).  Otherwise separate streaming passes keep every product at one
// gather per nonzero: random gathers (irregular CSR) cost the same whether
// or not p and r are formed in them, and a 3x3 block slot streams 9 values
// per gathered entry, so the fused form's second gather and its three extra
// stores cost the BSR products more than the two vector passes
// (elasticity 64^3 x 3: 296 against 270 us per iteration).
// SLA_FUSION=fused|unfused overrides the choice.
bool use_fused(const sla_mat& A) {
  if (const char* e = getenv("SLA_FUSION")) {
    if (!strcmp(e, "fused")) return true;
    if (!strcmp(e, "unfused")) return false;
  }
  return A.bs == 1 && A.fwd.sell;
}

template <typename T>
sla_status pcg_impl(const sla_mat& A, const sla_mat& G, double eps, const T* b, T* x, double rtol,
                    int maxit, void* work, hipStream_t s, sla_solve_info* info, double* hist_a,
                    double* hist_b, int hist_len, PollSlot* slot, bool quiet) {
  const int n = (int)A.n();
  Work w = carve(A, work);
  T *P[2] = {(T*)w.vec[0], (T*)w.vec[1]}, *R[2] = {(T*)w.vec[2], (T*)w.vec[3]};
  T *q = (T*)w.vec[4], *t = (T*)w.vec[5], *z = (T*)w.vec[6];
  // the three products run one after another on s, so they share one
  // long-row scratch (every ticket is back at 0 when a product ends)
  const LongScratch lsA{w.lpart, w.lcnt}, lsG = lsA, lsT = lsA;
  const int ntA = view_tiles(A, A.fwd), ntG = view_tiles(G, G.fwd), ntT = view_tiles(G, G.tr);
  const bool fused = use_fused(A);
  // Fused form: every kernel sums the previous one's per-workgroup partials
  // in its prologue, so all run on the resident-capacity grid.  Separate
  // form on BSR: the bare products read no partials and run one work item
  // per workgroup (up to kWideGrid times that grid; the dispatcher then
  // balances the last round; elasticity 64^3 x 3: A product 101 -> 94 us),
  // while the vector passes, which sum the products' partials, keep the
  // resident grid.  CSR keeps the resident grid throughout: on the
  // power-law system the gain was 2%, and the grid sets the partial sums'
  // rounding order, which moves that ill-conditioned system's stopping
  // iteration by a few percent.
  const bool wide = !fused && A.bs > 1;
  const int grid = wide ? wide_grid(std::max(ntA, std::max(ntG, ntT)))
                        : step_grid(std::max(ntA, std::max(ntG, ntT)));
  const int gridV = wide ? std::min(grid, max_grid()) : grid;
  // separate form on column blocks (random-graph CSR on its ordering): each
  // product is a column-block pass and a reduction whose epilogue and
  // partials are the step's own
  const bool blk = !fused && A.cb && G.cb && G.cb->has_tr && w.cbpart;
  const int npA = grid + (blk ? 0 : A.fwd.nlong_rows), npG = grid + (blk ? 0 : G.fwd.nlong_rows),
            npT = grid + (blk ? 0 : G.tr.nlong_rows);

  SLA_HIP(hipMemsetAsync(w.st, 0, zeroed_bytes(A), s));
  const MallPlan plan = mall_plan(A, G);
  const int win = win_level();

  StepArgs<T> aA{}, aT{}, aG{};
  fill_matrix(aA, A, A.fwd, lsA.part, lsA.cnt);
  fill_matrix(aT, G, G.tr, lsT.part, lsT.cnt);
  fill_matrix(aG, G, G.fwd, lsG.part, lsG.cnt);
  for (StepArgs<T>* a : {&aA, &aT, &aG}) {
    a->st = w.st;
    a->maxit = maxit;
    a->rtol = rtol;
    a->eps = eps;
    a->hist_a = hist_a;
    a->hist_b = hist_b;
    a->hist_len = hist_len;
  }
  // A step: pin = rho partials (from G step), pout = sigma partials
  aA.pin = w.prho;
  aA.npin = npG;
  aA.pout = w.psig;
  aA.in0 = z;
  aA.y = q;
  aA.xv = x;
  // G^T step: pin = sigma partials, pout = rr partials
  aT.pin = w.psig;
  aT.npin = npA;
  aT.pout = w.prr;
  aT.in1 = q;
  aT.y = t;
  aT.xv = x;
  // G step: pin = rr partials, pout = rho partials
  aG.pin = w.prr;
  aG.npin = npT;
  aG.pout = w.prho;
  aG.in0 = t;
  aG.y = z;

  BlockArgs<T> bA{}, bT{}, bG{};
  int gridB = kColBlocks;
  const size_t cbstride = align_up((size_t)n * sizeof(T)) / sizeof(T);
  if (blk) {
    auto set_blocks = [&](BlockArgs<T>& ba, const sla_mat& m, const ColBlockSet& cs,
                          const T* in) {
      for (int c = 0; c < kColBlocks; ++c) {
        StepArgs<T>& a = ba.blk[c];
        fill_matrix(a, m, cs.blk[c], w.lpart + cs.lpart_off[c], w.lcnt + cs.lrow_off[c]);
        a.in0 = in;
#ifdef SLA_DEBUG
        a.st = w.st;  // the gather check's count (the pass itself reads no state)
#endif
        a.y = (T*)w.cbpart + (size_t)c * cbstride;
        gridB = std::max(gridB, kColBlocks * std::min(a.ntiles, kWideGrid * max_grid() / kColBlocks));
      }
      ba.st = w.st;
    };
    set_blocks(bA, A, A.cb->fwd, nullptr);
    set_blocks(bT, G, G.cb->tr, nullptr);
    set_blocks(bG, G, G.cb->fwd, t);
  }

  // unfused iteration: vector passes (p/x update, r update) around
  // single-gather products
  StepArgs<T> aV = aA, aR = aT;
  aV.in0 = z;
  aV.xv = x;
  aV.pin = w.prho;
  aV.npin = npG;
  aR.in1 = q;
  aR.pin = w.psig;
  aR.npin = npA;
  aR.pout = w.prr;
  if (!fused) {
    aT.pout = nullptr;  // t = G^T r carries no reduction when unfused
    aA.pin = nullptr;
    aA.npin = 0;
  }

  Recorder rec;
  rec.mask = quiet ? 0 : g_prof_mask.load();
  rec.every = g_prof_every.load();
  rec.s = s;

  // start-up: r_0 = b, x = 0, t = G^T b, ||b||^2; z_0 = G t + eps r_0, rho_0
  aT.k = 0;
  aT.in0 = b;
  aT.own = R[0];
  aT.pout = w.prr;
  hipEvent_t e0 = rec.begin(1, 0);
  if (blk) {
    for (auto& a : bT.blk) a.in0 = b;
    SLA_HIP(launch_blk(bT, gridB, s, plan.nt_t));
    hipLaunchKernelGGL((blk_reduce<T, M_GT0>), dim3(grid), dim3(kWG), 0, s, aT,
                       (const T*)w.cbpart, cbstride);
    SLA_HIP(hipGetLastError());
  } else {
    SLA_HIP((launch_step<T, M_GT0>(G, aT, grid, s, plan.nt_t, win)));
  }
  rec.end(e0, 1, 0);
  if (!fused) aT.pout = nullptr;
  aG.k = 0;
  aG.rv = R[0];
  e0 = rec.begin(2, 0);
  if (blk) {
    SLA_HIP(launch_blk(bG, gridB, s, plan.nt_g));
    hipLaunchKernelGGL((blk_reduce<T, M_G0>), dim3(grid), dim3(kWG), 0, s, aG,
                       (const T*)w.cbpart, cbstride);
    SLA_HIP(hipGetLastError());
  } else {
    SLA_HIP((launch_step<T, M_G0>(G, aG, grid, s, plan.nt_g, win)));
  }
  rec.end(e0, 2, 0);

  // Batches of iterations, at most two queued; the G step of a batch's last
  // iteration fills that batch's host-mapped polling record.
  SolverState* hst = (SolverState*)slot->host;
  SolverState* dpoll = (SolverState*)slot->dev;
  int pend[3], pend_k[3];
  int npend = 0, pfirst = 0;
  int next_slot = 0;
  BatchPlanner plan_b(batch_iters(iteration_estimate_us(A, G, (int)sizeof(T), 1, fused ? 3 : 5)),
                      rtol);
  int k = 1;
  bool finished = false;
  while (!finished) {
    const int want = k <= maxit ? plan_b.next(k) : 0;
    if (k <= maxit && npend < 2 && (want > 0 || npend == 0)) {
      const int kend = std::min(maxit, k + std::max(want, plan_b.restart()) - 1);
      const int ps = next_slot;
      next_slot = (next_slot + 1) % 3;
      ((volatile SolverState*)&hst[ps])->exit_iter = -1;
      for (int kk = k; kk <= kend; ++kk) {
        if (fused) {
          aA.k = kk;
          aA.in1 = P[(kk - 1) & 1];
          aA.own = P[kk & 1];
          hipEvent_t ea = rec.begin(0, kk);
          if (kk == 1) SLA_HIP((launch_step<T, M_A1>(A, aA, grid, s, plan.nt_a, win)));
          else SLA_HIP((launch_step<T, M_A>(A, aA, grid, s, plan.nt_a, win)));
          rec.end(ea, 0, kk);
          aT.k = kk;
          aT.in0 = R[(kk - 1) & 1];
          aT.own = R[kk & 1];
          hipEvent_t et = rec.begin(1, kk);
          SLA_HIP((launch_step<T, M_GT>(G, aT, grid, s, plan.nt_t, win)));
          rec.end(et, 1, kk);
        } else {
          // p and x update, q = A p, r update, t = G^T r: single gathers
          aV.k = kk;
          aV.in1 = P[(kk - 1) & 1];
          aV.own = P[kk & 1];
          if (kk == 1)
            hipLaunchKernelGGL((vec_p_update<T, M_A1>), dim3(gridV), dim3(kWG), 0, s, aV);
          else
            hipLaunchKernelGGL((vec_p_update<T, M_A>), dim3(gridV), dim3(kWG), 0, s, aV);
          SLA_HIP(hipGetLastError());
          aA.k = kk;
          aA.in0 = P[kk & 1];
          hipEvent_t ea = rec.begin(0, kk);
          if (blk) {
            for (auto& a : bA.blk) a.in0 = P[kk & 1];
            SLA_HIP(launch_blk(bA, gridB, s, plan.nt_a));
            hipLaunchKernelGGL((blk_reduce<T, M_AU>), dim3(grid), dim3(kWG), 0, s, aA,
                               (const T*)w.cbpart, cbstride);
            SLA_HIP(hipGetLastError());
          } else {
            SLA_HIP((launch_step<T, M_AU>(A, aA, grid, s, plan.nt_a, win)));
          }
          rec.end(ea, 0, kk);
          aR.k = kk;
          aR.in0 = R[(kk - 1) & 1];
          aR.own = R[kk & 1];
          hipLaunchKernelGGL((vec_r_update<T>), dim3(gridV), dim3(kWG), 0, s, aR);
          SLA_HIP(hipGetLastError());
          aT.k = kk;
          aT.in0 = R[kk & 1];
          hipEvent_t et = rec.begin(1, kk);
          if (blk) {
            for (auto& a : bT.blk) a.in0 = R[kk & 1];
            SLA_HIP(launch_blk(bT, gridB, s, plan.nt_t));
            hipLaunchKernelGGL((blk_reduce<T, M_GTU>), dim3(grid), dim3(kWG), 0, s, aT,
                               (const T*)w.cbpart, cbstride);
            SLA_HIP(hipGetLastError());
          } else {
            SLA_HIP((launch_step<T, M_GTU>(G, aT, grid, s, plan.nt_t, win)));
          }
          rec.end(et, 1, kk);
          aG.npin = gridV;  // rr partials now come from vec_r_update
        }
        aG.k = kk;
        aG.rv = R[kk & 1];
        aG.poll = kk == kend ? dpoll + ps : nullptr;
        hipEvent_t eg = rec.begin(2, kk);
        if (blk) {
          SLA_HIP(launch_blk(bG, gridB, s, plan.nt_g));
          hipLaunchKernelGGL((blk_reduce<T, M_G>), dim3(grid), dim3(kWG), 0, s, aG,
                             (const T*)w.cbpart, cbstride);
          SLA_HIP(hipGetLastError());
        } else {
          SLA_HIP((launch_step<T, M_G>(G, aG, grid, s, plan.nt_g, win)));
        }
        rec.end(eg, 2, kk);
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
      SLA_HIP(wait_poll(&hst[ps], kb, s, &w.st->done, &r));
      if (r.done) finished = true;
      else plan_b.observe(r.exit_iter, r.rr, r.bb);
      continue;
    }
    finished = true;  // k > maxit and nothing queued
  }
  // batches still queued return at once; the stream synchronization below
  // waits for them
  hipLaunchKernelGGL(finalize_x<T>, dim3(std::max(1, std::min((n + kWG - 1) / kWG, 4096))),
                     dim3(kWG), 0, s, (const SolverState*)w.st, x, (const T*)P[0],
                     (const T*)P[1], n);
  SLA_HIP(hipGetLastError());
  SolverState* hs = &hst[3];
  SLA_HIP(hipMemcpyAsync(hs, w.st, sizeof(SolverState), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  const SolverState fin = *hs;
#ifdef SLA_DEBUG
  if (fin.dbg_bad) {
    char msg[96];
    snprintf(msg, sizeof msg, "debug build: %d gathered column indices out of range", fin.dbg_bad);
    set_error(msg);
    return SLA_ERR_INVALID_ARG;
  }
#endif

  int iters = 0;
  const sla_status st = exit_status(fin, info, &iters);
  if (st == SLA_ERR_HIP) return st;
  // profile: A / G^T launches of iterations 1..iters did work; G launches of
  // iterations < the exit iteration did work (the exit one returns early)
  rec.flush(std::max(iters, fin.exit_kind == EX_BREAK_SIGMA ? fin.exit_iter : iters),
            fin.exit_iter);
  return st;
}


// The one-workgroup solver applies when every operator has the SELL layout
// with at most kSmallW slots per row and n <= kSmallN (SLA_SMALL=0 turns it
// off).
bool small_ok(const sla_mat& A, const sla_mat& G) {
  if (const char* e = getenv("SLA_SMALL"))
    if (e[0] == '0') return false;
  if (A.bs != 1 || A.n() > kSmallN) return false;
  for (const MatView* v : {&A.fwd, &G.fwd, &G.tr})
    if (!v->sell || v->sell_w > kSmallW) return false;
  return true;
}

template <typename T>
sla_status small_impl(const sla_mat& A, const sla_mat& G, double eps, const T* b, T* x,
                      double rtol, int maxit, void* work, hipStream_t s, sla_solve_info* info,
                      double* hist_a, double* hist_b, int hist_len, PollSlot* slot) {
  Work w = carve(A, work);
  SmallArgs<T> a{};
  auto set = [](const MatView& v, const T*& val, const int32_t*& col, const int16_t*& d,
                const int32_t*& off) {
    val = (const T*)v.sv;
    col = v.sd ? nullptr : v.sc;
    d = v.sd;
    off = v.soff;
  };
  set(A.fwd, a.av, a.ac, a.ad, a.ao);
  set(G.fwd, a.gv, a.gc, a.gd, a.go);
  set(G.tr, a.tv, a.tc, a.td, a.to);
  a.n = (int)A.n();
  a.eps = eps;
  a.b = b;
  a.x = x;
  a.ld = 1;
  a.rtol = rtol;
  a.maxit = maxit;
  a.st = w.st;
  a.hist_a = hist_a;
  a.hist_b = hist_b;
  a.hist_len = hist_len;
  hipLaunchKernelGGL((small_pcg<T>), dim3(1), dim3(kSmallN), 0, s, a);
  SLA_HIP(hipGetLastError());
  SolverState* hs = (SolverState*)slot->host + 3;
  SLA_HIP(hipMemcpyAsync(hs, w.st, sizeof(SolverState), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  const SolverState fin = *hs;
  return exit_status(fin, info, nullptr);
}
}  // namespace

// ---------------------------------------------------------------------------
// Internal API used by api.cpp
// ---------------------------------------------------------------------------

LongScratch long_scratch_of(const sla_mat& m, bool transpose) {
  // slots of the handle's owned[] array (see api.cpp)
  const int base = transpose ? 4 : 2;
  return LongScratch{(double*)m.owned[base], (int*)m.owned[base + 1]};
}

// A row longer than kLdsCap holds more than kLdsCap of the nnz entries, and
// splits into at most len / kLongChunk + 1 chunks.
int64_t long_rows_bound(const sla_mat& A) {
  return std::max<int64_t>(std::max(A.fwd.nlong_rows, A.tr.nlong_rows), A.nnz() / kLdsCap + 1);
}
int64_t long_part_bound(const sla_mat& A) {
  return std::max<int64_t>(std::max(A.fwd.n_long_part, A.tr.n_long_part),
                           A.nnz() / kLongChunk + long_rows_bound(A) + 1);
}

size_t workspace_base(const sla_mat& A) {
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  return zeroed_bytes(A) + align_up((size_t)long_part_bound(A) * sizeof(double)) +
         3 * align_up(partial_slots(A) * sizeof(double)) + 7 * align_up((size_t)A.n() * es) +
         colblock_bytes(A);
}

size_t workspace_bytes(const sla_mat& A) {
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  return workspace_base(A) + (A.ord_want ? 2 * align_up((size_t)A.n() * es) : 0);
}

sla_status spmv(const sla_mat& A, bool transpose, const void* x, void* y, hipStream_t s,
                const LongScratch* scratch) {
  const MatView& v = transpose ? A.tr : A.fwd;
  if (A.n() == 0) return SLA_OK;
  hipEvent_t ea = nullptr, eb = nullptr;
  const bool prof = (g_prof_mask.load() & (1 << 3)) != 0;
  if (prof) {
    ea = timing_event();
    eb = timing_event();
    if (!ea || !eb) {
      set_error("hipEventCreate failed");
      return SLA_ERR_HIP;
    }
    SLA_HIP(hipEventRecord(ea, s));
  }
  const LongScratch ls = scratch ? *scratch : long_scratch_of(A, transpose);
  const bool nt = matrix_bytes(A) > mall_budget();
  // the plain product reads no partials: BSR takes one work item per
  // workgroup, as in the separate iteration form
  auto grid_of = [&](int ntiles) { return A.bs > 1 ? wide_grid(ntiles) : step_grid(ntiles); };
  if (A.dtype == SLA_F64) {
    StepArgs<double> a{};
    fill_matrix(a, A, v, ls.part, ls.cnt);
    a.in0 = (const double*)x;
    a.y = (double*)y;
    SLA_HIP((launch_step<double, M_PLAIN>(A, a, grid_of(a.ntiles), s, nt)));
  } else {
    StepArgs<float> a{};
    fill_matrix(a, A, v, ls.part, ls.cnt);
    a.in0 = (const float*)x;
    a.y = (float*)y;
    SLA_HIP((launch_step<float, M_PLAIN>(A, a, grid_of(a.ntiles), s, nt)));
  }
  if (prof) {
    SLA_HIP(hipEventRecord(eb, s));
    // read back later (prof_get / prof_reset), so that timed calls queue
    // back to back as they do inside a solve
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_spmv_pending.push_back({ea, eb});
  }
  return SLA_OK;
}

// z = G (G^T r) + eps r with t = G^T r in caller-provided memory; both
// products use the long-row scratch ls (tickets at zero).
static sla_status precond_into(const sla_mat& G, double eps, const void* r, void* t, void* z,
                               const LongScratch& ls, hipStream_t s) {
  sla_status st = spmv(G, true, r, t, s, &ls);
  if (st != SLA_OK) return st;
  const bool nt = matrix_bytes(G) > mall_budget();
  if (G.dtype == SLA_F64) {
    StepArgs<double> a{};
    fill_matrix(a, G, G.fwd, ls.part, ls.cnt);
    a.in0 = (const double*)t;
    a.rv = (const double*)r;
    a.y = (double*)z;
    a.eps = eps;
    SLA_HIP((launch_step<double, M_GZ>(G, a, step_grid(a.ntiles), s, nt)));
  } else {
    StepArgs<float> a{};
    fill_matrix(a, G, G.fwd, ls.part, ls.cnt);
    a.in0 = (const float*)t;
    a.rv = (const float*)r;
    a.y = (float*)z;
    a.eps = eps;
    SLA_HIP((launch_step<float, M_GZ>(G, a, step_grid(a.ntiles), s, nt)));
  }
  return SLA_OK;
}

sla_status precond_apply(const sla_mat& G, double eps, const void* r, void* z, void* work,
                         size_t, hipStream_t s) {
  if (G.n() == 0) return SLA_OK;
  Work w = carve(G, work);
  SLA_HIP(hipMemsetAsync(w.st, 0, zeroed_bytes(G), s));
  return precond_into(G, eps, r, w.vec[5], z, LongScratch{w.lpart, w.lcnt}, s);
}

sla_status sai_loss(const sla_mat& A, const sla_mat& G, double eps, const void* probes,
                    int32_t nprobe, double scale, void* work, double* out, hipStream_t s) {
  const int64_t n = A.n();
  if (nprobe == 0) return SLA_OK;
  // the workspace holds max(workspace_bytes(A), workspace_bytes(G)): carve
  // it for the operator with more entries, whose long-row bounds cover both
  const sla_mat& big = A.nnz() >= G.nnz() ? A : G;
  Work w = carve(big, work);
  SLA_HIP(hipMemsetAsync(w.st, 0, zeroed_bytes(big), s));
  const LongScratch ls{w.lpart, w.lcnt};
  const size_t es = A.dtype == SLA_F64 ? 8 : 4;
  const int grid = (int)std::min<int64_t>(max_grid(), std::max<int64_t>(1, (n + kWG - 1) / kWG));
  for (int32_t j = 0; j < nprobe; ++j) {
    const void* wj = (const char*)probes + (size_t)j * (size_t)n * es;
    if (n > 0) {
      sla_status st = precond_into(G, eps, wj, w.vec[5], w.vec[0], ls, s);
      if (st != SLA_OK) return st;
      st = spmv(A, false, w.vec[0], w.vec[1], s, &ls);
      if (st != SLA_OK) return st;
    }
    if (A.dtype == SLA_F64)
      sai_partial<double><<<grid, kWG, 0, s>>>((const double*)w.vec[1], (const double*)wj,
                                               scale, (int)n, w.psig);
    else
      sai_partial<float><<<grid, kWG, 0, s>>>((const float*)w.vec[1], (const float*)wj, scale,
                                              (int)n, w.psig);
    SLA_HIP(hipGetLastError());
    sai_final<<<1, kWG, 0, s>>>(w.psig, grid, out + j);
    SLA_HIP(hipGetLastError());
  }
  return SLA_OK;
}

sla_status pcg_solve(const sla_mat& A, const sla_mat& G, double eps, const void* b, void* x,
                     double rtol, int32_t maxit, void* work, size_t, hipStream_t s,
                     sla_solve_info* info, double* hist_a, double* hist_b, int32_t hist_len,
                     PollSlot* slot, bool quiet) {
  if (A.n() == 0) {
    if (info) *info = sla_solve_info{0, 1, 0.0, 0.0};
    return SLA_OK;
  }
  PollLease lease;
  if (!slot) {
    sla_status st = poll_acquire(&lease.p);
    if (st != SLA_OK) return st;
    slot = lease.p;
  }
  if (small_ok(A, G)) {
    if (A.dtype == SLA_F64)
      return small_impl<double>(A, G, eps, (const double*)b, (double*)x, rtol, maxit, work, s,
                                info, hist_a, hist_b, hist_len, slot);
    return small_impl<float>(A, G, eps, (const float*)b, (float*)x, rtol, maxit, work, s, info,
                             hist_a, hist_b, hist_len, slot);
  }
  if (A.dtype == SLA_F64)
    return pcg_impl<double>(A, G, eps, (const double*)b, (double*)x, rtol, maxit, work, s, info,
                            hist_a, hist_b, hist_len, slot, quiet);
  return pcg_impl<float>(A, G, eps, (const float*)b, (float*)x, rtol, maxit, work, s, info,
                         hist_a, hist_b, hist_len, slot, quiet);
}

bool small_applies(const sla_mat& A, const sla_mat& G) { return small_ok(A, G); }

size_t small_states_bytes(int k) { return align_up((size_t)k * sizeof(SolverState)); }

// k independent small solves (columns of n x k row-major b and x), one
// workgroup each, all in one launch.
sla_status small_solve_batch(const sla_mat& A, const sla_mat& G, double eps, const void* b,
                             void* x, int k, double rtol, int maxit, void* states,
                             hipStream_t s, sla_solve_info* info, sla_status* cst) {
  auto launch = [&](auto tag) -> hipError_t {
    using T = decltype(tag);
    SmallArgs<T> a{};
    auto set = [](const MatView& v, const T*& val, const int32_t*& col, const int16_t*& d,
                  const int32_t*& off) {
      val = (const T*)v.sv;
      col = v.sd ? nullptr : v.sc;
      d = v.sd;
      off = v.soff;
    };
    set(A.fwd, a.av, a.ac, a.ad, a.ao);
    set(G.fwd, a.gv, a.gc, a.gd, a.go);
    set(G.tr, a.tv, a.tc, a.td, a.to);
    a.n = (int)A.n();
    a.eps = eps;
    a.b = (const T*)b;
    a.x = (T*)x;
    a.ld = k;
    a.rtol = rtol;
    a.maxit = maxit;
    a.st = (SolverState*)states;
    hipLaunchKernelGGL((small_pcg<T>), dim3(k), dim3(kSmallN), 0, s, a);
    return hipGetLastError();
  };
  if (A.dtype == SLA_F64) SLA_HIP(launch(double(0)));
  else SLA_HIP(launch(float(0)));
  std::vector<SolverState> fin((size_t)k);
  SLA_HIP(hipMemcpyAsync(fin.data(), states, (size_t)k * sizeof(SolverState),
                         hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  sla_status worst = SLA_OK;
  for (int c = 0; c < k; ++c) {
    const sla_status st = exit_status(fin[c], info ? info + c : nullptr, nullptr);
    if (st == SLA_ERR_HIP) return st;
    if (cst) cst[c] = st;
    if (st < 0 && worst >= 0) worst = st;
    else if (st == SLA_NOT_CONVERGED && worst == SLA_OK) worst = st;
  }
  return worst;
}

sla_status pattern_grad(const sla_mat& A, const void* lam, const void* x, void* grad,
                        hipStream_t s) {
  if (A.nnzb == 0) return SLA_OK;
  // an elementwise product over the stored entries: no partials, so one
  // work item per workgroup where the tiles allow it
  if (A.bs == 1) {
    const int grid = wide_grid(A.fwd.ntiles);
    if (A.dtype == SLA_F64)
      hipLaunchKernelGGL(csr_grad<double>, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci,
                         A.fwd.tiles, A.fwd.ntiles, (const double*)lam, (const double*)x,
                         (double*)grad);
    else
      hipLaunchKernelGGL(csr_grad<float>, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci,
                         A.fwd.tiles, A.fwd.ntiles, (const float*)lam, (const float*)x,
                         (float*)grad);
  } else {
    // the LDS-staged kernel holds tiles whose block rows have at most
    // kGradMaxBlocks blocks
    const bool staged = A.fwd.max_row >= 0 && A.fwd.max_row <= kGradMaxBlocks;
    const int nt = (int)((A.nbr + kBsrTileRows - 1) / kBsrTileRows);
    const int grid = wide_grid(nt);
    if (A.dtype == SLA_F64) {
      auto kern = staged ? bsr3_grad<double, kBsrTileRows> : bsr3_grad_wide<double>;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci, (int)A.nbr, nt,
                         (const double*)lam, (const double*)x, (double*)grad);
    } else {
      auto kern = staged ? bsr3_grad<float, kBsrTileRows> : bsr3_grad_wide<float>;
      hipLaunchKernelGGL(kern, dim3(grid), dim3(kWG), 0, s, A.fwd.rp, A.fwd.ci, (int)A.nbr, nt,
                         (const float*)lam, (const float*)x, (float*)grad);
    }
  }
  SLA_HIP(hipGetLastError());
  return SLA_OK;
}

void prof_enable(int mask) { g_prof_mask.store(mask & 15); }
void prof_every(int every) { g_prof_every.store(every < 1 ? 1 : every); }
// Fold the pending standalone-SpMV event pairs into their class (waits for
// them); caller holds g_prof_mu.
void flush_spmv_pending() {
  for (auto& pr : g_spmv_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(pr.second) == hipSuccess &&
        hipEventElapsedTime(&ms, pr.first, pr.second) == hipSuccess) {
      g_prof[3].launches += 1;
      g_prof[3].ms += ms;
    }
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  g_spmv_pending.clear();
}
void prof_get(int cls, int64_t* launches, double* ms) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  flush_spmv_pending();
  if (launches) *launches = g_prof[cls].launches;
  if (ms) *ms = g_prof[cls].ms;
}
void prof_reset() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  flush_spmv_pending();
  for (auto& p : g_prof) p = ProfClass{};
}

int occupancy_grid(int cus) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, csr_step<double, M_A, true>, kWG,
                                                   0) !=
          hipSuccess ||
      per_cu <= 0)
    per_cu = 4;
  int g = cus * per_cu;
  g &= ~7;
  return std::max(8, g);
}

}  // namespace sla
