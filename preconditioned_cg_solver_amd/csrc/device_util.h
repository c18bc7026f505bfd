// Device helpers shared by the PCG kernels (single and several right-hand
// sides): deterministic workgroup reductions, the XCD-aware assignment of
// work items to workgroups, streaming loads of matrix data and the staging
// of CSR row tiles.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace sla {

// The host-mapped polling record of a batch of iterations, written by the
// lead thread of the batch's last G step once its prologue has decided: system-scope
// vector stores, the iteration index last (release), which the host waits
// for.  Only this kernel writes the record after the host cleared it.
__device__ __forceinline__ void post_poll(SolverState* p, int done, int k, double rr,
                                          double bb) {
  __hip_atomic_store(&p->done, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(&p->rr, rr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(&p->bb, bb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(&p->exit_iter, k, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// Reductions (deterministic: fixed association order)
// ---------------------------------------------------------------------------

// A double moved between lanes by a DPP pattern (both 32-bit halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, 0xf, 0xf, false);
  return __hiloint2double(hi, lo);
}

// Sum of the two 16-lane rows of each 32-lane half (even row + odd row, in
// that order in every lane) and of the two 32-lane halves (lower + upper):
// the gfx950 lane swaps, with the value as both operands, return the even
// and the odd row (the lower and the upper half) in every lane.
__device__ __forceinline__ double rows_pair_sum(double v) {
  const unsigned lo = (unsigned)__double2loint(v), hi = (unsigned)__double2hiint(v);
  const auto l = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}
__device__ __forceinline__ double halves_sum(double v) {
  const unsigned lo = (unsigned)__double2loint(v), hi = (unsigned)__double2hiint(v);
  const auto l = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto h = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return __hiloint2double((int)h[0], (int)l[0]) + __hiloint2double((int)h[1], (int)l[1]);
}

// Sum over the 64 lanes, the same value in every lane: within each 16-lane
// row by DPP moves (lane pairs l ^ 1, then l ^ 2, then the mirrored half of
// the 8-lane group, then the mirrored half of the row; each adds a lane pair
// in both orders, which IEEE addition makes identical), then across rows
// and halves by the lane swaps.  No LDS round trip.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  v = rows_pair_sum(v);
  return halves_sum(v);
}

// Sum over the workgroup; every thread gets lane 0 / wave order's value.
__device__ __forceinline__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int q = 1; q < kWaves; ++q) s += red[q];
  return s;
}

// This thread's share of a sum of partials, before the workgroup sum.
__device__ __forceinline__ double partial_share(const double* __restrict__ p, int np) {
  // each thread adds p[tid], p[tid + kWG], ... in index order; the loads of
  // eight strides are issued together (one memory round trip per eight
  // instead of one per partial: the partials were written by every XCD and
  // miss this XCD's L2 the first time).  Past the end a thread adds 0.0,
  // which leaves its sum unchanged.
  double s = 0.0;
  for (int i = threadIdx.x; i < np; i += 8 * kWG) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = i + u * kWG < np ? p[i + u * kWG] : 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  return s;
}

__device__ __forceinline__ double sum_partials(const double* __restrict__ p, int np, double* red) {
  return block_sum(partial_share(p, np), red);
}

// XCD-aware tile assignment: workgroups are dispatched round-robin over the
// 8 XCDs, so workgroup b runs on XCD b % 8.  Give each XCD a contiguous eighth
// of the tiles and let its workgroups stride through it, so neighbouring rows
// (and the vector entries they gather) stay in one XCD's L2.
__device__ __forceinline__ void tile_range(int ntiles, int& t0, int& t1, int& step) {
  const int G = gridDim.x, b = blockIdx.x;
  if (G >= 8 && (G & 7) == 0) {
    const int x = b & 7, slot = b >> 3;
    t0 = (int)(((long long)ntiles * x) >> 3) + slot;
    t1 = (int)(((long long)ntiles * (x + 1)) >> 3);
    step = G >> 3;
  } else {
    t0 = b;
    t1 = ntiles;
    step = G;
  }
}

// Matrix streams (values, column indices, row pointers) are read once per
// product.  With NT they are loaded non-temporally: they do not displace the
// gathered vector entries from L2, and they are not allocated in the 256 MB
// last-level Infinity Cache (MALL), which is then left to the operator the
// host chose to keep resident there across iterations.
template <bool NT, typename U>
__device__ __forceinline__ U ld_stream(const U* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// ---------------------------------------------------------------------------
// CSR row tiles
// ---------------------------------------------------------------------------

// Software pipelining of the CSR row tiles, staged through LDS by the
// kernels of one and of several right-hand sides (Args has the CSR arrays
// rp, v, ci): the next tile's row pointers, values and columns are loaded
// into registers (all loads of a thread in flight at once) while the
// current tile does its gathers, then committed to LDS at the top of the
// next round.
constexpr int kPer = kLdsCap / kWG;
template <typename T>
struct TileRegs {
  T v[kPer];
  int c[kPer];
  int rp, rp_last;
};

template <bool NT, typename T, typename Args>
__device__ __forceinline__ void tile_load(const Args& a, const Tile& d, TileRegs<T>& R) {
  const int nr = d.b - d.a, kb = d.d, ne = d.pad[0];
  const int tid = threadIdx.x;
  if (tid <= nr) R.rp = ld_stream<NT>(a.rp + d.a + tid);
  if (tid == 0 && nr == kWG) R.rp_last = ld_stream<NT>(a.rp + d.a + kWG);
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * kWG;
    if (e < ne) {
      R.v[j] = ld_stream<NT>(a.v + kb + e);
      R.c[j] = ld_stream<NT>(a.ci + kb + e);
    }
  }
}

template <typename T>
__device__ __forceinline__ void tile_commit(const Tile& d, const TileRegs<T>& R, T* s_val,
                                            int* s_col, int* s_rp) {
  const int nr = d.b - d.a, ne = d.pad[0];
  const int tid = threadIdx.x;
  if (tid <= nr) s_rp[tid] = R.rp;
  if (tid == 0 && nr == kWG) s_rp[kWG] = R.rp_last;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int e = tid + j * kWG;
    if (e < ne) {
      s_val[e] = R.v[j];
      s_col[e] = R.c[j];
    }
  }
}

}  // namespace sla
