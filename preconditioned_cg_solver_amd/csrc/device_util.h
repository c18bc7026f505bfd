// Device helpers shared by the PCG kernels (single and several right-hand
// sides): deterministic workgroup reductions, the XCD-aware assignment of
// work items to workgroups, and streaming loads of matrix data.
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace sla {

// ---------------------------------------------------------------------------
// Reductions (deterministic: fixed association order)
// ---------------------------------------------------------------------------

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
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

__device__ __forceinline__ double sum_partials(const double* __restrict__ p, int np, double* red) {
  double s = 0.0;
  for (int i = threadIdx.x; i < np; i += kWG) s += p[i];
  return block_sum(s, red);
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

}  // namespace sla
