// Setup kernels of the gfx950 PCG library: run once per matrix handle.
//
//  * row binning: consecutive rows are packed into SpMV tiles of at most
//    kTileRows rows and kLdsCap nonzeros (staged in LDS); rows longer than
//    kLdsCap are split into kLongChunk-nonzero chunks (row splitting);
//  * explicit transpose G^T (built once so the G^T product needs no scatter
//    and no atomics): a stable LSD radix sort of the entries by column, so
//    every transposed row lists its columns in ascending order and the result
//    is deterministic; 3x3 blocks are transposed as well;
//  * optional structure validation.
//
// Pages: "Learning Sparse Approximate Inverse Preconditioners for CG Solvers
// on GPUs", "Approach" (G and G^T products each iteration); the sparse-format
// guide "Efficient Sparse Matrix Algebra in Python", "SciPy sparse" (convert
// once, keep conversions out of hot loops).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <cstdio>
#include <climits>
#include <cstdlib>
#include <vector>

#include "internal.h"

namespace sla {
namespace {

constexpr int kScanItems = 8;                    // per thread
constexpr int kScanTile = kWG * kScanItems;      // 2048 per workgroup
constexpr int kRadixBits = 8;
constexpr int kRadixDigits = 1 << kRadixBits;
constexpr int kRadixItems = 8;
constexpr int kRadixTile = kWG * kRadixItems;    // 2048 keys per workgroup

// ---------------------------------------------------------------------------
// Exclusive prefix sum of int32 (device-wide, three phases, recursive).
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kWG) void scan_tiles(const int* __restrict__ in, int* __restrict__ out,
                                                  int* __restrict__ tile_sums, int m) {
  __shared__ int s_t[kWG];
  const int base = blockIdx.x * kScanTile + threadIdx.x * kScanItems;
  int v[kScanItems];
  int run = 0;
#pragma unroll
  for (int j = 0; j < kScanItems; ++j) {
    const int idx = base + j;
    v[j] = idx < m ? in[idx] : 0;
    const int t = v[j];
    v[j] = run;
    run += t;
  }
  s_t[threadIdx.x] = run;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread totals (integers: exact).
  for (int off = 1; off < kWG; off <<= 1) {
    const int add = (int)threadIdx.x >= off ? s_t[threadIdx.x - off] : 0;
    __syncthreads();
    s_t[threadIdx.x] += add;
    __syncthreads();
  }
  const int excl = s_t[threadIdx.x] - run;
#pragma unroll
  for (int j = 0; j < kScanItems; ++j) {
    const int idx = base + j;
    if (idx < m) out[idx] = v[j] + excl;
  }
  if (threadIdx.x == kWG - 1 && tile_sums) tile_sums[blockIdx.x] = s_t[kWG - 1];
}

__global__ __launch_bounds__(kWG) void scan_add(int* __restrict__ out, const int* __restrict__ offs,
                                                int m) {
  const int add = offs[blockIdx.x];
  const int base = blockIdx.x * kScanTile;
  for (int j = threadIdx.x; j < kScanTile; j += kWG) {
    const int idx = base + j;
    if (idx < m) out[idx] += add;
  }
}

// Exclusive scan of m ints (in may equal out).  Temporary memory is taken
// stream-ordered and released before returning.
sla_status exclusive_scan(const int* in, int* out, int m, hipStream_t s) {
  if (m <= 0) return SLA_OK;
  const int tiles = (m + kScanTile - 1) / kScanTile;
  if (tiles == 1) {
    hipLaunchKernelGGL(scan_tiles, dim3(1), dim3(kWG), 0, s, in, out, (int*)nullptr, m);
    SLA_HIP(hipGetLastError());
    return SLA_OK;
  }
  int* sums = nullptr;
  SLA_HIP(hipMallocAsync((void**)&sums, sizeof(int) * (size_t)tiles, s));
  hipLaunchKernelGGL(scan_tiles, dim3(tiles), dim3(kWG), 0, s, in, out, sums, m);
  SLA_HIP(hipGetLastError());
  sla_status st = exclusive_scan(sums, sums, tiles, s);
  if (st != SLA_OK) return st;
  hipLaunchKernelGGL(scan_add, dim3(tiles), dim3(kWG), 0, s, out, (const int*)sums, m);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipFreeAsync(sums, s));
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// Row binning into tiles.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int floor_pow2(int v) {
  int p = 1;
  while (p * 2 <= v) p *= 2;
  return p;
}
__device__ __forceinline__ int ilog2(int p) {
  int l = 0;
  while ((1 << l) < p) ++l;
  return l;
}

// Greedy packing of the rows [r0, r1) of one 256-row block.  `emit_lds(a, b,
// nnz)` gets row ranges that fit in LDS; `emit_long(row, kb, ke)` gets rows
// longer than kLdsCap.
template <class E>
__device__ void pack_block(const int* __restrict__ rp, int r0, int r1, E& em) {
  int cur = r0, cur_nnz = 0;
  for (int i = r0; i < r1; ++i) {
    const int kb = rp[i], ke = rp[i + 1];
    const int len = ke - kb;
    if (len > kLdsCap) {
      if (cur < i) em.lds(cur, i, cur_nnz);
      em.longrow(i, kb, ke);
      cur = i + 1;
      cur_nnz = 0;
    } else if (cur_nnz + len > kLdsCap) {
      em.lds(cur, i, cur_nnz);
      cur = i;
      cur_nnz = len;
    } else {
      cur_nnz += len;
    }
  }
  if (cur < r1) em.lds(cur, r1, cur_nnz);
}

struct CountEmit {
  int tiles = 0, longrows = 0, chunks = 0;
  __device__ void lds(int, int, int) { ++tiles; }
  __device__ void longrow(int, int kb, int ke) {
    const int nc = (ke - kb + kLongChunk - 1) / kLongChunk;
    tiles += nc;
    longrows += 1;
    chunks += nc;
  }
};

struct WriteEmit {
  const int* rp;
  Tile* out;
  int* lrows;  // row index of every long row, in long-row order
  int t, lr, ch;
  __device__ void lds(int a, int b, int nnz) {
    const int rows = b - a;
    const int avg = (nnz + rows - 1) / max(rows, 1);
    int want = 1;
    while (want < avg && want < 64) want *= 2;
    const int lanes = min(want, min(64, floor_pow2(kWG / rows)));
    Tile d;
    d.a = a;
    d.b = b;
    d.c = ilog2(lanes);
    d.d = rp[a];
    d.kind = kTileLds;
    d.pad[0] = nnz;
    d.pad[1] = d.pad[2] = 0;
    out[t++] = d;
  }
  __device__ void longrow(int row, int kb, int ke) {
    const int nc = (ke - kb + kLongChunk - 1) / kLongChunk;
    for (int c = 0; c < nc; ++c) {
      Tile d;
      d.a = row;
      d.b = kb + c * kLongChunk;
      d.c = min(ke, kb + (c + 1) * kLongChunk);
      d.d = ch + c;
      d.kind = kTileLong;
      d.pad[0] = lr;
      d.pad[1] = nc;
      d.pad[2] = ch;
      out[t++] = d;
    }
    lrows[lr] = row;
    lr += 1;
    ch += nc;
  }
};

__global__ void tiling_count(const int* __restrict__ rp, int n, int nblk, int* __restrict__ ct,
                             int* __restrict__ cl, int* __restrict__ cc) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  CountEmit em;
  pack_block(rp, b * kTileRows, min(n, (b + 1) * kTileRows), em);
  ct[b] = em.tiles;
  cl[b] = em.longrows;
  cc[b] = em.chunks;
}

__global__ void tiling_write(const int* __restrict__ rp, int n, int nblk, const int* __restrict__ ot,
                             const int* __restrict__ ol, const int* __restrict__ oc,
                             Tile* __restrict__ out, int* __restrict__ lrows) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblk) return;
  WriteEmit em{rp, out, lrows, ot[b], ol[b], oc[b]};
  pack_block(rp, b * kTileRows, min(n, (b + 1) * kTileRows), em);
}

// ---------------------------------------------------------------------------
// Transpose: stable LSD radix sort of (column, entry index) pairs.
// ---------------------------------------------------------------------------

__global__ void count_cols(const int* __restrict__ ci, int nnzb, int* __restrict__ cnt) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnzb; k += gridDim.x * blockDim.x)
    atomicAdd(&cnt[ci[k]], 1);
}

// Histogram of one digit per tile, stored digit-major: hist[d * ntiles + tile].
__global__ __launch_bounds__(kWG) void radix_hist(const int* __restrict__ keys, int m, int shift,
                                                  int ntiles, int* __restrict__ hist) {
  __shared__ int cnt[kRadixDigits];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRadixTile;
  for (int s = 0; s < kRadixItems; ++s) {
    const int e = base + s * kWG + threadIdx.x;
    if (e < m) atomicAdd(&cnt[(keys[e] >> shift) & (kRadixDigits - 1)], 1);
  }
  __syncthreads();
  hist[threadIdx.x * ntiles + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: element e of the tile goes to offs[d * ntiles + tile] +
// (number of earlier elements of the tile with the same digit).  Elements
// are ranked in rounds of 256 consecutive keys, one per thread in thread
// order; inside a wavefront the same-digit peers are found with ballots.
// `vals_in == nullptr` means the values are the element indices (first pass).
__global__ __launch_bounds__(kWG) void radix_scatter(const int* __restrict__ keys_in,
                                                     const int* __restrict__ vals_in, int m,
                                                     int shift, int ntiles,
                                                     const int* __restrict__ offs,
                                                     int* __restrict__ keys_out,
                                                     int* __restrict__ vals_out) {
  __shared__ int running[kRadixDigits];
  __shared__ int wcount[kWaves][kRadixDigits];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  running[tid] = offs[tid * ntiles + blockIdx.x];
  for (int q = 0; q < kWaves; ++q) wcount[q][tid] = 0;
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
  const int base = blockIdx.x * kRadixTile;
  for (int s = 0; s < kRadixItems; ++s) {
    const int e = base + s * kWG + tid;
    const bool valid = e < m;
    int key = 0, val = 0, d = 0;
    if (valid) {
      key = keys_in[e];
      val = vals_in ? vals_in[e] : e;
      d = (key >> shift) & (kRadixDigits - 1);
    }
    unsigned long long peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < kRadixBits; ++bit) {
      const bool on = (d >> bit) & 1;
      const unsigned long long bal = __ballot(on);
      peers &= on ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) wcount[w][d] = __popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = running[d] + rank;
      for (int q = 0; q < w; ++q) pos += wcount[q][d];
      keys_out[pos] = key;
      vals_out[pos] = val;
    }
    __syncthreads();
    int tot = 0;
    for (int q = 0; q < kWaves; ++q) {
      tot += wcount[q][tid];
      wcount[q][tid] = 0;
    }
    running[tid] += tot;
    __syncthreads();
  }
}

// Row of stored entry k: the last row whose row_ptr <= k.
__device__ __forceinline__ int row_of(const int* __restrict__ rp, int nbr, int k) {
  int lo = 0, hi = nbr;  // rp[lo] <= k < rp[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (rp[mid] <= k) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <typename T>
__global__ void transpose_fill(const int* __restrict__ rp, const T* __restrict__ v, int nbr,
                               int nnzb, int bs,
                               const int* __restrict__ order, int* __restrict__ t_ci,
                               T* __restrict__ t_v) {
  for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnzb; p += gridDim.x * blockDim.x) {
    const int k = order[p];
    t_ci[p] = row_of(rp, nbr, k);
    if (bs == 1) {
      t_v[p] = v[k];
    } else {
      const int bb = bs * bs;
      for (int r = 0; r < bs; ++r)
        for (int c = 0; c < bs; ++c)
          t_v[(size_t)p * bb + c * bs + r] = v[(size_t)k * bb + r * bs + c];
    }
  }
}

// ---------------------------------------------------------------------------
// Locality ordering of irregular matrices: a symmetric permutation P that
// puts high-degree rows first (so the entries most gathered share cache
// lines) and deals them round-robin over eight contiguous row segments (one
// per XCD share of the row-parallel kernels, so each gets the same mix).
// ---------------------------------------------------------------------------

// Sampled count of stored entries far from the diagonal: entry e_k =
// floor(k nnz / samples) for k < samples, far when |col - row| > near.
__global__ __launch_bounds__(kWG) void sample_far(const int* __restrict__ rp,
                                                  const int* __restrict__ ci, int n, int nnz,
                                                  int samples, int near, int* __restrict__ far) {
  __shared__ int cnt;
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  int mine = 0;
  for (int k = blockIdx.x * kWG + threadIdx.x; k < samples; k += gridDim.x * kWG) {
    const int e = (int)((int64_t)k * nnz / samples);
    const int r = row_of(rp, n, e);
    const int d = ci[e] - r;
    mine += (d > near || d < -near) ? 1 : 0;
  }
  atomicAdd(&cnt, mine);
  __syncthreads();
  if (threadIdx.x == 0) atomicAdd(far, cnt);
}

// Sort key of row i: longer rows first (ascending keys), lengths capped.
__global__ void order_keys(const int* __restrict__ rp, int n, int* __restrict__ keys) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    keys[i] = kOrderKeyMax - min(rp[i + 1] - rp[i], kOrderKeyMax);
}

// Rank k of the degree order (row srt[k]) goes to segment k mod 8, position
// floor(k / 8) inside it; segment x starts at seg.start[x].
struct SegStarts {
  int start[8];
};
__global__ void order_deal(const int* __restrict__ srt, int n, SegStarts seg,
                           int* __restrict__ perm, int* __restrict__ iperm) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < n; k += gridDim.x * blockDim.x) {
    const int pos = seg.start[k & 7] + (k >> 3);
    const int o = srt[k];
    perm[pos] = o;
    iperm[o] = pos;
  }
}

// Row lengths of P M P^T (slot n is 0, so the exclusive scan ends at nnz).
__global__ void perm_lengths(const int* __restrict__ rp, const int* __restrict__ perm, int n,
                             int* __restrict__ len) {
  for (int j = blockIdx.x * blockDim.x + threadIdx.x; j <= n; j += gridDim.x * blockDim.x)
    len[j] = j < n ? rp[perm[j] + 1] - rp[perm[j]] : 0;
}

// Entry k of P M P^T: row j of the new matrix is row perm[j] of M, entries
// in M's order, columns renamed through iperm.
template <typename T>
__global__ void perm_fill(const int* __restrict__ rp, const int* __restrict__ ci,
                          const T* __restrict__ v, const int* __restrict__ nrp,
                          const int* __restrict__ perm, const int* __restrict__ iperm, int n,
                          int nnz, int* __restrict__ nci, T* __restrict__ nv) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += gridDim.x * blockDim.x) {
    const int j = row_of(nrp, n, k);
    const int src = rp[perm[j]] + (k - nrp[j]);
    nci[k] = iperm[ci[src]];
    nv[k] = v[src];
  }
}

// Rows of n x cols row-major arrays: dst row j = src row perm[j] (into the
// ordering) or dst row perm[j] = src row j (back); src == nullptr writes
// zeros to dst.
template <typename T>
__global__ void permute_rows_k(const int* __restrict__ perm, const T* __restrict__ src,
                               T* __restrict__ dst, int n, int cols, bool into) {
  const int64_t m = (int64_t)n * cols;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int j = (int)(e / cols), c = (int)(e - (int64_t)j * cols);
    const int64_t o = (int64_t)perm[j] * cols + c;
    if (!src) dst[e] = T(0);
    else if (into) dst[e] = src[o];
    else dst[o] = src[e];
  }
}

// ---------------------------------------------------------------------------
// Validation.
// ---------------------------------------------------------------------------

__global__ void validate_rows(const int* __restrict__ rp, const int* __restrict__ ci, int nbr,
                              int nnzb, int* __restrict__ bad) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nbr; i += gridDim.x * blockDim.x) {
    const int kb = rp[i], ke = rp[i + 1];
    if (ke < kb || kb < 0 || ke > nnzb) {
      atomicOr(bad, 1);
      continue;
    }
    int prev = -1;
    for (int k = kb; k < ke; ++k) {
      const int c = ci[k];
      if (c < 0 || c >= nbr) atomicOr(bad, 2);
      if (c <= prev) atomicOr(bad, 4);
      prev = c;
    }
  }
}

// ---------------------------------------------------------------------------
// SELL-64 conversion.
// ---------------------------------------------------------------------------

// Per slice: slots (widest row x 64); global: widest row and largest
// |column - row| (to decide whether int16 offsets can hold the columns).
// One wavefront per slice (lane = row), wavefronts striding over the slices;
// the maxima are reduced in the workgroup and folded in with one atomic
// each per workgroup.
__global__ __launch_bounds__(kWG) void sell_widths(const int* __restrict__ rp,
                                                   const int* __restrict__ ci, int n, int nslices,
                                                   int* __restrict__ slots,
                                                   int* __restrict__ maxw,
                                                   int* __restrict__ maxd) {
  __shared__ int s_w[kWaves], s_d[kWaves];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int wmax = 0, dmax = 0;
  for (int sl = blockIdx.x * kWaves + wv; sl < nslices; sl += gridDim.x * kWaves) {
    const int i = sl * kSlice + lane;
    int w = 0, d = 0;
    if (i < n) {
      const int kb = rp[i], ke = rp[i + 1];
      w = ke - kb;
      if (ke > kb) d = max(abs(ci[kb] - i), abs(ci[ke - 1] - i));
    }
    for (int off = 32; off >= 1; off >>= 1) {
      w = max(w, __shfl_xor(w, off, 64));
      d = max(d, __shfl_xor(d, off, 64));
    }
    if (lane == 0) slots[sl] = w * kSlice;
    wmax = max(wmax, w);
    dmax = max(dmax, d);
  }
  if (lane == 0) {
    s_w[wv] = wmax;
    s_d[wv] = dmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kWaves; ++k) {
      wmax = max(wmax, s_w[k]);
      dmax = max(dmax, s_d[k]);
    }
    atomicMax(maxw, wmax);
    atomicMax(maxd, dmax);
  }
}

// Fill the SELL slots of one row (rows past n only get padding).  C is the
// column type: int (absolute column, -1 = padding) or short (offset from the
// row, kPad16 = padding).
template <typename T, typename C>
__global__ void sell_fill(const int* __restrict__ rp, const int* __restrict__ ci,
                          const T* __restrict__ v, int n, int nslices,
                          const int* __restrict__ soff, T* __restrict__ sv,
                          C* __restrict__ sc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // row (padded to slices)
  if (i >= nslices * kSlice) return;
  const int sl = i / kSlice, lane = i % kSlice;
  const int off = soff[sl], w = (soff[sl + 1] - off) / kSlice;
  const int kb = i < n ? rp[i] : 0, len = i < n ? rp[i + 1] - kb : 0;
  constexpr bool rel = sizeof(C) == 2;
  for (int j = 0; j < w; ++j) {
    const int dst = off + j * kSlice + lane;
    if (j < len) {
      sv[dst] = v[kb + j];
      sc[dst] = (C)(rel ? ci[kb + j] - i : ci[kb + j]);
    } else {
      sv[dst] = T(0);
      sc[dst] = (C)(rel ? kPad16 : -1);
    }
  }
}

// ---- slice-offset form ----

// Per slice (one wavefront, lane = row): the ascending union of the column
// offsets (col - row) of its rows, by repeated wavefront minima over each
// row's next offset.  count[s] = size of the union, or kOfsMax + 1 when it
// is larger or a row does not list its columns in increasing order.
__global__ __launch_bounds__(kWG) void slice_union(const int* __restrict__ rp,
                                                   const int* __restrict__ ci, int n, int nslices,
                                                   int* __restrict__ count,
                                                   int* __restrict__ ofs) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int sl = blockIdx.x * kWaves + wv; sl < nslices; sl += gridDim.x * kWaves) {
    const int i = sl * kSlice + lane;
    int k = i < n ? rp[i] : 0;
    const int ke = i < n ? rp[i + 1] : 0;
    int prev = INT_MIN, cnt = 0;
    bool bad = false;
    while (cnt <= kOfsMax) {
      const int cur = k < ke ? ci[k] - i : INT_MAX;
      if (k < ke && cur <= prev) bad = true;
      int m = cur;
      for (int off = 32; off >= 1; off >>= 1) m = min(m, __shfl_xor(m, off, 64));
      if (m == INT_MAX) break;
      if (cnt < kOfsMax && lane == 0) ofs[(size_t)sl * kOfsMax + cnt] = m;
      ++cnt;
      if (cur == m) {
        prev = cur;
        ++k;
      }
    }
    bad = __any(bad);
    if (lane == 0) count[sl] = bad ? kOfsMax + 1 : cnt;
  }
}

// Fill of the slice-offset form: row i of slice s puts its entry at offset
// ofs[s][j] into slot j (rows list their columns in increasing order, so a
// merge walk finds them); missing slots get value 0 and kPad16.
template <typename T>
__global__ void sell_fill_ofs(const int* __restrict__ rp, const int* __restrict__ ci,
                              const T* __restrict__ v, int n, int nslices,
                              const int* __restrict__ soff, const int* __restrict__ ofs,
                              T* __restrict__ sv, short* __restrict__ sd, int* __restrict__ so,
                              uint8_t* __restrict__ sm) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // row (padded to slices)
  if (i >= nslices * kSlice) return;
  const int sl = i / kSlice, lane = i % kSlice;
  const int off = soff[sl], w = (soff[sl + 1] - off) / kSlice;
  int k = i < n ? rp[i] : 0;
  const int ke = i < n ? rp[i + 1] : 0;
  unsigned mask = 0;
  for (int j = 0; j < w; ++j) {
    const int o = ofs[(size_t)sl * kOfsMax + j];
    const int dst = off + j * kSlice + lane;
    if (k < ke && ci[k] - i == o) {
      sv[dst] = v[k];
      sd[dst] = (short)o;
      mask |= 1u << j;
      ++k;
    } else {
      sv[dst] = T(0);
      sd[dst] = (short)kPad16;
    }
    if (lane == 0) so[off / kSlice + j] = o;
  }
  sm[i] = (uint8_t)mask;
}

// ---- sliced ELLPACK for 3x3 BSR ----

// Per slice: slots (widest block row); global: widest block row and largest
// |block column - block row| (whether int16 offsets can hold the columns).
// One thread per slice, threads striding over the slices; the maxima are
// reduced in the workgroup and folded in with one atomic each per workgroup.
__global__ __launch_bounds__(kWG) void bsell_widths(const int* __restrict__ rp,
                                                    const int* __restrict__ ci, int nbr,
                                                    int nslices, int* __restrict__ slots,
                                                    int* __restrict__ maxw,
                                                    int* __restrict__ maxd) {
  __shared__ int s_w[kWaves], s_d[kWaves];
  int wmax = 0, dmax = 0;
  for (int sl = blockIdx.x * kWG + threadIdx.x; sl < nslices; sl += gridDim.x * kWG) {
    int w = 0;
    const int r1 = min(nbr, (sl + 1) * kBSlice);
    for (int i = sl * kBSlice; i < r1; ++i) {
      const int kb = rp[i], ke = rp[i + 1];
      w = max(w, ke - kb);
      if (ke > kb) dmax = max(dmax, max(abs(ci[kb] - i), abs(ci[ke - 1] - i)));
    }
    slots[sl] = w;
    wmax = max(wmax, w);
  }
  for (int off = 32; off >= 1; off >>= 1) {
    wmax = max(wmax, __shfl_xor(wmax, off, 64));
    dmax = max(dmax, __shfl_xor(dmax, off, 64));
  }
  if ((threadIdx.x & 63) == 0) {
    s_w[threadIdx.x >> 6] = wmax;
    s_d[threadIdx.x >> 6] = dmax;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kWaves; ++k) {
      wmax = max(wmax, s_w[k]);
      dmax = max(dmax, s_d[k]);
    }
    atomicMax(maxw, wmax);
    atomicMax(maxd, dmax);
  }
}

// Fill the slots of one block row (block rows past nbr only get padding).
// C is the column type: int (absolute block column, -1 = padding) or short
// (offset from the block row, kPad16 = padding).
template <typename T, typename C>
__global__ void bsell_fill(const int* __restrict__ rp, const int* __restrict__ ci,
                           const T* __restrict__ v, int nbr, int nslices,
                           const int* __restrict__ soff, T* __restrict__ sv,
                           C* __restrict__ sc) {
  const int I = blockIdx.x * blockDim.x + threadIdx.x;  // block row (padded)
  if (I >= nslices * kBSlice) return;
  const int sl = I / kBSlice, li = I % kBSlice;
  const int off = soff[sl], w = soff[sl + 1] - off;
  const int kb = I < nbr ? rp[I] : 0, len = I < nbr ? rp[I + 1] - kb : 0;
  constexpr bool rel = sizeof(C) == 2;
  for (int j = 0; j < w; ++j) {
    const int q = off + j;
    const size_t dst = (size_t)q * kBSlotCols + li;
    if (j < len) {
      for (int e = 0; e < 9; ++e) sv[bsell_val(q, e / 3, e % 3, li)] = v[(size_t)(kb + j) * 9 + e];
      sc[dst] = (C)(rel ? ci[kb + j] - I : ci[kb + j]);
    } else {
      for (int e = 0; e < 9; ++e) sv[bsell_val(q, e / 3, e % 3, li)] = T(0);
      sc[dst] = (C)(rel ? kPad16 : -1);
    }
  }
}

// Longest row (in stored entries or blocks) of a CSR / BSR row pointer array.
__global__ __launch_bounds__(kWG) void row_len_max(const int* __restrict__ rp, int nbr,
                                                   int* __restrict__ out) {
  __shared__ int s_m[kWaves];
  int m = 0;
  for (int i = blockIdx.x * kWG + threadIdx.x; i < nbr; i += gridDim.x * kWG)
    m = max(m, rp[i + 1] - rp[i]);
  for (int off = 32; off >= 1; off >>= 1) m = max(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kWaves; ++k) m = max(m, s_m[k]);
    atomicMax(out, m);
  }
}

int grid_for(int64_t work, int per_block = kWG) {
  const int64_t g = (work + per_block - 1) / per_block;
  return (int)std::max<int64_t>(1, std::min<int64_t>(g, 65536));
}

}  // namespace

// ---------------------------------------------------------------------------
// Host entry points.
// ---------------------------------------------------------------------------

sla_status build_tiling(const int32_t* d_rp, int64_t n, MatView& view, void** owned_tiles,
                        hipStream_t s) {
  view.tiles = nullptr;
  view.ntiles = view.nlong = view.nlong_rows = view.n_long_part = 0;
  if (n == 0) return SLA_OK;
  const int nblk = (int)((n + kTileRows - 1) / kTileRows);
  int* buf = nullptr;
  SLA_HIP(hipMallocAsync((void**)&buf, sizeof(int) * 6 * (size_t)(nblk + 1), s));
  int *ct = buf, *cl = buf + (nblk + 1), *cc = buf + 2 * (nblk + 1);
  int *ot = buf + 3 * (nblk + 1), *ol = buf + 4 * (nblk + 1), *oc = buf + 5 * (nblk + 1);
  SLA_HIP(hipMemsetAsync(buf, 0, sizeof(int) * 6 * (size_t)(nblk + 1), s));
  hipLaunchKernelGGL(tiling_count, dim3((nblk + 127) / 128), dim3(128), 0, s, d_rp, (int)n, nblk,
                     ct, cl, cc);
  SLA_HIP(hipGetLastError());
  // scan nblk + 1 entries so the last slot holds the totals
  sla_status st;
  if ((st = exclusive_scan(ct, ot, nblk + 1, s)) != SLA_OK) return st;
  if ((st = exclusive_scan(cl, ol, nblk + 1, s)) != SLA_OK) return st;
  if ((st = exclusive_scan(cc, oc, nblk + 1, s)) != SLA_OK) return st;
  int tot[3];
  SLA_HIP(hipMemcpyAsync(&tot[0], ot + nblk, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&tot[1], ol + nblk, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&tot[2], oc + nblk, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  // one allocation: the tiles, then the row index of every long row
  Tile* tiles = nullptr;
  SLA_HIP(buf_alloc((void**)&tiles, sizeof(Tile) * (size_t)std::max(1, tot[0]) +
                                        sizeof(int) * (size_t)std::max(1, tot[1])));
  int* lrows = (int*)(tiles + std::max(1, tot[0]));
  hipLaunchKernelGGL(tiling_write, dim3((nblk + 127) / 128), dim3(128), 0, s, d_rp, (int)n, nblk,
                     (const int*)ot, (const int*)ol, (const int*)oc, tiles, lrows);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipFreeAsync(buf, s));
  SLA_HIP(hipStreamSynchronize(s));
  *owned_tiles = tiles;
  view.tiles = tiles;
  view.ntiles = tot[0];
  view.nlong_rows = tot[1];
  view.n_long_part = tot[2];
  view.nlong = tot[2];
  view.long_rows = lrows;
  return SLA_OK;
}

// Stable LSD radix sort of m non-negative keys below 2^bits, carrying the
// element indices.  `work` holds radix_work_ints(m) ints; *idx_out points
// into it and gives the element indices in ascending key order (equal keys
// keep their input order).
size_t radix_work_ints(int m) {
  const size_t tiles = ((size_t)std::max(1, m) + kRadixTile - 1) / kRadixTile;
  return 4 * (size_t)std::max(1, m) + (size_t)kRadixDigits * tiles;
}

sla_status radix_sort_indices(const int* keys, int m, int bits, int* work, const int** idx_out,
                              hipStream_t s) {
  const int passes = (bits + kRadixBits - 1) / kRadixBits;
  const int ntiles = (m + kRadixTile - 1) / kRadixTile;
  const size_t hist_n = (size_t)kRadixDigits * ntiles;
  int *ka = work, *va = work + m, *kb = work + 2 * (size_t)m, *vb = work + 3 * (size_t)m;
  int* hist = work + 4 * (size_t)m;
  const int* kin = keys;
  const int* vin = nullptr;
  sla_status st = SLA_OK;
  for (int p = 0; p < passes; ++p) {
    const int shift = p * kRadixBits;
    int* kout = (p & 1) ? kb : ka;
    int* vout = (p & 1) ? vb : va;
    hipLaunchKernelGGL(radix_hist, dim3(ntiles), dim3(kWG), 0, s, kin, m, shift, ntiles, hist);
    SLA_HIP(hipGetLastError());
    if ((st = exclusive_scan(hist, hist, (int)hist_n, s)) != SLA_OK) return st;
    hipLaunchKernelGGL(radix_scatter, dim3(ntiles), dim3(kWG), 0, s, kin, vin, m, shift, ntiles,
                       (const int*)hist, kout, vout);
    SLA_HIP(hipGetLastError());
    kin = kout;
    vin = vout;
  }
  *idx_out = vin;
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// Column-block copies.  Entries are sorted stably by their column block
// (col / seg), which lays the eight blocks out one after another, each in
// row order with the rows' own entry order; each block's row pointer is then
// found by binary search over the sorted entries' rows.
// ---------------------------------------------------------------------------

namespace {

__global__ void cb_keys(const int* __restrict__ ci, int nnz, int seg, int* __restrict__ keys) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += gridDim.x * blockDim.x)
    keys[k] = ci[k] / seg;
}

// per-block entry counts (integer atomics on a workgroup's LDS histogram)
__global__ __launch_bounds__(kWG) void cb_count(const int* __restrict__ keys, int nnz,
                                                int* __restrict__ cnt) {
  __shared__ int h[kColBlocks];
  if (threadIdx.x < kColBlocks) h[threadIdx.x] = 0;
  __syncthreads();
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += gridDim.x * blockDim.x)
    atomicAdd(&h[keys[k]], 1);
  __syncthreads();
  if (threadIdx.x < kColBlocks && h[threadIdx.x]) atomicAdd(&cnt[threadIdx.x], h[threadIdx.x]);
}

// sorted entry k: its column, value and row
template <typename T>
__global__ void cb_gather(const int* __restrict__ rp, int n, const int* __restrict__ ci,
                          const T* __restrict__ v, const int* __restrict__ idx, int nnz,
                          int* __restrict__ oci, T* __restrict__ ov, int* __restrict__ orow) {
  for (int k = blockIdx.x * blockDim.x + threadIdx.x; k < nnz; k += gridDim.x * blockDim.x) {
    const int src = idx[k];
    oci[k] = ci[src];
    ov[k] = v[src];
    orow[k] = row_of(rp, n, src);
  }
}

// row pointer of block b, relative to the block's first entry: the first
// sorted entry of the block whose row is >= r
__global__ void cb_rowptr(const int* __restrict__ orow, const int* __restrict__ bstart, int n,
                          int* __restrict__ rpb) {
  const int64_t m = (int64_t)kColBlocks * (n + 1);
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < m;
       e += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(e / (n + 1)), r = (int)(e - (int64_t)b * (n + 1));
    int lo = bstart[b], hi = bstart[b + 1];
    const int first = lo;
    while (lo < hi) {
      const int mid = lo + ((hi - lo) >> 1);
      if (orow[mid] < r) lo = mid + 1;
      else hi = mid;
    }
    rpb[e] = lo - first;
  }
}

}  // namespace

// One view split into kColBlocks column blocks (arrays owned by `cb`).
sla_status split_view(const sla_mat& m, const MatView& v, ColBlocks* cb, ColBlockSet* out,
                      hipStream_t s) {
  const int n = (int)m.nbr, nnz = (int)m.nnzb;
  const size_t es = m.dtype == SLA_F64 ? 8 : 4;
  const int seg = std::max(1, (n + kColBlocks - 1) / kColBlocks);
  int *oci = nullptr, *rpb = nullptr;
  void* ov = nullptr;
  SLA_HIP(buf_alloc((void**)&oci, sizeof(int) * (size_t)std::max(1, nnz)));
  cb->owned.push_back(oci);
  SLA_HIP(buf_alloc(&ov, es * (size_t)std::max(1, nnz)));
  cb->owned.push_back(ov);
  SLA_HIP(buf_alloc((void**)&rpb, sizeof(int) * (size_t)kColBlocks * ((size_t)n + 1)));
  cb->owned.push_back(rpb);
  int* tmp = nullptr;  // keys, block counts and starts, rows, radix work
  const size_t ntmp = 2 * (size_t)std::max(1, nnz) + 2 * kColBlocks + 2 + radix_work_ints(nnz);
  SLA_HIP(hipMallocAsync((void**)&tmp, sizeof(int) * ntmp, s));
  int* keys = tmp;
  int* orow = keys + std::max(1, nnz);
  int* cnt = orow + std::max(1, nnz);
  int* bstart = cnt + kColBlocks;
  int* work = bstart + kColBlocks + 2;
  SLA_HIP(hipMemsetAsync(cnt, 0, sizeof(int) * kColBlocks, s));
  int hb[kColBlocks + 1] = {0};
  if (nnz > 0) {
    hipLaunchKernelGGL(cb_keys, dim3(grid_for(nnz)), dim3(kWG), 0, s, v.ci, nnz, seg, keys);
    hipLaunchKernelGGL(cb_count, dim3(std::min(grid_for(nnz), 2048)), dim3(kWG), 0, s,
                       (const int*)keys, nnz, cnt);
    SLA_HIP(hipGetLastError());
    const int* idx = nullptr;
    sla_status st = radix_sort_indices(keys, nnz, 3, work, &idx, s);
    if (st != SLA_OK) return st;
    if (m.dtype == SLA_F64)
      hipLaunchKernelGGL(cb_gather<double>, dim3(grid_for(nnz)), dim3(kWG), 0, s, v.rp, n, v.ci,
                         (const double*)v.v, idx, nnz, oci, (double*)ov, orow);
    else
      hipLaunchKernelGGL(cb_gather<float>, dim3(grid_for(nnz)), dim3(kWG), 0, s, v.rp, n, v.ci,
                         (const float*)v.v, idx, nnz, oci, (float*)ov, orow);
    SLA_HIP(hipGetLastError());
    int hc[kColBlocks];
    SLA_HIP(hipMemcpyAsync(hc, cnt, sizeof(hc), hipMemcpyDeviceToHost, s));
    SLA_HIP(hipStreamSynchronize(s));
    for (int b = 0; b < kColBlocks; ++b) hb[b + 1] = hb[b] + hc[b];
    if (hb[kColBlocks] != nnz) {
      (void)hipFreeAsync(tmp, s);
      set_error("column-block split lost entries");
      return SLA_ERR_HIP;
    }
  }
  SLA_HIP(hipMemcpyAsync(bstart, hb, sizeof(hb), hipMemcpyHostToDevice, s));
  hipLaunchKernelGGL(cb_rowptr, dim3(grid_for((int64_t)kColBlocks * (n + 1))), dim3(kWG), 0, s,
                     (const int*)orow, (const int*)bstart, n, rpb);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipStreamSynchronize(s));
  SLA_HIP(hipFreeAsync(tmp, s));
  int lrows = 0, lparts = 0;
  for (int b = 0; b < kColBlocks; ++b) {
    MatView& bv = out->blk[b];
    bv = MatView{};
    bv.rp = rpb + (size_t)b * ((size_t)n + 1);
    bv.ci = oci + hb[b];
    bv.v = (const char*)ov + es * (size_t)hb[b];
    void* tiles = nullptr;
    sla_status st = build_tiling(bv.rp, n, bv, &tiles, s);
    if (tiles) cb->owned.push_back(tiles);
    if (st != SLA_OK) return st;
    out->lrow_off[b] = lrows;
    out->lpart_off[b] = lparts;
    lrows += bv.nlong_rows;
    lparts += bv.n_long_part;
  }
  // the blocks' long rows share the workspace's long-row scratch, sized
  // for the operator's (see long_rows_bound / long_part_bound)
  if (lrows > long_rows_bound(m) || lparts > long_part_bound(m)) {
    set_error("column-block long rows exceed the long-row scratch");
    return SLA_ERR_HIP;
  }
  return SLA_OK;
}

void free_colblocks(sla_mat* m) {
  if (!m->cb) return;
  for (void* p : m->cb->owned) buf_free(p);
  delete m->cb;
  m->cb = nullptr;
}

bool colblocks_wanted(const sla_mat& A) {
  const char* e = getenv("SLA_COLBLK");
  return A.bs == 1 && !(e && e[0] == '0');
}

sla_status build_colblocks(sla_mat* m, hipStream_t s) {
  if (m->cb || m->bs != 1 || m->n() == 0) return SLA_OK;
  ColBlocks* cb = new (std::nothrow) ColBlocks();
  if (!cb) {
    set_error("host allocation failed");
    return SLA_ERR_OOM;
  }
  m->cb = cb;
  sla_status st = split_view(*m, m->fwd, cb, &cb->fwd, s);
  if (st == SLA_OK && m->has_t) {
    st = split_view(*m, m->tr, cb, &cb->tr, s);
    cb->has_tr = st == SLA_OK;
  }
  if (st != SLA_OK) {
    (void)hipStreamSynchronize(s);
    free_colblocks(m);
  }
  return st;
}

sla_status build_transpose(const sla_mat& m, int32_t** t_rp_out, int32_t** t_ci_out, void** t_v_out,
                           hipStream_t s) {
  const int nbr = (int)m.nbr, nnzb = (int)m.nnzb, bs = m.bs;
  const size_t es = m.dtype == SLA_F64 ? 8 : 4;
  int32_t *t_rp = nullptr, *t_ci = nullptr;
  void* t_v = nullptr;
  SLA_HIP(buf_alloc((void**)&t_rp, sizeof(int) * ((size_t)nbr + 1)));
  SLA_HIP(buf_alloc((void**)&t_ci, sizeof(int) * (size_t)std::max(1, nnzb)));
  SLA_HIP(buf_alloc(&t_v, es * (size_t)bs * bs * (size_t)std::max(1, nnzb)));
  *t_rp_out = t_rp;
  *t_ci_out = t_ci;
  *t_v_out = t_v;
  // row pointer of the transpose: column counts, exclusive scan
  int* cnt = nullptr;
  SLA_HIP(hipMallocAsync((void**)&cnt, sizeof(int) * ((size_t)nbr + 1), s));
  SLA_HIP(hipMemsetAsync(cnt, 0, sizeof(int) * ((size_t)nbr + 1), s));
  if (nnzb > 0) {
    hipLaunchKernelGGL(count_cols, dim3(grid_for(nnzb)), dim3(kWG), 0, s, m.fwd.ci, nnzb, cnt);
    SLA_HIP(hipGetLastError());
  }
  sla_status st = exclusive_scan(cnt, t_rp, nbr + 1, s);
  if (st != SLA_OK) return st;
  SLA_HIP(hipFreeAsync(cnt, s));
  if (nnzb == 0) {
    SLA_HIP(hipStreamSynchronize(s));
    return SLA_OK;
  }
  // stable radix sort of the column keys, carrying entry indices
  int bits = 1;
  while (bits < 31 && ((int64_t)1 << bits) < (int64_t)nbr) ++bits;
  int* work = nullptr;
  SLA_HIP(hipMallocAsync((void**)&work, sizeof(int) * radix_work_ints(nnzb), s));
  const int* vin = nullptr;
  if ((st = radix_sort_indices(m.fwd.ci, nnzb, bits, work, &vin, s)) != SLA_OK) return st;
  if (m.dtype == SLA_F64)
    hipLaunchKernelGGL(transpose_fill<double>, dim3(grid_for(nnzb)), dim3(kWG), 0, s, m.fwd.rp,
                       (const double*)m.fwd.v, nbr, nnzb, bs, vin, t_ci, (double*)t_v);
  else
    hipLaunchKernelGGL(transpose_fill<float>, dim3(grid_for(nnzb)), dim3(kWG), 0, s, m.fwd.rp,
                       (const float*)m.fwd.v, nbr, nnzb, bs, vin, t_ci, (float*)t_v);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipFreeAsync(work, s));
  SLA_HIP(hipStreamSynchronize(s));
  return SLA_OK;
}

sla_status max_row_length(const int32_t* d_rp, int64_t nbr, int* out, hipStream_t s) {
  *out = 0;
  if (nbr == 0) return SLA_OK;
  int* d = nullptr;
  SLA_HIP(hipMallocAsync((void**)&d, sizeof(int), s));
  SLA_HIP(hipMemsetAsync(d, 0, sizeof(int), s));
  hipLaunchKernelGGL(row_len_max, dim3(std::min(grid_for(nbr), 1024)), dim3(kWG), 0, s, d_rp,
                     (int)nbr, d);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipMemcpyAsync(out, d, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipFreeAsync(d, s));
  SLA_HIP(hipStreamSynchronize(s));
  return SLA_OK;
}

sla_status validate_structure(const sla_mat& m, hipStream_t s) {
  int* bad = nullptr;
  SLA_HIP(hipMallocAsync((void**)&bad, sizeof(int), s));
  SLA_HIP(hipMemsetAsync(bad, 0, sizeof(int), s));
  if (m.nbr > 0) {
    hipLaunchKernelGGL(validate_rows, dim3(grid_for(m.nbr)), dim3(kWG), 0, s, m.fwd.rp, m.fwd.ci,
                       (int)m.nbr, (int)m.nnzb, bad);
    SLA_HIP(hipGetLastError());
  }
  int h = 0;
  SLA_HIP(hipMemcpyAsync(&h, bad, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipFreeAsync(bad, s));
  SLA_HIP(hipStreamSynchronize(s));
  if (h) {
    char msg[160];
    snprintf(msg, sizeof msg, "invalid sparse structure:%s%s%s",
             (h & 1) ? " row_ptr not monotone within [0, nnz]" : "", (h & 2) ? " column out of range" : "",
             (h & 4) ? " columns not strictly ascending within a row" : "");
    set_error(msg);
    return SLA_ERR_INVALID_ARG;
  }
  return SLA_OK;
}

// Slice-offset form of a SELL-64 matrix whose int16 offsets fit: built when
// every slice has at most kOfsMax distinct offsets over rows with sorted
// columns and the padding stays within kSellMaxPadPct (SLA_SELL_OFS=0: never).
// Returns SLA_OK with view.so == nullptr when the rows do not qualify.
sla_status build_sell_ofs(MatView& view, int64_t n, int64_t nnz, int32_t dtype, void** owned3,
                          void** owned_ofs2, hipStream_t s) {
  const char* e = getenv("SLA_SELL_OFS");
  if (e && e[0] == '0') return SLA_OK;
  const int nslices = (int)((n + kSlice - 1) / kSlice);
  int* cnt = nullptr;
  int* ofs = nullptr;
  SLA_HIP(hipMallocAsync((void**)&cnt, sizeof(int) * ((size_t)nslices + 1), s));
  SLA_HIP(hipMallocAsync((void**)&ofs, sizeof(int) * (size_t)nslices * kOfsMax, s));
  hipLaunchKernelGGL(slice_union, dim3(std::min(1024, (nslices + kWaves - 1) / kWaves)),
                     dim3(kWG), 0, s, view.rp, view.ci, (int)n, nslices, cnt, ofs);
  SLA_HIP(hipGetLastError());
  std::vector<int> hc((size_t)nslices + 1, 0);
  SLA_HIP(hipMemcpyAsync(hc.data(), cnt, sizeof(int) * (size_t)nslices, hipMemcpyDeviceToHost, s));
  SLA_HIP(hipStreamSynchronize(s));
  int64_t total = 0;
  int wmax = 0;
  bool ok = true;
  for (int sl = 0; sl < nslices && ok; ++sl) {
    ok = hc[sl] <= kOfsMax;
    wmax = std::max(wmax, hc[sl]);
    total += (int64_t)hc[sl] * kSlice;
    hc[sl] *= kSlice;
  }
  if (!ok || total * 100 > nnz * (100 + kSellMaxPadPct) ||
      !sliced_layout_fits(nslices, wmax, kSlice, kSellTail)) {
    SLA_HIP(hipFreeAsync(ofs, s));
    SLA_HIP(hipFreeAsync(cnt, s));
    SLA_HIP(hipStreamSynchronize(s));
    return SLA_OK;
  }
  hc[nslices] = 0;
  SLA_HIP(hipMemcpyAsync(cnt, hc.data(), sizeof(int) * ((size_t)nslices + 1),
                         hipMemcpyHostToDevice, s));
  // the slice offsets of the row-order layout (same size) are rewritten
  int* soff = (int*)owned3[2];
  sla_status st = exclusive_scan(cnt, soff, nslices + 1, s);
  if (st != SLA_OK) return st;
  const size_t es = dtype == SLA_F64 ? 8 : 4;
  const size_t alloc = (size_t)total + kSellTail;
  const size_t nslot = alloc / kSlice;
  void* sv = nullptr;
  void* sd = nullptr;
  void* so = nullptr;
  void* sm = nullptr;
  SLA_HIP(buf_alloc(&sv, es * alloc));
  owned3[0] = sv;
  SLA_HIP(buf_alloc(&sd, 2 * alloc));
  owned3[1] = sd;
  SLA_HIP(buf_alloc(&so, sizeof(int) * nslot));
  owned_ofs2[0] = so;
  SLA_HIP(buf_alloc(&sm, (size_t)nslices * kSlice));
  owned_ofs2[1] = sm;
  SLA_HIP(hipMemsetAsync((char*)sv + es * (size_t)total, 0, es * kSellTail, s));
  SLA_HIP(hipMemsetD16Async((hipDeviceptr_t)((short*)sd + total), (unsigned short)kPad16,
                            kSellTail, s));
  SLA_HIP(hipMemsetAsync(so, 0, sizeof(int) * nslot, s));
  const int rows = nslices * kSlice;
  const dim3 g((rows + 255) / 256), b(256);
  if (dtype == SLA_F64)
    hipLaunchKernelGGL(sell_fill_ofs<double>, g, b, 0, s, view.rp, view.ci,
                       (const double*)view.v, (int)n, nslices, (const int*)soff,
                       (const int*)ofs, (double*)sv, (short*)sd, (int*)so, (uint8_t*)sm);
  else
    hipLaunchKernelGGL(sell_fill_ofs<float>, g, b, 0, s, view.rp, view.ci,
                       (const float*)view.v, (int)n, nslices, (const int*)soff,
                       (const int*)ofs, (float*)sv, (short*)sd, (int*)so, (uint8_t*)sm);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipFreeAsync(ofs, s));
  SLA_HIP(hipFreeAsync(cnt, s));
  view.sv = sv;
  view.sc = nullptr;
  view.sd = (const int16_t*)sd;
  view.soff = soff;
  view.nslices = nslices;
  view.sell_w = wmax;
  view.so = (const int32_t*)so;
  view.sm = (const uint8_t*)sm;
  view.sell_slots = total;
  view.sell = true;
  return SLA_OK;
}

sla_status build_sell(MatView& view, int64_t n, int64_t nnz, int32_t dtype, void** owned3,
                      void** owned_ofs2, hipStream_t s) {
  view.sell = false;
  if (n == 0 || nnz == 0) return SLA_OK;
  const int nslices = (int)((n + kSlice - 1) / kSlice);
  int* buf = nullptr;
  SLA_HIP(hipMallocAsync((void**)&buf, sizeof(int) * ((size_t)nslices + 3), s));
  int* slots = buf;            // nslices + 1 (last one zero)
  int* maxw = buf + nslices + 1;
  int* maxd = buf + nslices + 2;
  SLA_HIP(hipMemsetAsync(buf, 0, sizeof(int) * ((size_t)nslices + 3), s));
  hipLaunchKernelGGL(sell_widths, dim3(std::min(1024, (nslices + kWaves - 1) / kWaves)), dim3(kWG),
                     0, s, view.rp, view.ci, (int)n, nslices, slots, maxw, maxd);
  SLA_HIP(hipGetLastError());
  int* soff = nullptr;
  SLA_HIP(buf_alloc((void**)&soff, sizeof(int) * ((size_t)nslices + 1)));
  owned3[2] = soff;
  sla_status st = exclusive_scan(slots, soff, nslices + 1, s);
  if (st != SLA_OK) return st;
  int h[3] = {0, 0, 0};
  SLA_HIP(hipMemcpyAsync(&h[0], maxw, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&h[1], soff + nslices, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&h[2], maxd, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipFreeAsync(buf, s));
  SLA_HIP(hipStreamSynchronize(s));
  // the slot counts were summed in int32: only a layout whose largest
  // possible size fits int32 has an exact total
  if (!sliced_layout_fits(nslices, h[0], kSlice, kSellTail)) return SLA_OK;
  const int64_t total = h[1];
  if (h[0] > kSellMaxWidth || total * 100 > nnz * (100 + kSellMaxPadPct)) return SLA_OK;
  view.max_dist = h[2];
  const size_t es = dtype == SLA_F64 ? 8 : 4;
  const char* e16 = getenv("SLA_SELL16");
  const bool rel16 = h[2] <= 32767 && !(e16 && e16[0] == '0');
  if (rel16) {
    st = build_sell_ofs(view, n, nnz, dtype, owned3, owned_ofs2, s);
    if (st != SLA_OK || view.sell) {
      if (st == SLA_OK) SLA_HIP(hipStreamSynchronize(s));
      return st;
    }
  }
  void* sv = nullptr;
  void* sc = nullptr;
  // kSellTail padding slots past the last slice let the products load whole
  // batches without bounds checks.
  const size_t alloc = (size_t)total + kSellTail;
  SLA_HIP(buf_alloc(&sv, es * alloc));
  owned3[0] = sv;
  SLA_HIP(buf_alloc(&sc, (rel16 ? 2 : 4) * alloc));
  owned3[1] = sc;
  SLA_HIP(hipMemsetAsync((char*)sv + es * (size_t)total, 0, es * kSellTail, s));
  if (rel16)
    SLA_HIP(hipMemsetD16Async((hipDeviceptr_t)((short*)sc + total), (unsigned short)kPad16,
                              kSellTail, s));
  else
    SLA_HIP(hipMemsetAsync((int*)sc + total, 0xff, 4 * (size_t)kSellTail, s));
  const int rows = nslices * kSlice;
  const dim3 g((rows + 255) / 256), b(256);
  if (dtype == SLA_F64 && rel16)
    hipLaunchKernelGGL((sell_fill<double, short>), g, b, 0, s, view.rp, view.ci,
                       (const double*)view.v, (int)n, nslices, (const int*)soff, (double*)sv,
                       (short*)sc);
  else if (dtype == SLA_F64)
    hipLaunchKernelGGL((sell_fill<double, int>), g, b, 0, s, view.rp, view.ci,
                       (const double*)view.v, (int)n, nslices, (const int*)soff, (double*)sv,
                       (int*)sc);
  else if (rel16)
    hipLaunchKernelGGL((sell_fill<float, short>), g, b, 0, s, view.rp, view.ci,
                       (const float*)view.v, (int)n, nslices, (const int*)soff, (float*)sv,
                       (short*)sc);
  else
    hipLaunchKernelGGL((sell_fill<float, int>), g, b, 0, s, view.rp, view.ci,
                       (const float*)view.v, (int)n, nslices, (const int*)soff, (float*)sv,
                       (int*)sc);
  SLA_HIP(hipGetLastError());
  view.sv = sv;
  view.sc = rel16 ? nullptr : (const int32_t*)sc;
  view.sd = rel16 ? (const int16_t*)sc : nullptr;
  view.soff = soff;
  view.nslices = nslices;
  view.sell_w = h[0];
  view.sell_slots = total;
  view.sell = true;
  return SLA_OK;
}

sla_status build_bsell(MatView& view, int64_t nbr, int64_t nnzb, int32_t dtype, void** owned3,
                       hipStream_t s) {
  view.sell = false;
  if (nbr == 0 || nnzb == 0) return SLA_OK;
  const int nslices = (int)((nbr + kBSlice - 1) / kBSlice);
  int* buf = nullptr;
  SLA_HIP(hipMallocAsync((void**)&buf, sizeof(int) * ((size_t)nslices + 3), s));
  int* slots = buf;            // nslices + 1 (last one zero)
  int* maxw = buf + nslices + 1;
  int* maxd = buf + nslices + 2;
  SLA_HIP(hipMemsetAsync(buf, 0, sizeof(int) * ((size_t)nslices + 3), s));
  hipLaunchKernelGGL(bsell_widths, dim3(std::min(256, (nslices + kWG - 1) / kWG)), dim3(kWG), 0,
                     s, view.rp, view.ci, (int)nbr, nslices, slots, maxw, maxd);
  SLA_HIP(hipGetLastError());
  int* soff = nullptr;
  SLA_HIP(buf_alloc((void**)&soff, sizeof(int) * ((size_t)nslices + 1)));
  owned3[2] = soff;
  sla_status st = exclusive_scan(slots, soff, nslices + 1, s);
  if (st != SLA_OK) return st;
  int h[3] = {0, 0, 0};
  SLA_HIP(hipMemcpyAsync(&h[0], maxw, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&h[1], soff + nslices, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipMemcpyAsync(&h[2], maxd, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipFreeAsync(buf, s));
  SLA_HIP(hipStreamSynchronize(s));
  if (!sliced_layout_fits(nslices, h[0], kBSlotVals, kBSellTail * kBSlotVals)) return SLA_OK;
  const int64_t total = h[1];  // slots
  if (h[0] > kBSellMaxWidth || total * kBSlice * 100 > nnzb * (100 + kSellMaxPadPct))
    return SLA_OK;
  if ((total + kBSellTail) * kBSlotVals >= (int64_t)INT32_MAX) return SLA_OK;
  const size_t es = dtype == SLA_F64 ? 8 : 4;
  const char* e16 = getenv("SLA_SELL16");
  const bool rel16 = h[2] <= 32767 && !(e16 && e16[0] == '0');
  const size_t cs = rel16 ? 2 : 4;
  // kBSellTail padding slots past the last slice let the products load whole
  // batches without bounds checks.
  const size_t alloc = (size_t)total + kBSellTail;
  void* sv = nullptr;
  void* sc = nullptr;
  SLA_HIP(buf_alloc(&sv, es * kBSlotVals * alloc));
  owned3[0] = sv;
  SLA_HIP(buf_alloc(&sc, cs * kBSlotCols * alloc));
  owned3[1] = sc;
  // every entry is defined: the fill writes the 189 used values and 21 used
  // columns of each slot, this clears the per-row and per-slot pads and the
  // tail slots (value 0, column padding)
  SLA_HIP(hipMemsetAsync(sv, 0, es * kBSlotVals * alloc, s));
  if (rel16)
    SLA_HIP(hipMemsetD16Async((hipDeviceptr_t)sc, (unsigned short)kPad16, kBSlotCols * alloc, s));
  else
    SLA_HIP(hipMemsetAsync(sc, 0xff, 4 * kBSlotCols * alloc, s));
  const int rows = nslices * kBSlice;
  const dim3 g((rows + 255) / 256), b(256);
  if (dtype == SLA_F64 && rel16)
    hipLaunchKernelGGL((bsell_fill<double, short>), g, b, 0, s, view.rp, view.ci,
                       (const double*)view.v, (int)nbr, nslices, (const int*)soff, (double*)sv,
                       (short*)sc);
  else if (dtype == SLA_F64)
    hipLaunchKernelGGL((bsell_fill<double, int>), g, b, 0, s, view.rp, view.ci,
                       (const double*)view.v, (int)nbr, nslices, (const int*)soff, (double*)sv,
                       (int*)sc);
  else if (rel16)
    hipLaunchKernelGGL((bsell_fill<float, short>), g, b, 0, s, view.rp, view.ci,
                       (const float*)view.v, (int)nbr, nslices, (const int*)soff, (float*)sv,
                       (short*)sc);
  else
    hipLaunchKernelGGL((bsell_fill<float, int>), g, b, 0, s, view.rp, view.ci,
                       (const float*)view.v, (int)nbr, nslices, (const int*)soff, (float*)sv,
                       (int*)sc);
  SLA_HIP(hipGetLastError());
  view.sv = sv;
  view.sc = rel16 ? nullptr : (const int32_t*)sc;
  view.sd = rel16 ? (const int16_t*)sc : nullptr;
  view.soff = soff;
  view.nslices = nslices;
  view.sell_w = h[0];
  view.sell = true;
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// Locality ordering (host side).
// ---------------------------------------------------------------------------

sla_status count_far_entries(const sla_mat& m, int samples, int near, int* far, hipStream_t s) {
  *far = 0;
  if (m.nnzb == 0 || samples <= 0) return SLA_OK;
  int* d = nullptr;
  SLA_HIP(hipMallocAsync((void**)&d, sizeof(int), s));
  SLA_HIP(hipMemsetAsync(d, 0, sizeof(int), s));
  hipLaunchKernelGGL(sample_far, dim3(grid_for(samples)), dim3(kWG), 0, s, m.fwd.rp, m.fwd.ci,
                     (int)m.nbr, (int)m.nnzb, samples, near, d);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipMemcpyAsync(far, d, sizeof(int), hipMemcpyDeviceToHost, s));
  SLA_HIP(hipFreeAsync(d, s));
  SLA_HIP(hipStreamSynchronize(s));
  return SLA_OK;
}

sla_status build_order(const sla_mat& m, int32_t** perm_out, int32_t** iperm_out,
                       hipStream_t s) {
  const int n = (int)m.nbr;
  int32_t *perm = nullptr, *iperm = nullptr;
  SLA_HIP(buf_alloc((void**)&perm, sizeof(int) * (size_t)std::max(1, n)));
  *perm_out = perm;
  SLA_HIP(buf_alloc((void**)&iperm, sizeof(int) * (size_t)std::max(1, n)));
  *iperm_out = iperm;
  if (n == 0) return SLA_OK;
  int* keys = nullptr;
  int* work = nullptr;
  SLA_HIP(hipMallocAsync((void**)&keys, sizeof(int) * (size_t)n, s));
  SLA_HIP(hipMallocAsync((void**)&work, sizeof(int) * radix_work_ints(n), s));
  hipLaunchKernelGGL(order_keys, dim3(grid_for(n)), dim3(kWG), 0, s, m.fwd.rp, n, keys);
  SLA_HIP(hipGetLastError());
  const int* srt = nullptr;
  sla_status st = radix_sort_indices(keys, n, kOrderKeyBits, work, &srt, s);
  if (st != SLA_OK) return st;
  SegStarts seg{};
  int acc = 0;
  for (int x = 0; x < 8; ++x) {
    seg.start[x] = acc;
    acc += x < n ? (n - x + 7) / 8 : 0;
  }
  hipLaunchKernelGGL(order_deal, dim3(grid_for(n)), dim3(kWG), 0, s, srt, n, seg, perm, iperm);
  SLA_HIP(hipGetLastError());
  SLA_HIP(hipFreeAsync(work, s));
  SLA_HIP(hipFreeAsync(keys, s));
  SLA_HIP(hipStreamSynchronize(s));
  return SLA_OK;
}

sla_status build_permuted(const sla_mat& m, const int32_t* perm, const int32_t* iperm,
                          int32_t** rp_out, int32_t** ci_out, void** v_out, hipStream_t s) {
  const int n = (int)m.nbr, nnz = (int)m.nnzb;
  const size_t es = m.dtype == SLA_F64 ? 8 : 4;
  int32_t *rp = nullptr, *ci = nullptr;
  void* v = nullptr;
  SLA_HIP(buf_alloc((void**)&rp, sizeof(int) * ((size_t)n + 1)));
  *rp_out = rp;
  SLA_HIP(buf_alloc((void**)&ci, sizeof(int) * (size_t)std::max(1, nnz)));
  *ci_out = ci;
  SLA_HIP(buf_alloc(&v, es * (size_t)std::max(1, nnz)));
  *v_out = v;
  int* len = nullptr;
  SLA_HIP(hipMallocAsync((void**)&len, sizeof(int) * ((size_t)n + 1), s));
  hipLaunchKernelGGL(perm_lengths, dim3(grid_for((int64_t)n + 1)), dim3(kWG), 0, s, m.fwd.rp,
                     perm, n, len);
  SLA_HIP(hipGetLastError());
  sla_status st = exclusive_scan(len, rp, n + 1, s);
  if (st != SLA_OK) return st;
  SLA_HIP(hipFreeAsync(len, s));
  if (nnz > 0) {
    if (m.dtype == SLA_F64)
      hipLaunchKernelGGL(perm_fill<double>, dim3(grid_for(nnz)), dim3(kWG), 0, s, m.fwd.rp,
                         m.fwd.ci, (const double*)m.fwd.v, (const int*)rp, perm, iperm, n, nnz,
                         ci, (double*)v);
    else
      hipLaunchKernelGGL(perm_fill<float>, dim3(grid_for(nnz)), dim3(kWG), 0, s, m.fwd.rp,
                         m.fwd.ci, (const float*)m.fwd.v, (const int*)rp, perm, iperm, n, nnz,
                         ci, (float*)v);
    SLA_HIP(hipGetLastError());
  }
  SLA_HIP(hipStreamSynchronize(s));
  return SLA_OK;
}

sla_status permute_rows(const int32_t* perm, const void* src, void* dst, int64_t n, int cols,
                        int32_t dtype, bool into, hipStream_t s) {
  if (n == 0 || cols == 0) return SLA_OK;
  const int g = grid_for(n * cols);
  if (dtype == SLA_F64)
    hipLaunchKernelGGL(permute_rows_k<double>, dim3(g), dim3(kWG), 0, s, perm,
                       (const double*)src, (double*)dst, (int)n, cols, into);
  else
    hipLaunchKernelGGL(permute_rows_k<float>, dim3(g), dim3(kWG), 0, s, perm, (const float*)src,
                       (float*)dst, (int)n, cols, into);
  SLA_HIP(hipGetLastError());
  return SLA_OK;
}

}  // namespace sla
