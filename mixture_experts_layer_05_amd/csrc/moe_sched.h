// Tile order and dynamic tile fetch for the persistent grouped GEMMs.
//
// A grouped GEMM over ragged expert segments has tiles of unequal cost: an
// expert's n rows are split over ceil(n / bm) row tiles of equal height, so
// tile heights (in 32-row blocks) differ between experts, and the tiles do
// not divide evenly over the workgroups.  With a static round-robin split the
// workgroups that draw one tile more, or the taller tiles, finish last.
// Here the experts are dealt to the XCDs by cost, and within an XCD every
// workgroup fetches its next tile from the XCD's per-launch counter, the
// costliest experts' tiles first, so the cheapest tiles come last and fill
// the gaps.
#pragma once

#include "moe_gemm_common.h"

namespace moe {

// Blocks of 32 rows in each row tile of an expert with n rows (0 for n = 0).
__device__ __forceinline__ int tile_blocks(int n, int bm) {
  if (n <= 0) return 0;
  const int mts = (n + bm - 1) / bm;
  return ((n + mts - 1) / mts + 31) >> 5;
}

// The tiles of one XCD.  Workgroup b runs on XCD b mod 8, and the XCDs do
// not share an L2, so an expert's tiles (which share its weight panels and,
// in fc2, its token rows) stay on one XCD: the experts are sorted by cost
// (tiles x row blocks, descending; ties in expert order) and dealt to the 8
// XCDs in snake order (0..7, 7..0, ...), which balances the XCDs.  Within
// XCD x the order is that of its experts, each expert's tiles column tiles
// outer, row tiles inner.
//   s_perm[i]    the expert at position i of the global cost order
//   s_cum[k]     tiles before the XCD's k-th expert, k = 0 .. nx (s_cum[nx]: all)
//   returns nx, the XCD's expert count
// s_key holds E ints of scratch.  Every thread of the workgroup calls it; it
// ends with a barrier.
template <int kThreads>
__device__ inline int tile_order_xcd(const int32_t* __restrict__ offsets, int E, int bm, int ntn,
                                     int xcd, int* s_cum, int* s_perm, int* s_key, int* s_tmp) {
  constexpr int kPer = (1024 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = tid * kPer + q;
    if (e < E) {
      const int n = offsets[e + 1] - offsets[e];
      s_key[e] = (n > 0 ? (n + bm - 1) / bm : 0) * ntn * tile_blocks(n, bm);
    }
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = tid * kPer + q;
    if (e < E) {
      const int c = s_key[e];
      int r = 0;
      for (int e2 = 0; e2 < E; ++e2) {           // LDS broadcast reads
        const int c2 = s_key[e2];
        r += (c2 > c || (c2 == c && e2 < e)) ? 1 : 0;
      }
      s_perm[r] = e;
    }
  }
  __syncthreads();
  // the XCD's k-th expert sits at global position 8 k + (k even ? x : 7 - x)
  const int nx = E / 8 + ((E % 8) > (((E / 8) & 1) ? 7 - xcd : xcd) ? 1 : 0);
  int loc[kPer], sum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int k = tid * kPer + q;
    int t = 0;
    if (k < nx) {
      const int e = s_perm[8 * k + ((k & 1) ? 7 - xcd : xcd)];
      const int n = offsets[e + 1] - offsets[e];
      t = (n > 0 ? (n + bm - 1) / bm : 0) * ntn;
    }
    loc[q] = t;
    sum += t;
  }
  const int lane = tid & 63, wave = tid >> 6;
  int v = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_tmp[w];
  int run = v + add - sum;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int k = tid * kPer + q;
    if (k <= nx) s_cum[k] = run;                 // s_cum[nx] from the thread holding k = nx
    run += loc[q];
  }
  __syncthreads();
  return nx;
}

// Tile L of XCD x's order -> (expert, row tile, column tile); the row split
// is that of tile_decode.
__device__ inline TileIdx tile_decode_xcd(const int32_t* __restrict__ offsets, int nx, int xcd,
                                          int bm, int L, const int* s_cum, const int* s_perm) {
  int lo = 0, hi = nx - 1;
  while (lo < hi) {  // largest k with s_cum[k] <= L (that expert is non-empty)
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= L) lo = mid; else hi = mid - 1;
  }
  TileIdx t;
  t.e = s_perm[8 * lo + ((lo & 1) ? 7 - xcd : xcd)];
  t.lo = offsets[t.e];
  t.hi = offsets[t.e + 1];
  const int n = t.hi - t.lo;
  const int mts = (n + bm - 1) / bm;
  const int local = L - s_cum[lo];
  t.nt = local / mts;
  t.mt = local - t.nt * mts;
  const int h = ((n + mts - 1) / mts + 31) & ~31;
  t.m0 = t.lo + t.mt * h;
  t.mend = min(t.m0 + h, t.hi);
  return t;
}

// Zeroes n per-launch tile counters with a kernel (not a memset node, so that
// the call can be captured in a graph).
hipError_t launch_zero_counters(hipStream_t stream, int* c, int n);

}  // namespace moe
