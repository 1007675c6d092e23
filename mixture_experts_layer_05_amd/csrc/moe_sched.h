// Dynamic tile fetch for the persistent grouped GEMMs.
//
// A grouped GEMM over ragged expert segments has tiles of unequal cost (an
// expert's n rows are split over ceil(n / bm) row tiles of equal height, so
// heights differ between experts) and the tiles do not divide evenly over
// the workgroups.  The tiles are split into 8 contiguous ranges, one per XCD
// (workgroup b runs on XCD b mod 8, and tiles that share an expert's weight
// panel or token rows are neighbours, so they share that XCD's L2); within a
// range, each workgroup takes its first two tiles by position and then
// fetches the next from the XCD's per-launch counter, so workgroups that drew
// cheap tiles take more of them.
#pragma once

#include "moe_gemm_common.h"

namespace moe {

// This workgroup's share of the tiles: XCD range [xbeg, xbeg + xcnt).
struct XcdRange {
  int xbeg, xcnt;
};
__device__ __forceinline__ XcdRange xcd_range(int total, int xcd) {
  const int q = total >> 3, rq = total & 7;
  return {xcd * q + min(xcd, rq), q + (xcd < rq ? 1 : 0)};
}

// Zeroes n per-launch tile counters with a kernel (not a memset node, so that
// the call can be captured in a graph).
hipError_t launch_zero_counters(hipStream_t stream, int* c, int n);

}  // namespace moe
