// Tile enumeration over ragged expert segments, shared by the grouped-GEMM
// kernels.  Tiles are listed per expert (experts in order), column tiles
// outer, row tiles inner, and found on the device from expert_offsets, so
// no host synchronisation is needed.
#pragma once

#include "moe_internal.h"

namespace moe {

struct TileIdx {
  int e, mt, nt;
  int lo, hi;      // the expert's segment
  int m0, mend;    // this tile's rows
};

// Block-wide exclusive scan over the experts' tile counts, into s_cum[0..E]
// (s_cum[E] = total).  E <= 1024, blockDim.x == kThreads (a multiple of 64,
// at most 1024).  Every thread of the block must call it.
template <int kThreads>
__device__ inline void tile_prefix(const int32_t* __restrict__ offsets, int E, int bm, int ntn,
                                   int* s_cum, int* s_tmp) {
  constexpr int kPer = (1024 + kThreads - 1) / kThreads;
  const int tid = threadIdx.x;
  int loc[kPer], sum = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = tid * kPer + q;
    int t = 0;
    if (e < E) {
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
    const int e = tid * kPer + q;
    if (e < E) s_cum[e] = run;
    run += loc[q];
  }
  if (tid == kThreads - 1) s_cum[E] = v + add;
  __syncthreads();
}

// Workgroups are handed to the 8 XCDs round-robin (block b -> XCD b % 8).
// Give each XCD a contiguous range of logical tiles instead, so the row
// tiles that share one expert's weight panel run at the same time on the
// same XCD and share its L2.  Bijective on [0, total).
__device__ inline int xcd_remap(int b, int total) {
  const int x = b & 7, pos = b >> 3;
  const int q = total >> 3, r = total & 7;
  return x * q + (x < r ? x : r) + pos;
}

// logical tile -> (expert, row tile, column tile) given s_cum from tile_prefix.
// An expert's n rows are split over ceil(n / bm) row tiles of equal height
// h = ceil(n / tiles) rounded up to 32 (h <= bm, every tile non-empty), e.g.
// 260 rows at bm = 128 as 96 + 96 + 68 rather than 128 + 128 + 4.  An
// expert's tiles are consecutive: column tiles outer and row tiles inner
// (the row tiles of one weight panel run together and share it in L2), or,
// for an expert with more row tiles than column tiles (a heavily routed one),
// row tiles outer and column tiles inner, so that each row tile's token rows
// are read by its ntn column tiles together instead of once per pass over
// the expert's row tiles.
__device__ inline TileIdx tile_decode(const int32_t* __restrict__ offsets, int E, int bm, int ntn,
                                      int L, const int* s_cum) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {  // largest e with s_cum[e] <= L (that expert is non-empty)
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= L) lo = mid; else hi = mid - 1;
  }
  TileIdx t;
  t.e = lo;
  t.lo = offsets[lo];
  t.hi = offsets[lo + 1];
  const int n = t.hi - t.lo;
  const int mts = (n + bm - 1) / bm;
  const int local = L - s_cum[lo];
  if (mts > ntn) {
    t.mt = local / ntn;
    t.nt = local - t.mt * ntn;
  } else {
    t.nt = local / mts;
    t.mt = local - t.nt * mts;
  }
  const int h = ((n + mts - 1) / mts + 31) & ~31;
  t.m0 = t.lo + t.mt * h;
  t.mend = min(t.m0 + h, t.hi);
  return t;
}

// The same decode for a single group of n rows (no offsets array), row tiles
// outer: the ntn column tiles of a row tile are neighbours, so they run on
// one XCD together and read its token rows from one L2 (the router's weight
// is small and stays in every L2).
__device__ inline TileIdx tile_decode_one(int n, int bm, int ntn, int L) {
  TileIdx t;
  t.e = 0;
  t.lo = 0;
  t.hi = n;
  const int mts = (n + bm - 1) / bm;
  t.mt = L / ntn;
  t.nt = L - t.mt * ntn;
  const int h = ((n + mts - 1) / mts + 31) & ~31;
  t.m0 = t.mt * h;
  t.mend = min(t.m0 + h, n);
  return t;
}

typedef __attribute__((address_space(3))) void lds_void;

constexpr unsigned kRsrcWord3 = 0x00020000u;  // raw buffer, 32-bit data format
constexpr int kOob = 0x7fff0000;              // offset past any buffer: reads zero

// Row-layout staging (K contiguous): a staged row holds 32 k = 4 chunks of
// 16 bytes; chunk kc of row r sits at position kc ^ swz_f(r).  The MFMA
// operand read (16 consecutive rows, one chunk per lane) and the 1 KB
// direct-to-LDS block writes are then free of bank conflicts.
__device__ __forceinline__ int swz_f(int r) {
  return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// Raw buffer descriptor words: base address, num_records bytes, 32-bit data
// format; offsets at or past num_records read zero.
__device__ __forceinline__ i32x4 buf_desc(const void* base, int num_records) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{static_cast<int>(a), static_cast<int>((a >> 32) & 0xffff), num_records,
               static_cast<int>(kRsrcWord3)};
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)(const_cast<void*>(p)))));
}

// 16 bytes per lane from buffer offset voff + soff into LDS at dst + 16 lane
// (dst uniform).  Inline asm, so the compiler does not track it as an LDS
// write (it would otherwise wait for every load in flight before LDS reads
// it cannot tell apart from the slot being filled); callers order it with
// their own s_waitcnt vmcnt + s_barrier, which clobber memory.
__device__ __forceinline__ void dma16(const i32x4& desc, const void* dst, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(dst)), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

// 4 bytes per lane into LDS at dst + 4 lane: one cache line per lane, used
// to pull operand lines into L2 ahead of the 16-byte-per-lane loads (the
// LDS bytes written are never read).
__device__ __forceinline__ void dma4(const i32x4& desc, const void* dst, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(lds_addr(dst)), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

inline int tiles_bound(int64_t N, int E, int bm) {
  return static_cast<int>((N + bm - 1) / bm + E);
}

// Forward launcher shared with the backward's recompute path.  bf16 only.
// a_buf [N, F] receives silu(G) * U; gu_save (or NULL) receives [G | U];
// when run_fc2, y_perm = (a_buf W2^T) * row_scale.  With gather (or NULL),
// row r of the first GEMM is row gather[r] of x_perm [a_rows, d].
hipError_t launch_grouped_fwd_bf16(hipStream_t stream, int64_t N, int64_t d, int64_t F, int32_t E,
                                   const void* x_perm, const void* w1, const void* w2,
                                   const int32_t* offsets, const float* row_scale, void* y_perm,
                                   void* gu_save, uint16_t* a_buf, bool run_fc2,
                                   const int32_t* gather = nullptr, int64_t a_rows = 0,
                                   bool packed = false);

// Router logits with the forward kernel as a one-group GEMM, K split into
// `ksplit` slabs: logits[s][T][E] = x[:, slab s] W_r[:, slab s]^T (+ bias
// on slab 0), fp32.  bf16 only.
int router_ksplit(int64_t T, int64_t d, int32_t E);
// With gate_w ([d] shared-gate weights), also gate_out[s][T] = x[:, slab s]
// . gate_w[slab s] (fp32), when router_gate_fused(T, d, E) (the slab's gate
// weights fit in LDS beside the rings).  zero_counts: E ints set to zero
// (for the top-k kernel that follows), or NULL.
bool router_gate_fused(int64_t T, int64_t d, int32_t E);
hipError_t launch_router_logits_bf16(hipStream_t stream, int64_t T, int64_t d, int32_t E,
                                    const void* x, const void* w_router, const float* bias,
                                    float* logits, int ksplit, const void* gate_w = nullptr,
                                    float* gate_out = nullptr, int32_t* zero_counts = nullptr);

}  // namespace moe
