// moe_permute: stable counting sort of the (token, slot) pairs by expert and
// the row gather x -> x_perm.
//
// Passage: "Megatron-Bridge 深度剖析", section "Expert Parallel 基础", step 2
// (after dispatch the tokens sit grouped by expert) and section "Permute
// Fusion" (the permute is a memory copy of the hidden states).
//
// Pairs are taken token-major (pair p = t*k + j) and cut into blocks of 64
// tokens (the blocks of moe_route's histogram rows).  Row of a pair with
// expert e in block b:
//     off[e] + sum_{b' < b} H[b'][e] + #{earlier pairs of block b with e}
// which is exactly the stable order (expert, token, slot).  No atomics
// decide an order, so the result is deterministic.
//   K1 hist    : H[b][e] per block (LDS histogram); skipped when the caller
//                passes moe_route's block histograms
//   K2 colscan : per expert, exclusive scan of H[.][e] over blocks; total
//                count per expert
//   K3 rows    : every block rebuilds off[] from the totals (LDS scan),
//                ranks its pairs, writes slot_of / row_token / row_w.  The
//                rank of a pair is the number of earlier tokens of the block
//                that chose the same expert: a 64-bit mask of the block's
//                tokens per expert (LDS atomic OR, order-free) and a
//                popcount below the token.  A block where a token names one
//                expert twice ranks by counting earlier pairs instead.
//   K4 copy    : one wavefront per token reads x[t] once (16-byte lanes)
//                and writes it to its k rows
#include <mutex>

#include "moe_internal.h"

namespace moe {

constexpr int kPermThreads = 256;
constexpr int kPermRow = MOE_ROUTE_BLOCK_TOKENS;   // tokens per histogram row
constexpr int kPermBlk = 64;                       // tokens per ranking block (a 64-bit mask)
constexpr int kRowsPerBlk = kPermBlk / kPermRow;
constexpr int kPermMaxPairs = kPermBlk * 32;       // k <= 32
static_assert(kPermBlk % kPermRow == 0, "rows tile the blocks");

// inclusive scan of one value per thread over a 256-thread block
__device__ inline int block_incl_scan(int v, int* s_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == 63) s_tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += s_tmp[w];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(kPermThreads) void perm_hist_kernel(
    int T, int E, int k, const int32_t* __restrict__ topk_idx, int32_t* __restrict__ H) {
  extern __shared__ int s_cnt[];
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPermRow * k;
  const int64_t pend = min(static_cast<int64_t>(T) * k, p0 + static_cast<int64_t>(kPermRow) * k);
  for (int e = threadIdx.x; e < E; e += kPermThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int64_t p = p0 + threadIdx.x; p < pend; p += kPermThreads) {
    const int e = topk_idx[p];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  int32_t* hrow = H + static_cast<size_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kPermThreads) hrow[e] = s_cnt[e];
}

// one block per expert: exclusive scan of column e of H over the blocks
// (dst may equal src)
__global__ __launch_bounds__(kPermThreads) void perm_colscan_kernel(
    int nblk, int E, const int32_t* src, int32_t* dst, int32_t* __restrict__ total) {
  __shared__ int s_tmp[4];
  __shared__ int s_last;
  const int e = blockIdx.x;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += kPermThreads) {
    const int b = b0 + threadIdx.x;
    const int v = b < nblk ? src[static_cast<size_t>(b) * E + e] : 0;
    const int inc = block_incl_scan(v, s_tmp);
    if (b < nblk) dst[static_cast<size_t>(b) * E + e] = carry + inc - v;
    if (threadIdx.x == kPermThreads - 1) s_last = inc;   // chunk total
    __syncthreads();
    carry += s_last;
    __syncthreads();
  }
  if (threadIdx.x == 0) total[e] = carry;
}

__global__ __launch_bounds__(kPermThreads) void perm_rows_kernel(
    int T, int E, int k, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const int32_t* __restrict__ H,
    const int32_t* __restrict__ total, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ slot_of, int32_t* __restrict__ row_token,
    float* __restrict__ row_w) {
  extern __shared__ __align__(8) int smem[];
  unsigned long long* s_mask = reinterpret_cast<unsigned long long*>(smem);   // [E]
  int* s_off = smem + 2 * E;                                                  // [E + 1]
  int* s_e = s_off + E + 1;                                                   // [64 k]
  __shared__ int s_tmp[4];
  __shared__ int s_dup;
  const int tid = threadIdx.x;

  // off[] = exclusive scan of the per-expert totals (each thread 4 experts)
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    loc[q] = e < E ? total[e] : 0;
    sum += loc[q];
  }
  const int incl = block_incl_scan(sum, s_tmp);
  int run = incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < E) s_off[e] = run;
    run += loc[q];
  }
  if (tid == kPermThreads - 1) s_off[E] = incl;
  for (int e = tid; e < E; e += kPermThreads) s_mask[e] = 0ull;
  if (tid == 0) s_dup = 0;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int e = tid; e <= E; e += kPermThreads) expert_offsets[e] = s_off[e];

  // the block's pairs: expert of each (-1: dropped) and each expert's tokens
  const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPermBlk * k;
  const int np = static_cast<int>(min(static_cast<int64_t>(T) * k - p0,
                                      static_cast<int64_t>(kPermBlk) * k));
  for (int i = tid; i < np; i += kPermThreads) {
    int e = topk_idx[p0 + i];
    if (e < 0 || e >= E) e = -1;
    s_e[i] = e;
    if (e >= 0) {
      const unsigned long long bit = 1ull << (i / k);
      if (atomicOr(&s_mask[e], bit) & bit) s_dup = 1;   // a token names e twice
    }
  }
  __syncthreads();
  const bool dup = s_dup != 0;
  const int32_t* hrow = H + static_cast<size_t>(blockIdx.x) * kRowsPerBlk * E;   // its first row
  for (int i = tid; i < np; i += kPermThreads) {
    const int64_t p = p0 + i;
    const int e = s_e[i];
    if (e < 0) {
      slot_of[p] = -1;
      continue;
    }
    int rank = 0;
    if (!dup) {
      rank = __popcll(s_mask[e] & ((1ull << (i / k)) - 1ull));
    } else {
      for (int q = 0; q < i; ++q) rank += (s_e[q] == e);
    }
    const int row = s_off[e] + hrow[e] + rank;
    slot_of[p] = row;
    row_token[row] = static_cast<int>(p / k);
    if (row_w) row_w[row] = topk_w[p];
  }
}

// one wavefront per token: read the row once, write it to its k rows
__global__ __launch_bounds__(kPermThreads) void perm_copy_kernel(
    int T, int k, int nchunk16, const int32_t* __restrict__ slot_of,
    const u32x4* __restrict__ x, u32x4* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kPermThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int my_row = lane < k ? slot_of[static_cast<size_t>(t) * k + lane] : -1;
  const u32x4* src = x + static_cast<size_t>(t) * nchunk16;
  for (int c0 = 0; c0 < nchunk16; c0 += 64 * 4) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = c0 + i * 64 + lane;
      if (c < nchunk16) v[i] = src[c];
    }
    for (int j = 0; j < k; ++j) {
      const int row = __shfl(my_row, j, kWave);
      if (row < 0) continue;
      u32x4* dst = x_perm + static_cast<size_t>(row) * nchunk16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int c = c0 + i * 64 + lane;
        if (c < nchunk16) dst[c] = v[i];
      }
    }
  }
}

// Scratch of moe_permute_noalloc: the per-block expert histograms and the
// per-expert totals of moe_permute, in a file-scope device array (each GPU
// the library runs on holds one copy until the process ends).
constexpr size_t kPermScratchInts = size_t(1) << 20;          // 4 MiB
static __device__ __align__(256) int32_t scratch[kPermScratchInts];

// The device address of `scratch` on the current device, looked up once per
// device (with that device current); NULL if the lookup fails.  In host code
// the array's name is only a host-side stand-in for the symbol: kernels,
// copies and memsets must be given this address instead.
static void* perm_scratch_ptr() {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static void* ptr[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) ptr[dev] = p;
  });
  return ptr[dev];
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_permute_workspace_size(int64_t T, int32_t E, int32_t k) {
  if (T < 1 || E < 1 || k < 1) return 0;
  const int64_t nrow = (T + kPermRow - 1) / kPermRow;
  return static_cast<size_t>((nrow * E + E) * sizeof(int32_t) + 256);
}

extern "C" moe_status moe_permute(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                                  int32_t E, int32_t k, const void* x,
                                  const int32_t* topk_idx, const float* topk_w,
                                  const int32_t* block_counts,
                                  int32_t* expert_offsets, int32_t* slot_of,
                                  int32_t* row_token, float* row_w, void* x_perm,
                                  void* ws, size_t ws_bytes) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!topk_idx || !expert_offsets || !slot_of || !row_token || (x_perm && !x))
    return MOE_ERR_INVALID_ARG;
  if ((topk_w == nullptr) != (row_w == nullptr)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || E < 1 || E > 1024 || k < 1 || k > 32) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  const size_t row_bytes = static_cast<size_t>(d) * elt_size(dt);
  if (row_bytes % 16) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(x_perm) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      !aligned16(expert_offsets) || !aligned16(slot_of) || !aligned16(row_token) ||
      !aligned16(row_w) || !aligned16(block_counts) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_permute_workspace_size(T, E, k)) return MOE_ERR_WORKSPACE;

  const int nrow = static_cast<int>((T + kPermRow - 1) / kPermRow);
  const int nblk = static_cast<int>((T + kPermBlk - 1) / kPermBlk);
  int32_t* H = static_cast<int32_t*>(ws);
  int32_t* total = H + static_cast<size_t>(nrow) * E;

  hipError_t err = hipSuccess;
  if (!block_counts)
    err = launch(perm_hist_kernel, dim3(nrow), dim3(kPermThreads), E * sizeof(int), stream, (int)T,
                 E, k, topk_idx, H);
  if (err == hipSuccess)
    err = launch(perm_colscan_kernel, dim3(E), dim3(kPermThreads), 0, stream, nrow, E,
                 block_counts ? block_counts : static_cast<const int32_t*>(H), H, total);
  if (err == hipSuccess)
    err = launch(perm_rows_kernel, dim3(nblk), dim3(kPermThreads),
                 (3 * E + 1 + kPermMaxPairs) * sizeof(int), stream, (int)T, E, k, topk_idx,
                 topk_w, (const int32_t*)H, (const int32_t*)total, expert_offsets, slot_of,
                 row_token, row_w);
  if (err == hipSuccess && x_perm)   // NULL x_perm: the consumer gathers rows by row_token
    err = launch(perm_copy_kernel, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(kPermThreads),
                 0, stream, (int)T, k, static_cast<int>(row_bytes / 16), slot_of,
                 static_cast<const u32x4*>(x), static_cast<u32x4*>(x_perm));
  return hip_status(err);
}

extern "C" moe_status moe_permute_noalloc(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                                          int32_t E, int32_t k, const void* x,
                                          const int32_t* topk_idx, const float* topk_w,
                                          int32_t* expert_offsets, int32_t* slot_of,
                                          int32_t* row_token, float* row_w, void* x_perm) {
  // the shape checks of moe_permute come first (its size function returns 0
  // for shapes it rejects)
  if (T < 1 || E < 1 || E > 1024 || k < 1 || k > 32) return MOE_ERR_SHAPE;
  if (moe_permute_workspace_size(T, E, k) > kPermScratchInts * sizeof(int32_t))
    return MOE_ERR_WORKSPACE;   // more scratch than the static array holds
  void* ws = perm_scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  return moe_permute(stream, dt, T, d, E, k, x, topk_idx, topk_w, nullptr, expert_offsets,
                     slot_of, row_token, row_w, x_perm, ws, kPermScratchInts * sizeof(int32_t));
}
