// moe_unpermute_combine: y[t] = sum_j w[t,j] * y_perm[slot_of[t,j]] (+ gate[t] * y_shared[t])
//
// Passage: "Megatron-Bridge 深度剖析", section "Expert Parallel 基础", step 3
// (expert results return to the tokens' original layout) and section
// "Shared Expert Overlap" (the shared expert's output joins the routed one).
//
// One wavefront per token; each lane owns 16-byte column chunks.  The k rows
// are summed in fp32 in slot order j = 0..k-1, the shared row is added last,
// and the result is rounded to the storage type once.  Memory-bound: every
// byte of y_perm is read exactly once, y once written.
#include "moe_gemm_common.h"

namespace moe {

constexpr int kCombThreads = 256;

// kMaxK >= k: the k row loads of kU column chunks per lane are issued
// together (one round trip for up to kU KB of every row); each chunk's sum
// still runs in slot order.  The loads are raw buffer loads with one
// descriptor per row (the row's bytes, or none for a dropped choice), so a
// chunk past the row or a missing row reads zero without a branch around
// the load, and all of them leave before the first wait.  y is written with
// non-temporal stores (this pass does not read it back).
template <bool kBF16, int kMaxK, int kU>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(
    int T, int k, int N, int nchunk16, const u32x4* __restrict__ y_perm,
    const int32_t* __restrict__ slot_of, const float* __restrict__ topk_w,
    const u32x4* __restrict__ y_shared, const float* __restrict__ shared_gate,
    u32x4* __restrict__ y) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kCombThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  int my_row = -1;
  float my_w = 1.0f;
  if (lane < k) {
    my_row = slot_of[static_cast<size_t>(t) * k + lane];
    if (my_row >= N) my_row = -1;
    if (topk_w) my_w = topk_w[static_cast<size_t>(t) * k + lane];
  }
  const int row_bytes = nchunk16 * 16;
  // every lane holds all k rows and weights (wave-uniform)
  __amdgpu_buffer_rsrc_t rs[kMaxK];
  bool has[kMaxK];
  float wj[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    const int row = j < k ? __builtin_amdgcn_readfirstlane(__shfl(my_row, j, kWave)) : -1;
    has[j] = row >= 0;
    rs[j] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(y_perm + static_cast<size_t>(has[j] ? row : 0) * nchunk16), 0,
        has[j] ? row_bytes : 0, kRsrcWord3);
    wj[j] = j < k ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                        __builtin_bit_cast(int, __shfl(my_w, j, kWave))))
                  : 0.0f;
  }
  const float g = (y_shared && shared_gate) ? shared_gate[t] : 1.0f;
  const bool sh = y_shared != nullptr;
  const __amdgpu_buffer_rsrc_t rsh = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(sh ? y_shared + static_cast<size_t>(t) * nchunk16 : y_perm), 0,
      sh ? row_bytes : 0, kRsrcWord3);
  constexpr int kVals = kBF16 ? 8 : 4;
  constexpr int kNt = 2;   // cache policy: non-temporal
  for (int c0 = lane; c0 < nchunk16; c0 += 64 * kU) {
    u32x4 v[kU][kMaxK], vs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int off = (c0 + 64 * u) * 16;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        v[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs[j], off, 0, kNt));
      if (sh) vs[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsh, off, 0, kNt));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = c0 + 64 * u;
      float acc[kVals];
#pragma unroll
      for (int q = 0; q < kVals; ++q) acc[q] = 0.0f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (!has[j]) continue;                    // wave-uniform
        if constexpr (kBF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(wj[j], bf16lo(v[u][j][q]), acc[2 * q]);
            acc[2 * q + 1] = fmaf(wj[j], bf16hi(v[u][j][q]), acc[2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(wj[j], __uint_as_float(v[u][j][q]), acc[q]);
        }
      }
      if (sh) {
        if constexpr (kBF16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[2 * q] = fmaf(g, bf16lo(vs[u][q]), acc[2 * q]);
            acc[2 * q + 1] = fmaf(g, bf16hi(vs[u][q]), acc[2 * q + 1]);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[q] = fmaf(g, __uint_as_float(vs[u][q]), acc[q]);
        }
      }
      u32x4 o;
      if constexpr (kBF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = __float_as_uint(acc[q]);
      }
      if (c < nchunk16) __builtin_nontemporal_store(o, y + static_cast<size_t>(t) * nchunk16 + c);
    }
  }
}

template <bool kBF16>
static auto pick_combine(int k) {
  // kU * kMaxK <= 32 row chunks in flight per lane (<= 128 VGPRs of loads);
  // for k <= 8, 2 chunks per lane (16 loads, 64 VGPRs) keep more wavefronts
  // resident than 4 (A/B, warm: c3 58.2 -> 56.2 us, c4 125.3 -> 121.7 us,
  // c2 unchanged)
  if (k <= 2) return combine_kernel<kBF16, 2, 4>;
  if (k <= 4) return combine_kernel<kBF16, 4, 4>;
  if (k <= 8) return combine_kernel<kBF16, 8, 2>;
  if (k <= 16) return combine_kernel<kBF16, 16, 2>;
  return combine_kernel<kBF16, 32, 1>;
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_unpermute_combine(hipStream_t stream, moe_dtype dt, int64_t T,
                                            int64_t d, int32_t k, int64_t N,
                                            const void* y_perm, const int32_t* slot_of,
                                            const float* topk_w, const void* y_shared,
                                            const float* shared_gate, void* y) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!y_perm || !slot_of || !y || (shared_gate && !y_shared)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || k < 1 || k > 32 || N < 0 || N >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  const size_t row_bytes = static_cast<size_t>(d) * elt_size(dt);
  if (row_bytes % 16) return MOE_ERR_ALIGNMENT;
  if (!aligned16(y_perm) || !aligned16(slot_of) || !aligned16(topk_w) || !aligned16(y_shared) ||
      !aligned16(shared_gate) || !aligned16(y))
    return MOE_ERR_ALIGNMENT;
  auto kern = dt == MOE_BF16 ? pick_combine<true>(k) : pick_combine<false>(k);
  return hip_status(launch(kern, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(kCombThreads), 0,
                           stream, (int)T, k, (int)N, static_cast<int>(row_bytes / 16),
                           static_cast<const u32x4*>(y_perm), slot_of, topk_w,
                           static_cast<const u32x4*>(y_shared), shared_gate,
                           static_cast<u32x4*>(y)));
}
