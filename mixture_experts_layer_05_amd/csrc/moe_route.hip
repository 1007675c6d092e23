// moe_route: router logits (bf16 MFMA or fp32 FMA), score function,
// wavefront top-k, weight normalisation, per-expert counts, shared gate.
//
// Passage: "Megatron-Bridge 深度剖析", section "MoE 加速深度剖析 / Expert
// Parallel 基础", step 1 of the diagram: the router turns each token into
// its top-k experts with scores (top-6 sigmoid in the example); the score
// function is a TransformerConfig choice (section "Megatron-Core 架构速览").
//
// One workgroup = 4 wavefronts = kRouteTM tokens.
//   phase 1: logits tile z[kRouteTM][E] into LDS.  bf16: each wave owns
//            32-expert column blocks and runs v_mfma_f32_32x32x16_bf16 over d
//            with operands loaded straight from global memory (64 contiguous
//            bytes per lane per step).  fp32: one dot product per thread.
//   phase 2: each wave takes tokens in turn; lane l holds the scores of
//            experts l, l+64, ...; k rounds of a wave-wide arg-max (ties to
//            the lower expert index) pick the experts in descending order.
//   phase 3: the block's LDS histogram is added to the global counts with
//            integer atomics (order-independent, so deterministic).
#include "moe_internal.h"

namespace moe {

constexpr int kRouteTM = 32;
constexpr int kRouteThreads = 256;

__global__ void zero_i32_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

template <bool kBF16>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int T, int d, int E, int k, int score_fn, int normalize,
    const void* __restrict__ xv, const void* __restrict__ wrv,
    const float* __restrict__ bias, const void* __restrict__ wgv,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, float* __restrict__ gate) {
  extern __shared__ float smem[];
  const int ldz = E + 1;
  float* s_z = smem;                                  // [kRouteTM][E+1]
  int* s_cnt = reinterpret_cast<int*>(smem + kRouteTM * ldz);  // [E]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t0 = blockIdx.x * kRouteTM;

  for (int e = tid; e < E; e += kRouteThreads) s_cnt[e] = 0;

  // ---------------- phase 1: logits -------------------------------------
  if constexpr (kBF16) {
    const uint16_t* x = static_cast<const uint16_t*>(xv);
    const uint16_t* wr = static_cast<const uint16_t*>(wrv);
    const int h = lane >> 5;          // which half of the 16-wide k step
    const int r32 = lane & 31;
    int trow = t0 + r32;
    if (trow >= T) trow = T - 1;      // clamped rows are computed, not stored
    const uint16_t* xrow = x + static_cast<size_t>(trow) * d;
    const int ncb = (E + 31) / 32;
    for (int cb = wave; cb < ncb; cb += 4) {
      int erow = cb * 32 + r32;
      const bool evalid = erow < E;
      const uint16_t* wrow = wr + static_cast<size_t>(evalid ? erow : 0) * d;
      f32x16 acc = {};
      for (int kc = 0; kc < d; kc += 64) {
        bf16x8 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k8 = kc + 32 * h + 8 * i;
          if (k8 < d) {
            a[i] = *reinterpret_cast<const bf16x8*>(xrow + k8);
            b[i] = evalid ? *reinterpret_cast<const bf16x8*>(wrow + k8) : bf16x8{};
          } else {
            a[i] = bf16x8{};
            b[i] = bf16x8{};
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i], acc, 0, 0, 0);
      }
      // accumulator r of lane l holds C[row][col], col = l % 32,
      // row = 8*(r/4) + 4*(l/32) + r%4
      if (evalid) {
        const float bb = bias ? bias[erow] : 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * h + (r & 3);
          s_z[row * ldz + erow] = acc[r] + bb;
        }
      }
    }
  } else {
    const float* x = static_cast<const float*>(xv);
    const float* wr = static_cast<const float*>(wrv);
    for (int idx = tid; idx < kRouteTM * E; idx += kRouteThreads) {
      const int tl = idx / E, e = idx - tl * E;
      int trow = t0 + tl;
      if (trow >= T) trow = T - 1;
      const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(trow) * d);
      const float4* wrr = reinterpret_cast<const float4*>(wr + static_cast<size_t>(e) * d);
      float acc = 0.0f;
      for (int i = 0; i < d / 4; ++i) {
        const float4 a = xr[i], b = wrr[i];
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
      }
      s_z[tl * ldz + e] = acc + (bias ? bias[e] : 0.0f);
    }
  }
  __syncthreads();

  // ---------------- phase 2: scores and top-k per token ------------------
  constexpr int kMaxPerLane = 16;     // E <= 1024
  const int nper = (E + 63) / 64;
  for (int tl = wave; tl < kRouteTM; tl += 4) {
    const int t = t0 + tl;
    if (t >= T) break;
    float p[kMaxPerLane];
    const float* zrow = s_z + tl * ldz;
    if (score_fn == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        p[i] = (i < nper && e < E) ? zrow[e] : -INFINITY;
        m = fmaxf(m, p[i]);
      }
      m = wave_max(m);
      float s = 0.0f;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        p[i] = (i < nper && e < E) ? expf(p[i] - m) : 0.0f;
        s += p[i];
      }
      s = wave_sum(s);
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        p[i] = (i < nper && e < E) ? p[i] / s : -INFINITY;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        p[i] = (i < nper && e < E) ? sigmoidf_(zrow[e]) : -INFINITY;
      }
    }
    uint32_t taken = 0;
    int my_e = E;
    float my_p = 0.0f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int bi = E;
#pragma unroll
      for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        // strict '>' keeps the lower expert index among equal scores
        if (!((taken >> i) & 1u) && p[i] > bv) { bv = p[i]; bi = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == j) { my_e = bi; my_p = bv; }
    }
    float denom = 1.0f;
    if (normalize) denom = wave_sum(lane < k ? my_p : 0.0f);
    if (lane < k) {
      topk_idx[static_cast<size_t>(t) * k + lane] = my_e;
      topk_w[static_cast<size_t>(t) * k + lane] = normalize ? my_p / denom : my_p;
      if (my_e < E) atomicAdd(&s_cnt[my_e], 1);
    }
    if (gate) {
      float g = 0.0f;
      if constexpr (kBF16) {
        const uint16_t* xr = static_cast<const uint16_t*>(xv) + static_cast<size_t>(t) * d;
        const uint16_t* wg = static_cast<const uint16_t*>(wgv);
        for (int k8 = lane * 8; k8 < d; k8 += 512) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(xr + k8);
          const u32x4 b = *reinterpret_cast<const u32x4*>(wg + k8);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g = fmaf(bf16lo(a[q]), bf16lo(b[q]), g);
            g = fmaf(bf16hi(a[q]), bf16hi(b[q]), g);
          }
        }
      } else {
        const float* xr = static_cast<const float*>(xv) + static_cast<size_t>(t) * d;
        const float* wg = static_cast<const float*>(wgv);
        for (int i = lane; i < d; i += 64) g = fmaf(xr[i], wg[i], g);
      }
      g = wave_sum(g);
      if (lane == 0) gate[t] = sigmoidf_(g);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads)
    if (s_cnt[e]) atomicAdd(&counts[e], s_cnt[e]);
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(hipStream_t stream, moe_dtype dt, int64_t T,
                                int64_t d, int32_t E, int32_t k,
                                moe_score_fn fn, int32_t normalize,
                                const void* x, const void* w_router,
                                const float* logit_bias, const void* w_gate,
                                int32_t* topk_idx, float* topk_w,
                                int32_t* expert_counts, float* gate) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (fn != MOE_SCORE_SOFTMAX && fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (!x || !w_router || !topk_idx || !topk_w || !expert_counts) return MOE_ERR_INVALID_ARG;
  if ((w_gate == nullptr) != (gate == nullptr)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31) || d >= (int64_t(1) << 30)) return MOE_ERR_SHAPE;
  if (d % 8) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(expert_counts) || !aligned16(gate) || !aligned16(logit_bias))
    return MOE_ERR_ALIGNMENT;

  hipError_t err = launch(zero_i32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream,
                          expert_counts, E);
  if (err != hipSuccess) return MOE_ERR_HIP;
  const int nblk = static_cast<int>((T + kRouteTM - 1) / kRouteTM);
  const size_t lds = (static_cast<size_t>(kRouteTM) * (E + 1) + E) * sizeof(float);
  auto kern = dt == MOE_BF16 ? route_kernel<true> : route_kernel<false>;
  err = allow_lds(kern, lds);
  if (err == hipSuccess)
    err = launch(kern, dim3(nblk), dim3(kRouteThreads), lds, stream, (int)T, (int)d, E, k,
                 (int)fn, normalize, x, w_router, logit_bias, w_gate, topk_idx, topk_w,
                 expert_counts, gate);
  return hip_status(err);
}
