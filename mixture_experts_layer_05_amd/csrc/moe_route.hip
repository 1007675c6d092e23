// moe_route: router logits, score function, wavefront top-k, weight
// normalisation, per-expert counts and the shared-expert gate.
//
// Passage: "Megatron-Bridge 深度剖析", section "MoE 加速深度剖析 / Expert
// Parallel 基础", step 1 of the diagram: the router turns each token into
// its top-k experts with scores (top-6 sigmoid in the example); the score
// function is a TransformerConfig choice (section "Megatron-Core 架构速览").
//
//   1. logits z[T, E] (fp32, in the workspace): bf16 runs the grouped-GEMM
//      forward kernel as a one-group GEMM with a bias epilogue (MFMA, LDS
//      ring), K split into slabs; fp32 runs a plain FMA dot product per
//      (token, expert);
//   2. route_topk: one wavefront per token; lane l holds the scores of
//      experts l, l+64, ...; k rounds of a wave-wide arg-max (ties to the
//      lower expert index) pick the experts in descending score order (or
//      descending score + selection bias, when a selection-only expert bias
//      is given: the weights still come from the unbiased scores); the
//      workgroup's choices are counted in LDS and written as one histogram
//      row; the gate is a wave-wide dot product x[t] . w_gate;
//   3. route_count: counts[e] = sum of the histogram rows (one workgroup per
//      expert; no global atomics, so a hot expert costs nothing extra).
#include "moe_gemm_common.h"

namespace moe {

constexpr int kTopkThreads = 1024;  // 16 tokens per workgroup, one per wave
constexpr int kTopkTokens = kTopkThreads / 64;

__global__ __launch_bounds__(256) void route_logits_f32_kernel(
    int T, int d, int E, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ z) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<int64_t>(T) * E) return;
  const int t = static_cast<int>(idx / E), e = static_cast<int>(idx - static_cast<int64_t>(t) * E);
  const float4* xr = reinterpret_cast<const float4*>(x + static_cast<size_t>(t) * d);
  const float4* wrr = reinterpret_cast<const float4*>(wr + static_cast<size_t>(e) * d);
  float acc = 0.0f;
  for (int i = 0; i < d / 4; ++i) {
    const float4 a = xr[i], b = wrr[i];
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  z[idx] = acc + (bias ? bias[e] : 0.0f);
}

// One wavefront per token.  kPer = scores held per lane (E <= 64 kPer).
template <bool kBF16, int kPer>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    int T, int d, int E, int k, int score_fn, int normalize, int nslab, const float* __restrict__ z,
    const float* __restrict__ sel_bias, const void* __restrict__ xv, const void* __restrict__ wgv,
    int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int32_t* __restrict__ hist, float* __restrict__ gate) {
  extern __shared__ int s_cnt[];     // [E] histogram of this workgroup's choices
  for (int e = threadIdx.x; e < E; e += kTopkThreads) s_cnt[e] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * kTopkTokens + (threadIdx.x >> 6);
  if (t < T) {
  // logits = sum of the K slabs, in slab order (the loads of 8 slabs are
  // issued before their sum, not one round trip per slab)
  const size_t slab = static_cast<size_t>(T) * E;
  const float* zrow = z + static_cast<size_t>(t) * E;
  float p[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) p[i] = 0.0f;
  for (int s0 = 0; s0 < nslab; s0 += 8) {
    float v[8][kPer];
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        v[q][i] = (s0 + q < nslab && e < E) ? zrow[(s0 + q) * slab + e] : 0.0f;
      }
#pragma unroll
    for (int q = 0; q < 8; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (s0 + q < nslab) p[i] += v[q][i];
  }
  if (score_fn == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i < E) m = fmaxf(m, p[i]);
    m = wave_max_dpp(m);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      p[i] = (lane + 64 * i < E) ? expf(p[i] - m) : 0.0f;
      s += p[i];
    }
    s = wave_sum_dpp(s);
#pragma unroll
    for (int i = 0; i < kPer; ++i) p[i] = (lane + 64 * i < E) ? p[i] / s : -INFINITY;
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) p[i] = (lane + 64 * i < E) ? sigmoidf_(p[i]) : -INFINITY;
  }
  // ranking keys: the scores, or score + selection bias (fp32)
  float key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    key[i] = (sel_bias && e < E) ? p[i] + sel_bias[e] : p[i];
  }
  // k rounds: the largest remaining key (wave max), then the lowest expert
  // index holding it (wave min); both reductions stay in registers (DPP).
  uint32_t taken = 0;
  int my_e = E;
  float my_p = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = E;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      // strict '>' keeps the lower expert index among equal keys
      if (!((taken >> i) & 1u) && key[i] > bv) { bv = key[i]; bi = lane + 64 * i; }
    }
    const float mv = wave_max_dpp(bv);
    bi = wave_min_dpp(bv == mv ? bi : 0x7fffffff);
    bi = bi < E ? bi : E;
    // the winner's (unbiased) score, from the lane that holds it
    float pw = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i == (bi >> 6)) pw = p[i];
    pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pw), bi & 63));
    if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) { my_e = bi; my_p = pw; }
  }
  float denom = 1.0f;
  if (normalize) denom = wave_sum_dpp(lane < k ? my_p : 0.0f);
  if (lane < k) {
    topk_idx[static_cast<size_t>(t) * k + lane] = my_e;
    topk_w[static_cast<size_t>(t) * k + lane] = normalize ? my_p / denom : my_p;
    if (my_e < E) atomicAdd(&s_cnt[my_e], 1);   // LDS integer atomics: order-free
  }
  if (gate) {
    // the row's loads go out four (bf16: 4 x 1 KB per wave) or eight at a
    // time before their products are summed, in the same order as one at a
    // time (past d: 0 * 0, which leaves g unchanged)
    float g = 0.0f;
    if constexpr (kBF16) {
      const uint16_t* xr = static_cast<const uint16_t*>(xv) + static_cast<size_t>(t) * d;
      const uint16_t* wg = static_cast<const uint16_t*>(wgv);
      for (int k0 = lane * 8; k0 < d; k0 += 4 * 512) {
        u32x4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int k8 = k0 + u * 512;
          a[u] = k8 < d ? *reinterpret_cast<const u32x4*>(xr + k8) : u32x4{0, 0, 0, 0};
          b[u] = k8 < d ? *reinterpret_cast<const u32x4*>(wg + k8) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            g = fmaf(bf16lo(a[u][q]), bf16lo(b[u][q]), g);
            g = fmaf(bf16hi(a[u][q]), bf16hi(b[u][q]), g);
          }
      }
    } else {
      const float* xr = static_cast<const float*>(xv) + static_cast<size_t>(t) * d;
      const float* wg = static_cast<const float*>(wgv);
      for (int i0 = lane; i0 < d; i0 += 8 * 64) {
        float a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * 64;
          a[u] = i < d ? xr[i] : 0.0f;
          b[u] = i < d ? wg[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) g = fmaf(a[u], b[u], g);
      }
    }
    g = wave_sum_dpp(g);
    if (lane == 0) gate[t] = sigmoidf_(g);
  }
  }
  __syncthreads();
  int32_t* hrow = hist + static_cast<size_t>(blockIdx.x) * E;
  for (int e = threadIdx.x; e < E; e += kTopkThreads) hrow[e] = s_cnt[e];
}

// counts[e] = sum over workgroups of hist[b][e] (one workgroup per expert)
__global__ __launch_bounds__(256) void route_count_kernel(int nblk, int E,
                                                          const int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ counts) {
  __shared__ int s_part[4];
  const int e = blockIdx.x;
  int v = 0;
  for (int b = threadIdx.x; b < nblk; b += 256) v += hist[static_cast<size_t>(b) * E + e];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) counts[e] = s_part[0] + s_part[1] + s_part[2] + s_part[3];
}

template <bool kBF16>
static auto pick_topk(int E) {
  if (E <= 64) return route_topk_kernel<kBF16, 1>;
  if (E <= 128) return route_topk_kernel<kBF16, 2>;
  if (E <= 256) return route_topk_kernel<kBF16, 4>;
  if (E <= 512) return route_topk_kernel<kBF16, 8>;
  return route_topk_kernel<kBF16, 16>;
}

}  // namespace moe

using namespace moe;

static int route_slabs(moe_dtype dt, int64_t T, int64_t d, int32_t E) {
  return dt == MOE_BF16 ? router_ksplit(T, d, E) : 1;
}

static size_t route_hist_bytes(int64_t T, int32_t E) {
  const int64_t nblk = (T + kTopkTokens - 1) / kTopkTokens;
  return (static_cast<size_t>(nblk) * E * sizeof(int32_t) + 255) & ~static_cast<size_t>(255);
}

extern "C" size_t moe_route_workspace_size(int64_t T, int64_t d, int32_t E, moe_dtype dt) {
  if (T < 1 || d < 1 || E < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  // per-workgroup histograms; fp32 logits, one slab per K split
  return route_hist_bytes(T, E) +
         static_cast<size_t>(route_slabs(dt, T, d, E)) * T * E * sizeof(float);
}

extern "C" moe_status moe_route(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                                int32_t E, int32_t k, moe_score_fn fn, int32_t normalize,
                                const void* x, const void* w_router,
                                const float* logit_bias, const float* selection_bias,
                                const void* w_gate, int32_t* topk_idx, float* topk_w,
                                int32_t* expert_counts, float* gate, void* ws, size_t ws_bytes) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (fn != MOE_SCORE_SOFTMAX && fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (!x || !w_router || !topk_idx || !topk_w || !expert_counts) return MOE_ERR_INVALID_ARG;
  if ((w_gate == nullptr) != (gate == nullptr)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31) || d >= (int64_t(1) << 20) ||
      16 * T * static_cast<int64_t>(E) >= (int64_t(1) << 31) ||
      static_cast<int64_t>(E) * d * 2 >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (d % 8) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(expert_counts) || !aligned16(gate) ||
      !aligned16(logit_bias) || !aligned16(selection_bias) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_route_workspace_size(T, d, E, dt)) return MOE_ERR_WORKSPACE;

  int32_t* hist = static_cast<int32_t*>(ws);
  float* z = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + route_hist_bytes(T, E));
  hipError_t err;
  const int nslab = route_slabs(dt, T, d, E);
  if (dt == MOE_BF16) {
    err = launch_router_logits_bf16(stream, T, d, E, x, w_router, logit_bias, z, nslab);
  } else {
    const int64_t n = T * E;
    err = launch(route_logits_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                 stream, (int)T, (int)d, E, static_cast<const float*>(x),
                 static_cast<const float*>(w_router), logit_bias, z);
  }
  if (err != hipSuccess) return MOE_ERR_HIP;
  auto kern = dt == MOE_BF16 ? pick_topk<true>(E) : pick_topk<false>(E);
  const int nblk = static_cast<int>((T + kTopkTokens - 1) / kTopkTokens);
  err = launch(kern, dim3(nblk), dim3(kTopkThreads), E * sizeof(int), stream, (int)T, (int)d, E, k,
               (int)fn, normalize, nslab, (const float*)z, selection_bias, x, w_gate, topk_idx,
               topk_w, hist, gate);
  if (err == hipSuccess)
    err = launch(route_count_kernel, dim3(E), dim3(256), 0, stream, nblk, E, (const int32_t*)hist,
                 expert_counts);
  return hip_status(err);
}

namespace moe {

// Router logits alone (fp32, K slabs summed by the reader), shared with the
// router backward, which recomputes every expert's score when the logit
// gradient is dense.
int route_logit_slabs(moe_dtype dt, int64_t T, int64_t d, int32_t E) {
  return route_slabs(dt, T, d, E);
}
hipError_t launch_route_logits(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d, int32_t E,
                               const void* x, const void* w_router, const float* logit_bias,
                               float* z) {
  if (dt == MOE_BF16)
    return launch_router_logits_bf16(stream, T, d, E, x, w_router, logit_bias, z,
                                     route_slabs(dt, T, d, E));
  const int64_t n = T * E;
  return launch(route_logits_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                stream, (int)T, (int)d, E, static_cast<const float*>(x),
                static_cast<const float*>(w_router), logit_bias, z);
}

}  // namespace moe
