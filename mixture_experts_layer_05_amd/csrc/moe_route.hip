// moe_route: router logits, score function, top-k, weight normalisation,
// per-expert counts and the shared-expert gate.
//
// Passage: "Megatron-Bridge 深度剖析", section "MoE 加速深度剖析 / Expert
// Parallel 基础", step 1 of the diagram: the router turns each token into
// its top-k experts with scores (top-6 sigmoid in the example); the score
// function is a TransformerConfig choice (section "Megatron-Core 架构速览").
//
// Two launches:
//   1. logits z[T, E] (fp32, in the workspace): bf16 runs the grouped-GEMM
//      forward kernel as a one-group GEMM with a bias epilogue (MFMA, LDS
//      ring), K split into slabs, and (when the slab's gate weights fit in
//      LDS) the K slabs of x . w_gate from the same staged token rows; fp32
//      runs a plain FMA dot product per (token, expert).  Either kernel
//      also zeroes expert_counts (when asked for).
//   2. route_topk: a group of G lanes per token (G = 16 for E <= 256, four
//      tokens per wavefront; G = 64 above), 64 tokens per workgroup; lane i
//      of a group holds the scores of experts i, i + G, ...; k rounds of a
//      group-wide arg-max (ties to the lower expert index, reduced with DPP
//      row operations) pick the experts in descending score order (or
//      descending score + selection bias, when a selection-only expert bias
//      is given: the weights still come from the unbiased scores).  The
//      workgroup's choices are counted in LDS; the counts are added to
//      expert_counts (integer atomics: the sums do not depend on their
//      order) and optionally written as the 64-token block's histogram row,
//      which moe_permute can take instead of counting again.
#include <climits>

#include "moe_gemm_common.h"

namespace moe {

constexpr int kTopkThreads = 1024;
constexpr int kTopkBlk = MOE_ROUTE_BLOCK_TOKENS;   // tokens per workgroup and histogram row

__global__ __launch_bounds__(256) void route_logits_f32_kernel(
    int T, int d, int E, const float* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ bias, float* __restrict__ z, int32_t* __restrict__ zero_counts) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (zero_counts && idx < E) zero_counts[idx] = 0;
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

// Reductions over a group of G lanes (16: one DPP row; 64: the wavefront),
// the result in every lane of the group, in a fixed order.
template <int G>
__device__ __forceinline__ float grp_max(float v) {
  v = fmaxf(v, __int_as_float(dpp_<kDppXor1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppXor2>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppHalfMirror>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_<kDppMirror>(__float_as_int(v))));
  if constexpr (G == 64) {
    const int b = __float_as_int(v);
    v = fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)),
                    __int_as_float(__builtin_amdgcn_readlane(b, 16))),
              fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)),
                    __int_as_float(__builtin_amdgcn_readlane(b, 48))));
  }
  return v;
}
template <int G>
__device__ __forceinline__ int grp_min(int v) {
  v = min(v, dpp_<kDppXor1>(v));
  v = min(v, dpp_<kDppXor2>(v));
  v = min(v, dpp_<kDppHalfMirror>(v));
  v = min(v, dpp_<kDppMirror>(v));
  if constexpr (G == 64)
    v = min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
            min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
  return v;
}
// pairs, quads, half rows, rows (then rows 0..3 for G = 64)
template <int G>
__device__ __forceinline__ float grp_sum(float v) {
  v += __int_as_float(dpp_<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppXor2>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppHalfMirror>(__float_as_int(v)));
  v += __int_as_float(dpp_<kDppMirror>(__float_as_int(v)));
  if constexpr (G == 64) {
    const int b = __float_as_int(v);
    v = (__int_as_float(__builtin_amdgcn_readlane(b, 0)) +
         __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
        (__int_as_float(__builtin_amdgcn_readlane(b, 32)) +
         __int_as_float(__builtin_amdgcn_readlane(b, 48)));
  }
  return v;
}

// G lanes per token, kPer = ceil(E / G) scores per lane; 1024 threads take
// the workgroup's 64 tokens in 64 / (16 * 64 / G) passes.  A token's lanes
// are all active or all inactive, so the row-wise DPP reads only its own
// lanes.
template <bool kBF16, int G, int kPer, bool kOnLogits>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    int T, int d, int E, int k, int score_fn, int normalize, int nslab, const float* __restrict__ z,
    const float* __restrict__ sel_bias, const void* __restrict__ xv, const void* __restrict__ wgv,
    const float* __restrict__ gz, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ counts, int32_t* __restrict__ block_counts, float* __restrict__ gate) {
  static_assert(G == 16 || G == 64, "group width");
  static_assert(kPer <= 32, "taken mask");
  constexpr int kTokPass = kTopkThreads / G;           // tokens per pass
  static_assert(kTopkBlk % kTokPass == 0, "passes cover the block");
  constexpr int kSlots = (32 + G - 1) / G;             // choices held per lane (k <= 32)
  extern __shared__ int s_cnt[];     // [E] histogram of this workgroup's choices
  // then (16-lane groups) the choices of the pass's tokens, 32 per token
  int2* const s_ch = reinterpret_cast<int2*>(s_cnt + ((E + 1) & ~1));
  for (int e = threadIdx.x; e < E; e += kTopkThreads) s_cnt[e] = 0;
  __syncthreads();
  const int gi = threadIdx.x & (G - 1);
  const size_t slab = static_cast<size_t>(T) * E;
#pragma unroll 1
  for (int pass = 0; pass < kTopkBlk / kTokPass; ++pass) {
    const int t = blockIdx.x * kTopkBlk + pass * kTokPass + threadIdx.x / G;
    if (t >= T) continue;
    // logits = sum of the K slabs, in slab order (a batch of slabs' loads
    // is issued before their sum)
    const float* zrow = z + static_cast<size_t>(t) * E;
    float p[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) p[j] = 0.0f;
    constexpr int kQ = kPer >= 16 ? 2 : (kPer >= 8 ? 4 : 8);   // slabs per batch
    for (int s0 = 0; s0 < nslab; s0 += kQ) {
      float v[kQ][kPer];
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int e = gi + G * j;
          v[q][j] = (s0 + q < nslab && e < E) ? zrow[(s0 + q) * slab + e] : 0.0f;
        }
#pragma unroll
      for (int q = 0; q < kQ; ++q)
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (s0 + q < nslab) p[j] += v[q][j];
    }
    // With normalised weights and no selection bias, the choice and the
    // weights depend on the logits of the chosen experts only: softmax and
    // sigmoid are increasing, so the logits rank the experts as the scores
    // do, and the softmax's denominator over all E cancels in the
    // renormalisation.  The scores are then formed for the k winners alone.
    constexpr bool on_logits = kOnLogits;   // the host passes normalize && !sel_bias
    if (!on_logits && score_fn == MOE_SCORE_SOFTMAX) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (gi + G * j < E) m = fmaxf(m, p[j]);
      m = grp_max<G>(m);
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        p[j] = (gi + G * j < E) ? expf(p[j] - m) : 0.0f;
        s += p[j];
      }
      s = grp_sum<G>(s);
#pragma unroll
      for (int j = 0; j < kPer; ++j) p[j] = p[j] / s;
    } else if (!on_logits) {
#pragma unroll
      for (int j = 0; j < kPer; ++j) p[j] = sigmoidf_(p[j]);
    }
    // ranking keys: the scores (the logits when ranking on them), or score +
    // selection bias (fp32); -inf for lanes past E and for experts already
    // chosen.  A -inf logit (a masked expert) scores 0, which stays
    // selectable: ranking on logits it becomes the lowest finite key, below
    // every finite logit, and scores 0 again when its weight is formed.
    float key[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int e = gi + G * j;
      float kv = sel_bias ? p[j] + sel_bias[e < E ? e : 0] : p[j];
      if (on_logits && kv == -INFINITY) kv = -__FLT_MAX__;
      key[j] = e < E ? kv : -INFINITY;
    }
    int my_e[kSlots];
    float my_p[kSlots];
#pragma unroll
    for (int r = 0; r < kSlots; ++r) { my_e[r] = E; my_p[r] = 0.0f; }
    if constexpr (G == 16) {
      // This lane's three best remaining (key, score, expert) candidates,
      // best first: a scan in ascending expert order with strict '>' keeps the
      // lower index first among equal keys, and NaN or -inf keys never enter
      // (index E marks an empty place).  A round takes the winner from the
      // head of its owner's list; a lane whose list runs out (its third win)
      // scans again, skipping the experts it already gave (`taken`).
      float ka, kb, kc, sa, sb, sc;
      int ia, ib, ic, left;
      uint32_t taken = 0;
      auto top3 = [&](bool skip_taken) {
        ka = kb = kc = -INFINITY;
        sa = sb = sc = 0.0f;
        ia = ib = ic = E;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const float v = (skip_taken && ((taken >> j) & 1u)) ? -INFINITY : key[j];
          const int e = gi + G * j;
          const bool c1 = v > ka, c2 = v > kb, c3 = v > kc;
          kc = c2 ? kb : (c3 ? v : kc);
          ic = c2 ? ib : (c3 ? e : ic);
          kb = c1 ? ka : (c2 ? v : kb);
          ib = c1 ? ia : (c2 ? e : ib);
          ka = c1 ? v : ka;
          ia = c1 ? e : ia;
          if constexpr (!kOnLogits) {        // the score rides along when it is not the key
            sc = c2 ? sb : (c3 ? p[j] : sc);
            sb = c1 ? sa : (c2 ? p[j] : sb);
            sa = c1 ? p[j] : sa;
          }
        }
        left = 3;
      };
      top3(false);
      // choice j of this token, (expert, score), written by the lane that
      // decides it and read back after the k rounds
      int2* const ch = s_ch + (threadIdx.x / G) * 32;
      for (int j = 0; j < k; ++j) {
        // the largest remaining key of the group; a single lane holding it
        // is the winner (its list head).  When a group has several (equal
        // keys, or no key left at all) the lowest expert index among them
        // wins, found by a group min; the wavefront takes that path only
        // when one of its groups needs it.
        const float mv = grp_max<G>(ka);
        const bool cand = ka == mv;
        const unsigned long long bal = __ballot(cand);
        const bool multi = __popcll((bal >> (threadIdx.x & 48)) & 0xffffull) > 1;
        bool own, writer;
        int wi;
        if (__ballot(multi) != 0ull) {
          wi = grp_min<G>(cand ? ia : INT_MAX);
          wi = wi < E ? wi : E;
          own = wi < E && ia == wi;
          writer = own || (wi == E && gi == 0);
        } else {
          wi = ia;
          own = cand;
          writer = own;
        }
        if (writer) {
          // the winner's (unbiased) score: the key itself when ranking on
          // logits (-inf for an empty place: its weight is 0), else its list
          // head's score
          const float pw = on_logits ? mv : (own ? sa : 0.0f);
          ch[j] = make_int2(own ? wi : E, __float_as_int(pw));
        }
        if (own) {
          taken |= 1u << (wi / G);
          ka = kb; sa = sb; ia = ib;
          kb = kc; sb = sc; ib = ic;
          kc = -INFINITY; sc = 0.0f; ic = E;
          --left;
        }
        if (left == 0 && j + 1 < k) top3(true);   // rare: a lane's fourth choice
      }
      // other lanes' LDS writes are read back: keep the compiler from moving
      // the reads above them (one wavefront's LDS accesses execute in order)
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int r = 0; r < kSlots; ++r) {
        const int j = gi + G * r;
        if (j < k) {
          const int2 c = ch[j];      // written by a lane of this wavefront, in order
          my_e[r] = c.x;
          my_p[r] = __int_as_float(c.y);
        }
      }
    } else {
      // A wavefront per token: a lane holds few scores, so it rescans them
      // all after each of its wins.
      // This lane's best remaining key (strict '>' in ascending expert order
      // keeps the lower index among equal keys); E when none is selectable
      float bv;
      int bi;
      auto local_best = [&]() {
        bv = -INFINITY;
        bi = E;
#pragma unroll
        for (int j = 0; j < kPer; ++j)
          if (key[j] > bv) { bv = key[j]; bi = gi + G * j; }
      };
      local_best();
      for (int j = 0; j < k; ++j) {
        // the largest remaining key of the group, then the lowest expert index
        // holding it
        const float mv = grp_max<G>(bv);
        int wi = grp_min<G>(bv == mv ? bi : INT_MAX);
        wi = wi < E ? wi : E;
        // the winner's (unbiased) score, from the lane that holds it (scores
        // are >= 0, so a max over zeros elsewhere returns it)
        const bool own = wi < E && (wi & (G - 1)) == gi;
        float pw = 0.0f;
#pragma unroll
        for (int jj = 0; jj < kPer; ++jj)
          if (own && jj == wi / G) { pw = p[jj]; key[jj] = -INFINITY; }
        pw = on_logits ? mv : grp_max<G>(pw);
#pragma unroll
        for (int r = 0; r < kSlots; ++r)
          if (j == gi + G * r) { my_e[r] = wi; my_p[r] = pw; }
        local_best();
      }
    }
    if (on_logits) {
      // the winners' scores from their logits (the first winner's is the
      // largest logit of the token: the softmax's shift); a place with no
      // selectable expert (index E) holds -inf and scores 0
      const float m0 = grp_max<G>(gi == 0 ? my_p[0] : -INFINITY);
#pragma unroll
      for (int r = 0; r < kSlots; ++r)
        my_p[r] = score_fn == MOE_SCORE_SOFTMAX ? expf(my_p[r] - m0) : sigmoidf_(my_p[r]);
    }
    float denom = 1.0f;
    if (normalize) {
      float s = 0.0f;
#pragma unroll
      for (int r = 0; r < kSlots; ++r)
        if (gi + G * r < k) s += my_p[r];
      denom = grp_sum<G>(s);
    }
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const int j = gi + G * r;
      if (j < k) {
        topk_idx[static_cast<size_t>(t) * k + j] = my_e[r];
        topk_w[static_cast<size_t>(t) * k + j] = normalize ? my_p[r] / denom : my_p[r];
        if (my_e[r] < E) atomicAdd(&s_cnt[my_e[r]], 1);   // LDS integer atomics: order-free
      }
    }
    if (gate && gz) {
      // the logits GEMM's K slabs of x[t] . w_gate, in slab order
      if (gi == 0) {
        float g = 0.0f;
        for (int s = 0; s < nslab; ++s) g += gz[static_cast<size_t>(s) * T + t];
        gate[t] = sigmoidf_(g);
      }
    } else if (gate) {
      // x[t] . w_gate: lane i of the group takes 16-byte chunks i, i + G,
      // ... (bf16) or 4-byte elements (fp32), four at a time, in order
      float g = 0.0f;
      if constexpr (kBF16) {
        const uint16_t* xr = static_cast<const uint16_t*>(xv) + static_cast<size_t>(t) * d;
        const uint16_t* wg = static_cast<const uint16_t*>(wgv);
        for (int k0 = gi * 8; k0 < d; k0 += 4 * 8 * G) {
          u32x4 a[4], b[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int k8 = k0 + u * 8 * G;
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
        for (int i0 = gi; i0 < d; i0 += 4 * G) {
          float a[4], b[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * G;
            a[u] = i < d ? xr[i] : 0.0f;
            b[u] = i < d ? wg[i] : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) g = fmaf(a[u], b[u], g);
        }
      }
      g = grp_sum<G>(g);
      if (gi == 0) gate[t] = sigmoidf_(g);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kTopkThreads) {
    const int c = s_cnt[e];
    if (block_counts) block_counts[static_cast<size_t>(blockIdx.x) * E + e] = c;
    if (c && counts) atomicAdd(&counts[e], c);
  }
}

template <bool kBF16, bool kOnLogits>
static auto pick_topk_(int E) {
  if (E <= 16) return route_topk_kernel<kBF16, 16, 1, kOnLogits>;
  if (E <= 32) return route_topk_kernel<kBF16, 16, 2, kOnLogits>;
  if (E <= 64) return route_topk_kernel<kBF16, 16, 4, kOnLogits>;
  if (E <= 128) return route_topk_kernel<kBF16, 16, 8, kOnLogits>;
  if (E <= 256) return route_topk_kernel<kBF16, 16, 16, kOnLogits>;
  if (E <= 512) return route_topk_kernel<kBF16, 64, 8, kOnLogits>;
  return route_topk_kernel<kBF16, 64, 16, kOnLogits>;
}
// ranking on the logits: normalised weights and no selection bias
template <bool kBF16>
static auto pick_topk(int E, bool on_logits) {
  return on_logits ? pick_topk_<kBF16, true>(E) : pick_topk_<kBF16, false>(E);
}

}  // namespace moe

using namespace moe;

static int route_slabs(moe_dtype dt, int64_t T, int64_t d, int32_t E) {
  return dt == MOE_BF16 ? router_ksplit(T, d, E) : 1;
}

// bf16 with the gate formed in the logits GEMM: one fp32 slab of gate dot
// products per K split
static size_t route_gate_bytes(moe_dtype dt, int64_t T, int64_t d, int32_t E) {
  if (dt != MOE_BF16 || !router_gate_fused(T, d, E)) return 0;
  return static_cast<size_t>(route_slabs(dt, T, d, E)) * T * sizeof(float);
}

extern "C" size_t moe_route_workspace_size(int64_t T, int64_t d, int32_t E, moe_dtype dt) {
  if (T < 1 || d < 1 || E < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  // fp32 logits, one slab per K split; the gate's slabs
  return static_cast<size_t>(route_slabs(dt, T, d, E)) * T * E * sizeof(float) +
         route_gate_bytes(dt, T, d, E);
}

extern "C" moe_status moe_route(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                                int32_t E, int32_t k, moe_score_fn fn, int32_t normalize,
                                const void* x, const void* w_router,
                                const float* logit_bias, const float* selection_bias,
                                const void* w_gate, int32_t* topk_idx, float* topk_w,
                                int32_t* expert_counts, int32_t* block_counts, float* gate,
                                void* ws, size_t ws_bytes) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (fn != MOE_SCORE_SOFTMAX && fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if ((w_gate == nullptr) != (gate == nullptr)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31) || d >= (int64_t(1) << 20) ||
      16 * T * static_cast<int64_t>(E) >= (int64_t(1) << 31) ||
      static_cast<int64_t>(E) * d * 2 >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (d % 8) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(expert_counts) || !aligned16(block_counts) ||
      !aligned16(gate) || !aligned16(logit_bias) || !aligned16(selection_bias) ||
      !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_route_workspace_size(T, d, E, dt)) return MOE_ERR_WORKSPACE;

  float* z = static_cast<float*>(ws);
  hipError_t err;
  const int nslab = route_slabs(dt, T, d, E);
  float* gz = nullptr;
  if (w_gate && route_gate_bytes(dt, T, d, E) > 0) gz = z + static_cast<size_t>(nslab) * T * E;
  if (dt == MOE_BF16) {
    err = launch_router_logits_bf16(stream, T, d, E, x, w_router, logit_bias, z, nslab, w_gate, gz,
                                    expert_counts);
  } else {
    const int64_t n = T * E;
    err = launch(route_logits_f32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                 stream, (int)T, (int)d, E, static_cast<const float*>(x),
                 static_cast<const float*>(w_router), logit_bias, z, expert_counts);
  }
  if (err != hipSuccess) return MOE_ERR_HIP;
  const bool on_logits = normalize && selection_bias == nullptr;
  auto kern = dt == MOE_BF16 ? pick_topk<true>(E, on_logits) : pick_topk<false>(E, on_logits);
  const int nblk = static_cast<int>((T + kTopkBlk - 1) / kTopkBlk);
  // LDS: the histogram, then (16-lane groups) 32 choices per token of a pass
  const size_t lds = ((E + 1) & ~1) * sizeof(int) + (E <= 256 ? kTopkThreads / 16 * 32 * 8 : 0);
  err = launch(kern, dim3(nblk), dim3(kTopkThreads), lds, stream, (int)T, (int)d, E, k,
               (int)fn, normalize, nslab, (const float*)z, selection_bias, x, w_gate,
               (const float*)gz, topk_idx, topk_w, expert_counts, block_counts, gate);
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
                static_cast<const float*>(w_router), logit_bias, z, (int32_t*)nullptr);
}

}  // namespace moe
