// The layer's backward around the grouped GEMM: combine backward and
// permute + router backward.
//
// Passages: "Megatron-Bridge 深度剖析", section "Activation Recomputation"
// (the backward of an MoE layer recomputes the router softmax and the
// dispatch permute), section "Expert Parallel 基础" step 3 (combine: the
// expert results return to token order, weighted) and "Shared Expert
// Overlap" (the gated shared expert joins the routed result).  The
// derivatives are the chain rule of the forward:
//   combine  y[t] = sum_j w[t,j] Y[s(t,j)] + gate[t] Ysh[t]
//            dY[s(t,j)] = w[t,j] dy[t];  dw[t,j] = <dy[t], Y[s(t,j)]>;
//            dgate[t] = <dy[t], Ysh[t]>
//   permute  dx[t] += sum_j dX[s(t,j)]
//   router   w = normalise(score(z)) on the selection; dz is non-zero on the
//            selected experts only (see rbwd_token_kernel), except for
//            softmax scores without renormalisation, where it is dense
//            (rbwd_dense_dz_kernel);
//            dx[t] += sum_e dz[t,e] W_r[e];  dW_r[e] = sum_t dz[t,e] x[t]
//   gate     g = sigmoid(x . w_gate): dgl = dgate g (1 - g);
//            dx[t] += dgl[t] w_gate;  dw_gate = sum_t dgl[t] x[t]
// All sums run in fp32 in a fixed order (deterministic, no atomics); every
// output is rounded once.
#include "moe_internal.h"

namespace moe {

constexpr int kLbThreads = 256;   // 4 wavefronts, one token each

// 8 values of a 16-byte chunk as fp32
template <bool kBF16>
__device__ __forceinline__ void load8(const void* base, size_t chunk, float (&v)[8]) {
  if constexpr (kBF16) {
    const u32x4 c = static_cast<const u32x4*>(base)[chunk];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = bf16lo(c[q]);
      v[2 * q + 1] = bf16hi(c[q]);
    }
  } else {
    const u32x4 c0 = static_cast<const u32x4*>(base)[2 * chunk];
    const u32x4 c1 = static_cast<const u32x4*>(base)[2 * chunk + 1];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q] = __uint_as_float(c0[q]);
      v[4 + q] = __uint_as_float(c1[q]);
    }
  }
}
// The same load split in two: the raw 16 (bf16) or 32 (fp32) bytes, then
// their conversion.  Batches of raw loads issued without branches go out
// together; a load under a branch, converted inside it, is waited for there.
template <bool kBF16>
struct Raw8 {
  u32x4 c[kBF16 ? 1 : 2];
};
template <bool kBF16>
__device__ __forceinline__ Raw8<kBF16> load_raw8(const void* base, size_t chunk) {
  Raw8<kBF16> r;
  if constexpr (kBF16) {
    r.c[0] = static_cast<const u32x4*>(base)[chunk];
  } else {
    r.c[0] = static_cast<const u32x4*>(base)[2 * chunk];
    r.c[1] = static_cast<const u32x4*>(base)[2 * chunk + 1];
  }
  return r;
}
// the same for data read once (streamed past the caches: non-temporal)
template <bool kBF16>
__device__ __forceinline__ Raw8<kBF16> load_raw8_nt(const void* base, size_t chunk) {
  Raw8<kBF16> r;
  const u32x4* b = static_cast<const u32x4*>(base);
  if constexpr (kBF16) {
    r.c[0] = __builtin_nontemporal_load(b + chunk);
  } else {
    r.c[0] = __builtin_nontemporal_load(b + 2 * chunk);
    r.c[1] = __builtin_nontemporal_load(b + 2 * chunk + 1);
  }
  return r;
}
template <bool kBF16>
__device__ __forceinline__ void cvt8(const Raw8<kBF16>& r, float (&v)[8]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (kBF16) {
      v[2 * q] = bf16lo(r.c[0][q]);
      v[2 * q + 1] = bf16hi(r.c[0][q]);
    } else {
      v[q] = __uint_as_float(r.c[0][q]);
      v[4 + q] = __uint_as_float(r.c[1][q]);
    }
  }
}

template <bool kBF16>
__device__ __forceinline__ void store8(void* base, size_t chunk, const float (&v)[8]) {
  if constexpr (kBF16) {
    u32x4 c;
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = pack_bf16x2(v[2 * q], v[2 * q + 1]);
    static_cast<u32x4*>(base)[chunk] = c;
  } else {
    u32x4 c0, c1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c0[q] = __float_as_uint(v[q]);
      c1[q] = __float_as_uint(v[4 + q]);
    }
    static_cast<u32x4*>(base)[2 * chunk] = c0;
    static_cast<u32x4*>(base)[2 * chunk + 1] = c1;
  }
}

// sum over this lane's chunks c = lane, lane + 64, ... of <a[arow + c], b[brow + c]>
// (8 values each), in chunk order; the loads of four chunks go out together
template <bool kBF16>
__device__ __forceinline__ float row_dot(const void* a, size_t arow, const void* b, size_t brow,
                                         int nchunk, int lane) {
  float dot = 0.0f;
  for (int c0 = lane; c0 < nchunk; c0 += 4 * 64) {
    Raw8<kBF16> ra[4], rb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // chunks past the row re-read chunk c0 (not summed)
      const int c = c0 + u * 64 < nchunk ? c0 + u * 64 : c0;
      ra[u] = load_raw8<kBF16>(a, arow + c);
      rb[u] = load_raw8<kBF16>(b, brow + c);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (c0 + u * 64 < nchunk) {
        float av[8], bv[8];
        cvt8<kBF16>(ra[u], av);
        cvt8<kBF16>(rb[u], bv);
#pragma unroll
        for (int q = 0; q < 8; ++q) dot = fmaf(av[q], bv[q], dot);
      }
  }
  return dot;
}

// ---------------------------------------------------------------------------
// Combine backward: one wavefront per token; a lane owns chunks of 8 columns.
// ---------------------------------------------------------------------------
template <bool kBF16>
__global__ __launch_bounds__(kLbThreads) void combine_bwd_kernel(
    int T, int k, int N, int nchunk, const void* __restrict__ dy, const void* __restrict__ y_perm,
    const int32_t* __restrict__ slot_of, const float* __restrict__ topk_w,
    const void* __restrict__ y_shared, void* __restrict__ dy_perm, float* __restrict__ d_topk_w,
    float* __restrict__ d_gate) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kLbThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t trow = static_cast<size_t>(t) * nchunk;
  for (int j = 0; j < k; ++j) {
    int row = slot_of[static_cast<size_t>(t) * k + j];
    if (row >= N) row = -1;
    float dot = 0.0f;
    if (row >= 0) {
      const float w = topk_w[static_cast<size_t>(t) * k + j];
      const size_t rrow = static_cast<size_t>(row) * nchunk;
      // four chunks' loads at a time (past the row: chunk c0 again, unused)
      for (int c0 = lane; c0 < nchunk; c0 += 4 * 64) {
        Raw8<kBF16> rg[4], ry[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + u * 64 < nchunk ? c0 + u * 64 : c0;
          rg[u] = load_raw8<kBF16>(dy, trow + c);
          ry[u] = load_raw8_nt<kBF16>(y_perm, rrow + c);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + u * 64 < nchunk) {
            float g[8], yv[8], o[8];
            cvt8<kBF16>(rg[u], g);
            cvt8<kBF16>(ry[u], yv);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              dot = fmaf(g[q], yv[q], dot);
              o[q] = w * g[q];
            }
            store8<kBF16>(dy_perm, rrow + c0 + u * 64, o);
          }
      }
    }
    dot = wave_sum(dot);
    if (lane == 0) d_topk_w[static_cast<size_t>(t) * k + j] = row >= 0 ? dot : 0.0f;
  }
  if (y_shared && d_gate) {
    float dot = row_dot<kBF16>(dy, trow, y_shared, trow, nchunk, lane);
    dot = wave_sum(dot);
    if (lane == 0) d_gate[t] = dot;
  }
}

// ---------------------------------------------------------------------------
// Router + permute backward, per token (one wavefront each).
//
// With the selection e_1..e_k fixed, w_j = s_j / S (normalise, S = sum_j s_j)
// or w_j = s_j, s = score(z).  Writing c = sum_j dw_j w_j:
//   softmax, normalised:  dz[e_j] = w_j (dw_j - c), dz = 0 off the selection
//                         (the full-softmax denominator cancels in w);
//   sigmoid, normalised:  dz[e_j] = (dw_j - c) / S * s_j (1 - s_j);
//   sigmoid:              dz[e_j] = dw_j s_j (1 - s_j).
// (Softmax without renormalisation has a dense dz: rbwd_dense_dz_kernel forms
// it, two GEMMs give its dx term and dW_r, and this kernel adds the dx term.)
// The sigmoid forms need s_j = sigmoid(z_j): z_j = x[t] . W_r[e_j] (+ b) is
// recomputed here in fp32.
// ---------------------------------------------------------------------------
constexpr int kDxBatch = 2;    // choices whose rows are loaded together in the dx pass
constexpr int kDxChunks = 4;   // 16-byte chunks of a row per lane in the dx pass

template <bool kBF16>
__global__ __launch_bounds__(kLbThreads) void rbwd_token_kernel(
    int T, int k, int E, int N, int nchunk, int sigmoid, int normalize,
    const void* __restrict__ x, const void* __restrict__ w_router,
    const float* __restrict__ logit_bias, const void* __restrict__ w_gate,
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w,
    const float* __restrict__ d_topk_w, const float* __restrict__ d_gate,
    const int32_t* __restrict__ slot_of, const void* __restrict__ dx_perm,
    const void* __restrict__ dx_add, void* __restrict__ dx, float* __restrict__ dz_slot,
    float* __restrict__ dgl_tok, const float* __restrict__ dx_dense) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kLbThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t trow = static_cast<size_t>(t) * nchunk;
  // lane j < k holds choice j
  int e = -1, row = -1;
  float w = 0.0f, dw = 0.0f;
  if (lane < k) {
    e = topk_idx[static_cast<size_t>(t) * k + lane];
    row = slot_of[static_cast<size_t>(t) * k + lane];
    w = topk_w[static_cast<size_t>(t) * k + lane];
    dw = d_topk_w[static_cast<size_t>(t) * k + lane];
    if (e < 0 || e >= E) e = -1;
    if (row >= N) row = -1;
  }
  float s = 0.0f;   // sigmoid score of choice `lane` (sigmoid only)
  if (sigmoid) {
    for (int j = 0; j < k; ++j) {
      const int ej = __shfl(e, j, kWave);
      float dot = 0.0f;
      if (ej >= 0) dot = row_dot<kBF16>(x, trow, w_router, static_cast<size_t>(ej) * nchunk,
                                        nchunk, lane);
      dot = wave_sum(dot);
      if (lane == j && ej >= 0) s = sigmoidf_(dot + (logit_bias ? logit_bias[ej] : 0.0f));
    }
  }
  const bool mine = lane < k && e >= 0;
  const float c = wave_sum(mine ? dw * w : 0.0f);
  const float S = sigmoid && normalize ? wave_sum(mine ? s : 0.0f) : 1.0f;
  float dz = 0.0f;
  if (mine) {
    if (!sigmoid) dz = w * (dw - c);                          // softmax, normalised
    else if (normalize) dz = (dw - c) / S * s * (1.0f - s);
    else dz = dw * s * (1.0f - s);
  }
  // every row of an expert segment is some token's valid choice, so the
  // rows read by the dW_r pass are all written here
  if (lane < k && row >= 0) dz_slot[row] = dz;
  // shared gate
  float dgl = 0.0f;
  if (w_gate && d_gate) {
    float dot = row_dot<kBF16>(x, trow, w_gate, 0, nchunk, lane);
    dot = wave_sum(dot);
    const float g = sigmoidf_(dot);
    dgl = d_gate[t] * g * (1.0f - g);
    if (lane == 0) dgl_tok[t] = dgl;
  }
  // dx[t] = sum_j dX[row_j] + sum_j dz_j W_r[e_j] + dgl w_gate + dx_add[t].
  // Four chunks of the row per lane at a time (1 KB each per wave): for each
  // choice the loads cover 4 KB of its dX row and W_r row, two choices' loads
  // go out together, and every column sums the choices in order (lanes >= k
  // hold row = e = -1, so j >= k adds nothing).  Loads past the row or of an
  // unused choice re-read valid memory and are not summed.
  for (int c0 = lane; c0 < nchunk; c0 += kDxChunks * 64) {
    float acc[kDxChunks][8];
#pragma unroll
    for (int u = 0; u < kDxChunks; ++u)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[u][q] = 0.0f;
    int cu[kDxChunks];
#pragma unroll
    for (int u = 0; u < kDxChunks; ++u) cu[u] = c0 + u * 64 < nchunk ? c0 + u * 64 : c0;
    for (int j0 = 0; j0 < k; j0 += kDxBatch) {
      Raw8<kBF16> rx[kDxBatch][kDxChunks], rw[kDxBatch][kDxChunks];
      float dzj[kDxBatch];
      bool hx[kDxBatch], hw[kDxBatch];
#pragma unroll
      for (int b = 0; b < kDxBatch; ++b) {
        const int rj = __shfl(row, j0 + b, kWave);
        const int ej = __shfl(e, j0 + b, kWave);
        dzj[b] = __shfl(dz, j0 + b, kWave);
        hx[b] = dx_perm && rj >= 0;
        hw[b] = ej >= 0 && dzj[b] != 0.0f && !dx_dense;   // dense: in dx_dense
        const size_t xr = static_cast<size_t>(hx[b] ? rj : 0) * nchunk;
        const size_t wr = static_cast<size_t>(hw[b] ? ej : 0) * nchunk;
#pragma unroll
        for (int u = 0; u < kDxChunks; ++u) {
          if (dx_perm) rx[b][u] = load_raw8_nt<kBF16>(dx_perm, xr + cu[u]);
          rw[b][u] = load_raw8<kBF16>(w_router, wr + cu[u]);
        }
      }
#pragma unroll
      for (int b = 0; b < kDxBatch; ++b)
#pragma unroll
        for (int u = 0; u < kDxChunks; ++u) {
          float v[8];
          if (hx[b]) {
            cvt8<kBF16>(rx[b][u], v);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] += v[q];
          }
          if (hw[b]) {
            cvt8<kBF16>(rw[b][u], v);
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[u][q] = fmaf(dzj[b], v[q], acc[u][q]);
          }
        }
    }
#pragma unroll
    for (int u = 0; u < kDxChunks; ++u) {
      if (c0 + u * 64 >= nchunk) continue;
      const int cc = c0 + u * 64;
      if (w_gate && d_gate) {
        float v[8];
        load8<kBF16>(w_gate, cc, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] = fmaf(dgl, v[q], acc[u][q]);
      }
      if (dx_add) {
        float v[8];
        load8<kBF16>(dx_add, trow + cc, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] += v[q];
      }
      if (dx_dense) {                             // sum_e dz[t,e] W_r[e] (fp32 rows)
        float v[8];
        load8<false>(dx_dense, trow + cc, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[u][q] += v[q];
      }
      store8<kBF16>(dx, trow + cc, acc[u]);
    }
  }
}

// Dense logit gradient of softmax scores without renormalisation (the
// weights are the scores of the chosen experts, w_j = p[e_j]):
//     dz[t,e] = p[t,e] (ds[t,e] - c[t]),   c[t] = sum_j d_topk_w[t,j] p[t,e_j],
// ds = d_topk_w on the selection and 0 elsewhere; p = softmax(z[t,:]) from the
// recomputed fp32 logits (K slabs summed in slab order), max-subtracted as
// in the forward.  One wavefront per token; lane l holds experts l + 64 i.
template <int kPer>
__global__ __launch_bounds__(kLbThreads) void rbwd_dense_dz_kernel(
    int T, int E, int k, int nslab, const float* __restrict__ z, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ d_topk_w, float* __restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (kLbThreads / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t slab = static_cast<size_t>(T) * E;
  float p[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    float v = 0.0f;
    for (int s = 0; s < nslab; ++s) v += e < E ? z[s * slab + static_cast<size_t>(t) * E + e] : 0.0f;
    p[i] = v;
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (lane + 64 * i < E) m = fmaxf(m, p[i]);
  m = wave_max_dpp(m);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    p[i] = (lane + 64 * i < E) ? expf(p[i] - m) : 0.0f;
    sum += p[i];
  }
  sum = wave_sum_dpp(sum);
#pragma unroll
  for (int i = 0; i < kPer; ++i) p[i] = (lane + 64 * i < E) ? p[i] / sum : 0.0f;
  // choices: lane j < k holds (e_j, dw_j)
  int ej = -1;
  float dwj = 0.0f;
  if (lane < k) {
    ej = topk_idx[static_cast<size_t>(t) * k + lane];
    dwj = d_topk_w[static_cast<size_t>(t) * k + lane];
    if (ej < 0 || ej >= E) ej = -1;
  }
  // c = sum_j dw_j p[e_j] in choice order; ds of this lane's experts
  float c = 0.0f;
  float ds[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) ds[i] = 0.0f;
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(ej, j, kWave);
    const float dw = __shfl(dwj, j, kWave);
    if (e < 0) continue;                          // uniform: every lane reads the same e
    float pe = 0.0f;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (i == (e >> 6)) pe = p[i];
    pe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), e & 63));
    c += dw * pe;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (lane + 64 * i == e) ds[i] = dw;
  }
  float* row = dz + static_cast<size_t>(t) * E;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    if (e < E) row[e] = p[i] * (ds[i] - c);
  }
}

// C[M, N] (+)= sum_k A(m, k) B(k, n) in fp32, k ascending (a fixed order):
// A fp32 at A[m sam + k sak], B of the activation type, row-major with row
// stride ldb, C fp32 row-major with row stride ldc.  64 x 64 tiles, 16-wide
// K steps through LDS, 4 x 4 outputs per thread.  The dense router
// gradient's two products: dx_dense = dz W_r and dW_r = dz^T x.
constexpr int kRgM = 64, kRgN = 64, kRgK = 16;
template <bool kBF16>
__global__ __launch_bounds__(256) void rbwd_gemm_kernel(int M, int N, int K,
                                                        const float* __restrict__ A, int64_t sam,
                                                        int64_t sak, const void* __restrict__ B,
                                                        int64_t ldb, float* __restrict__ C,
                                                        int64_t ldc, int accumulate) {
  __shared__ float As[kRgK][kRgM + 4];
  __shared__ float Bs[kRgK][kRgN + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * kRgM, n0 = blockIdx.x * kRgN;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kRgK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i;              // 64 x 16 values; m fastest when A is m-contiguous
      const int mm = sam == 1 ? idx % kRgM : idx / kRgK;
      const int kk = sam == 1 ? idx / kRgM : idx % kRgK;
      const int m = m0 + mm, kq = k0 + kk;
      As[kk][mm] = (m < M && kq < K) ? A[m * sam + kq * sak] : 0.0f;
      const int nn = idx % kRgN, kb = idx / kRgN; // n fastest
      const int n = n0 + nn, kr = k0 + kb;
      float bv = 0.0f;
      if (n < N && kr < K) {
        if constexpr (kBF16)
          bv = bf16_to_f32(static_cast<const uint16_t*>(B)[kr * ldb + n]);
        else
          bv = static_cast<const float*>(B)[kr * ldb + n];
      }
      Bs[kb][nn] = bv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRgK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float* c = C + m * ldc + n;
      *c = accumulate ? *c + acc[i][j] : acc[i][j];
    }
  }
}

// dW_r[e, cols] (+)= sum over expert e's rows r of dz_slot[r] *
// x[row_token[r], cols].  Grid (E, column blocks of 512); a lane owns 8
// columns; wave w of the workgroup sums rows lo + w, lo + w + 4, ... in row
// order, and the four wave sums are added in wave order (a fixed order: the
// result does not depend on timing).  The row indices of 64 rows come in
// with one load per lane; the x loads go out 16 rows at a time.
constexpr int kDwrWaves = 4;
constexpr int kDwrBatch = 16;
template <bool kBF16>
__global__ __launch_bounds__(64 * kDwrWaves) void rbwd_dwr_kernel(int d, int nchunk,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ row_token,
                                                                  const float* __restrict__ dz_slot,
                                                                  const void* __restrict__ x,
                                                                  float* __restrict__ dw_router,
                                                                  int accumulate) {
  __shared__ float s_part[kDwrWaves - 1][64 * 8];
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.y * 64 + lane;
  const bool live = c < nchunk;
  const int cl = live ? c : 0;   // lanes past the row read chunk 0 and store nothing
  const int lo = offsets[e], hi = offsets[e + 1];
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  for (int base = lo + wave; base < hi; base += 64 * kDwrWaves) {
    // this wave's rows base + 4 u, u < 64: lane u fetches row u's token and dz
    const int rl = base + kDwrWaves * lane;
    const int tok_l = rl < hi ? row_token[rl] : 0;
    const float g_l = rl < hi ? dz_slot[rl] : 0.0f;
    for (int u0 = 0; u0 < 64 && base + kDwrWaves * u0 < hi; u0 += kDwrBatch) {
      Raw8<kBF16> rv[kDwrBatch];
      float g[kDwrBatch];
#pragma unroll
      for (int u = 0; u < kDwrBatch; ++u) {   // rows past the segment read token 0 (not summed)
        const int tk = __shfl(tok_l, u0 + u, kWave);
        g[u] = __shfl(g_l, u0 + u, kWave);
        rv[u] = load_raw8<kBF16>(x, static_cast<size_t>(tk) * nchunk + cl);
      }
#pragma unroll
      for (int u = 0; u < kDwrBatch; ++u)
        if (base + kDwrWaves * (u0 + u) < hi) {
          float v[8];
          cvt8<kBF16>(rv[u], v);
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = fmaf(g[u], v[q], acc[q]);
        }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) s_part[wave - 1][q * 64 + lane] = acc[q];
  }
  __syncthreads();
  if (wave > 0 || !live) return;
#pragma unroll
  for (int w = 0; w < kDwrWaves - 1; ++w)
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += s_part[w][q * 64 + lane];
  float* dst = dw_router + static_cast<size_t>(e) * d + 8 * c;
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = accumulate ? dst[q] + acc[q] : acc[q];
}

// dw_gate = sum_t dgl[t] x[t]: partial sums over token blocks of 256 in
// token order, then a fixed-order sum over the blocks.
constexpr int kGateRows = 256;
template <bool kBF16>
__global__ __launch_bounds__(64) void rbwd_dwg_partial_kernel(int T, int nchunk,
                                                              const float* __restrict__ dgl_tok,
                                                              const void* __restrict__ x,
                                                              float* __restrict__ part) {
  const int c = blockIdx.x * 64 + threadIdx.x;
  if (c >= nchunk) return;
  const int t0 = blockIdx.y * kGateRows, t1 = min(T, t0 + kGateRows);
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
  // 16 tokens' loads at a time, summed in token order
  for (int tb = t0; tb < t1; tb += 16) {
    Raw8<kBF16> rv[16];
    float g[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {   // tokens past the block re-read token tb (not summed)
      const int t = tb + u < t1 ? tb + u : tb;
      g[u] = dgl_tok[t];
      rv[u] = load_raw8<kBF16>(x, static_cast<size_t>(t) * nchunk + c);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (tb + u < t1) {
        float v[8];
        cvt8<kBF16>(rv[u], v);
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = fmaf(g[u], v[q], acc[q]);
      }
  }
  float* dst = part + static_cast<size_t>(blockIdx.y) * nchunk * 8 + 8 * c;
#pragma unroll
  for (int q = 0; q < 8; ++q) dst[q] = acc[q];
}
__global__ __launch_bounds__(256) void rbwd_dwg_sum_kernel(int d, int nblk,
                                                           const float* __restrict__ part,
                                                           float* __restrict__ dw_gate,
                                                           int accumulate) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= d) return;
  float s = 0.0f;
  for (int b = 0; b < nblk; ++b) s += part[static_cast<size_t>(b) * d + i];
  dw_gate[i] = accumulate ? dw_gate[i] + s : s;
}

inline size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_combine_backward(hipStream_t stream, moe_dtype dt, int64_t T, int64_t d,
                                           int32_t k, int64_t N, const void* dy,
                                           const void* y_perm, const int32_t* slot_of,
                                           const float* topk_w, const void* y_shared,
                                           void* dy_perm, float* d_topk_w, float* d_gate) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!dy || !y_perm || !slot_of || !topk_w || !dy_perm || !d_topk_w) return MOE_ERR_INVALID_ARG;
  if ((y_shared == nullptr) != (d_gate == nullptr)) return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || k < 1 || k > 32 || N < 0 || N >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (d % 8) return MOE_ERR_ALIGNMENT;
  if (!aligned16(dy) || !aligned16(y_perm) || !aligned16(slot_of) || !aligned16(topk_w) ||
      !aligned16(y_shared) || !aligned16(dy_perm) || !aligned16(d_topk_w) || !aligned16(d_gate))
    return MOE_ERR_ALIGNMENT;
  auto kern = dt == MOE_BF16 ? combine_bwd_kernel<true> : combine_bwd_kernel<false>;
  return hip_status(launch(kern, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(kLbThreads), 0,
                           stream, (int)T, k, (int)N, (int)(d / 8), dy, y_perm, slot_of, topk_w,
                           y_shared, dy_perm, d_topk_w, d_gate));
}

static bool rbwd_dense(moe_score_fn fn, int32_t normalize) {
  return fn == MOE_SCORE_SOFTMAX && !normalize;
}

extern "C" size_t moe_route_backward_workspace_size(int64_t T, int64_t d, int32_t E, int32_t k,
                                                    moe_dtype dt, moe_score_fn fn,
                                                    int32_t normalize) {
  if (T < 1 || d < 1 || E < 1 || k < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  const int64_t nblk = (T + kGateRows - 1) / kGateRows;
  size_t b = align256(static_cast<size_t>(T) * k * sizeof(float)) +
             align256(static_cast<size_t>(T) * sizeof(float)) +
             align256(static_cast<size_t>(nblk) * d * sizeof(float));
  if (rbwd_dense(fn, normalize))   // logit slabs, dense dz [T, E], dx term [T, d]
    b += align256(static_cast<size_t>(route_logit_slabs(dt, T, d, E)) * T * E * sizeof(float)) +
         align256(static_cast<size_t>(T) * E * sizeof(float)) +
         align256(static_cast<size_t>(T) * d * sizeof(float));
  return b;
}

extern "C" moe_status moe_route_backward(
    hipStream_t stream, moe_dtype dt, int64_t T, int64_t d, int32_t E, int32_t k, moe_score_fn fn,
    int32_t normalize, const void* x, const void* w_router, const float* logit_bias,
    const void* w_gate, const int32_t* topk_idx, const float* topk_w, const float* d_topk_w,
    const float* d_gate, const int32_t* expert_offsets, const int32_t* slot_of,
    const int32_t* row_token, const void* dx_perm, const void* dx_add, void* dx,
    float* dw_router, float* dw_gate, int32_t accumulate, void* ws, size_t ws_bytes) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (fn != MOE_SCORE_SOFTMAX && fn != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (!x || !w_router || !topk_idx || !topk_w || !d_topk_w || !expert_offsets || !slot_of ||
      !row_token || !dx || !dw_router)
    return MOE_ERR_INVALID_ARG;
  if ((w_gate == nullptr) != (d_gate == nullptr) || (w_gate == nullptr) != (dw_gate == nullptr))
    return MOE_ERR_INVALID_ARG;
  if (T < 1 || d < 1 || E < 1 || E > 1024 || k < 1 || k > 32 || k > E) return MOE_ERR_SHAPE;
  if (T * static_cast<int64_t>(k) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (d % 8) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(logit_bias) || !aligned16(w_gate) ||
      !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(d_topk_w) || !aligned16(d_gate) ||
      !aligned16(expert_offsets) || !aligned16(slot_of) || !aligned16(row_token) ||
      !aligned16(dx_perm) || !aligned16(dx_add) || !aligned16(dx) || !aligned16(dw_router) ||
      !aligned16(dw_gate) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_route_backward_workspace_size(T, d, E, k, dt, fn, normalize))
    return MOE_ERR_WORKSPACE;
  if (rbwd_dense(fn, normalize) &&
      (T * static_cast<int64_t>(E) >= (int64_t(1) << 31) || T * d >= (int64_t(1) << 31)))
    return MOE_ERR_SHAPE;
  const int N = static_cast<int>(T * k);
  const int nchunk = static_cast<int>(d / 8);
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  float* dz_slot = reinterpret_cast<float*>(wsb);
  size_t off = align256(static_cast<size_t>(N) * sizeof(float));
  float* dgl = reinterpret_cast<float*>(wsb + off);
  off += align256(static_cast<size_t>(T) * sizeof(float));
  float* part = reinterpret_cast<float*>(wsb + off);
  const int nblk = static_cast<int>((T + kGateRows - 1) / kGateRows);
  const bool bf = dt == MOE_BF16;
  hipError_t err = hipSuccess;
  const bool dense = rbwd_dense(fn, normalize);
  float* dx_dense = nullptr;
  if (dense) {
    // logits -> dense dz [T, E] -> dx_dense = dz W_r [T, d] (fp32)
    off += align256(static_cast<size_t>(nblk) * d * sizeof(float));
    float* z = reinterpret_cast<float*>(wsb + off);
    off += align256(static_cast<size_t>(route_logit_slabs(dt, T, d, E)) * T * E * sizeof(float));
    float* dz = reinterpret_cast<float*>(wsb + off);
    off += align256(static_cast<size_t>(T) * E * sizeof(float));
    dx_dense = reinterpret_cast<float*>(wsb + off);
    err = launch_route_logits(stream, dt, T, d, E, x, w_router, logit_bias, z);
    if (err == hipSuccess) {
      auto kern = E <= 64 ? rbwd_dense_dz_kernel<1> : E <= 128 ? rbwd_dense_dz_kernel<2>
                : E <= 256 ? rbwd_dense_dz_kernel<4> : E <= 512 ? rbwd_dense_dz_kernel<8>
                : rbwd_dense_dz_kernel<16>;
      err = launch(kern, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(kLbThreads), 0, stream,
                   (int)T, E, k, route_logit_slabs(dt, T, d, E), (const float*)z, topk_idx,
                   d_topk_w, dz);
    }
    if (err == hipSuccess) {
      auto kern = bf ? rbwd_gemm_kernel<true> : rbwd_gemm_kernel<false>;
      err = launch(kern, dim3(static_cast<unsigned>((d + kRgN - 1) / kRgN),
                              static_cast<unsigned>((T + kRgM - 1) / kRgM)),
                   dim3(256), 0, stream, (int)T, (int)d, E, (const float*)dz, (int64_t)E,
                   (int64_t)1, w_router, (int64_t)d, dx_dense, (int64_t)d, 0);
    }
    if (err == hipSuccess) {   // dW_r = dz^T x
      auto kern = bf ? rbwd_gemm_kernel<true> : rbwd_gemm_kernel<false>;
      err = launch(kern, dim3(static_cast<unsigned>((d + kRgN - 1) / kRgN),
                              static_cast<unsigned>((E + kRgM - 1) / kRgM)),
                   dim3(256), 0, stream, E, (int)d, (int)T, (const float*)dz, (int64_t)1,
                   (int64_t)E, x, (int64_t)d, dw_router, (int64_t)d, accumulate);
    }
    if (err != hipSuccess) return MOE_ERR_HIP;
  }
  {
    auto kern = bf ? rbwd_token_kernel<true> : rbwd_token_kernel<false>;
    err = launch(kern, dim3(static_cast<unsigned>((T + 3) / 4)), dim3(kLbThreads), 0, stream,
                 (int)T, k, E, N, nchunk, fn == MOE_SCORE_SIGMOID ? 1 : 0, normalize ? 1 : 0, x,
                 w_router, logit_bias, w_gate, topk_idx, topk_w, d_topk_w, d_gate, slot_of,
                 dx_perm, dx_add, dx, dz_slot, dgl, (const float*)dx_dense);
  }
  if (err == hipSuccess && !dense) {
    auto kern = bf ? rbwd_dwr_kernel<true> : rbwd_dwr_kernel<false>;
    err = launch(kern, dim3(E, (nchunk + 63) / 64), dim3(64 * kDwrWaves), 0, stream, (int)d,
                 nchunk, expert_offsets, row_token, dz_slot, x, dw_router, accumulate);
  }
  if (err == hipSuccess && w_gate) {
    auto kern = bf ? rbwd_dwg_partial_kernel<true> : rbwd_dwg_partial_kernel<false>;
    err = launch(kern, dim3((nchunk + 63) / 64, nblk), dim3(64), 0, stream, (int)T, nchunk, dgl, x,
                 part);
    if (err == hipSuccess)
      err = launch(rbwd_dwg_sum_kernel, dim3(static_cast<unsigned>((d + 255) / 256)), dim3(256),
                   0, stream, (int)d, nblk, part, dw_gate, accumulate);
  }
  return hip_status(err);
}
