// Grouped SwiGLU expert FFN, backward: fc2 dgrad + SwiGLU backward, fc1
// dgrad, fc2 and fc1 wgrad.
//
// Passages: "Megatron-Bridge 深度剖析", section "计算融合 / Grouped GEMM" (one
// grouped launch over all experts' segments), "通信隐藏与混合精度 / TP 通信重叠"
// (the backward's dgrad and wgrad GEMMs) and "其他融合优化"
// (gradient_accumulation_fusion: fp32 weight-gradient accumulation).
//
// bf16 engine (gfx950):
//   * workgroup = 256 threads = 4 wavefronts in a 2 x 2 grid; block tile
//     128 (rows of the A operand) x 128 (rows of the B operand) x 64 (K);
//     wave tile 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16 accumulators;
//   * both operands are staged in LDS as [row][k] (k contiguous), double
//     buffered through registers; the 8-byte k-groups are XOR-swizzled by
//     row so both the 16-byte MFMA operand reads and the transposing
//     8-byte writes spread over the banks;
//   * an operand whose K runs along memory rows ("K-strided": the weights
//     in dgrad, the activations in wgrad) is read as 4 (k) x 8 (row) blocks
//     of 16-byte loads and transposed in registers (v_perm) before the LDS
//     write, so all four backward GEMMs use one core;
//   * dgrad tiles over ragged expert segments are decoded on the device from
//     expert_offsets (no host synchronisation) and handed to XCDs in
//     contiguous ranges; wgrad tiles are per expert, K = the expert's rows
//     (an empty expert yields zeros);
//   * epilogues fuse the SwiGLU backward (dG = dA U silu'(G), dU = dA
//     silu(G)) with the recomputed A * row_scale for the fc2 wgrad, and the
//     fp32 (optionally accumulating) weight-gradient store.
//   Deterministic: each output element is produced by one workgroup with a
//   fixed K order; no atomics.
#include "moe_gemm_common.h"

namespace moe {

constexpr int kGT = 256;          // threads per workgroup
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLDK = 72;          // LDS row pitch in bf16 elements
constexpr int kTileElems = 128 * kLDK;

enum Epi { EPI_DGRAD2 = 2, EPI_DGRAD1 = 3, EPI_WGRAD = 4 };

struct GGParams {
  int E, F, d;
  int ntn;                        // column tiles per row tile
  const int32_t* offsets;         // [E+1]
  // A operand (rows of C)
  const uint16_t* a;
  int lda;
  // B operand (columns of C), expert 0; expert e at b + e * b_estride
  const uint16_t* b;
  int ldb;
  size_t b_estride;
  int K;                          // contraction length (token-tiled GEMMs)
  const float* scale;             // [N] row scale or NULL
  const uint16_t* gu_in;          // [N, 2F] (DGRAD2)
  uint16_t* out;                  // DGRAD2: dH [N,2F]; DGRAD1: dX [N,d]
  uint16_t* out2;                 // DGRAD2: A*scale [N,F]
  float* outf;                    // WGRAD: dW (expert 0)
  size_t outf_estride;
  int wg_m, wg_n;                 // WGRAD: output rows / cols per expert
  int accumulate;
};

// element (r, k) of a staged operand; k a multiple of 4
__device__ __forceinline__ int lds_off(int r, int k) {
  return r * kLDK + ((((k >> 2) ^ ((r >> 2) & 14))) << 2) + (k & 3);
}

// ---- K-contiguous operand: 128 rows x 64 k; 4 x 16 B per thread ---------
struct RegsK { u32x4 v[4]; };

template <typename RowFn>
__device__ __forceinline__ void load_kcontig(RegsK& s, const uint16_t* base, int ld, RowFn rowfn,
                                             int k0, int K) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + kGT * i;
    const int r = c >> 3, kk = (c & 7) * 8;
    if (k0 + kk < K) {
      s.v[i] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(rowfn(r)) * ld + k0 + kk);
    } else {
      s.v[i] = u32x4{0, 0, 0, 0};
    }
  }
}
__device__ __forceinline__ void store_kcontig(const RegsK& s, uint16_t* lds) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + kGT * i;
    const int r = c >> 3, kk = (c & 7) * 8;
    *reinterpret_cast<u32x4*>(lds + lds_off(r, kk)) = s.v[i];
  }
}

// ---- K-strided operand: element (k, r) at base + krow(k) * ld + col0 + r -
// thread covers k = 4*kb .. 4*kb+3 and rows r = 8*rb .. 8*rb+7
__device__ __forceinline__ void load_kstrided(RegsK& s, const uint16_t* base, int ld, int krow0,
                                              int kvalid, int col0, int ncols, int k0) {
  const int rb = threadIdx.x & 15, kb = threadIdx.x >> 4;
  const int c = col0 + rb * 8;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = k0 + kb * 4 + q;
    if (k < kvalid && c < ncols) {
      s.v[q] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(krow0 + k) * ld + c);
    } else {
      s.v[q] = u32x4{0, 0, 0, 0};
    }
  }
}
__device__ __forceinline__ void store_kstrided(const RegsK& s, uint16_t* lds) {
  const int rb = threadIdx.x & 15, kb = threadIdx.x >> 4;
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) {
    const uint32_t sel = (rr & 1) ? 0x07060302u : 0x05040100u;
    const int w = rr >> 1;
    u32x2 o;
    o[0] = __builtin_amdgcn_perm(s.v[1][w], s.v[0][w], sel);
    o[1] = __builtin_amdgcn_perm(s.v[3][w], s.v[2][w], sel);
    *reinterpret_cast<u32x2*>(lds + lds_off(rb * 8 + rr, kb * 4)) = o;
  }
}

// ---- one staged K tile through the MFMAs ----------------------------------
__device__ __forceinline__ void mfma_tile(const uint16_t* As, const uint16_t* Bs, f32x16 (&acc)[2][2],
                                          int wm, int wn, int lane) {
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < kBK / 16; ++kk) {
    const int ko = kk * 16 + 8 * h;
    bf16x8 a0 = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 64 + r32, ko));
    bf16x8 a1 = *reinterpret_cast<const bf16x8*>(As + lds_off(wm * 64 + 32 + r32, ko));
    bf16x8 b0 = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wn * 32 + r32, ko));
    bf16x8 b1 = *reinterpret_cast<const bf16x8*>(Bs + lds_off(64 + wn * 32 + r32, ko));
    acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[0][0], 0, 0, 0);
    acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, acc[0][1], 0, 0, 0);
    acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, acc[1][0], 0, 0, 0);
    acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[1][1], 0, 0, 0);
  }
}

template <int kEpi>
__global__ __launch_bounds__(kGT, 2) void gg_kernel(GGParams p) {
  extern __shared__ __align__(16) uint16_t lds[];
  uint16_t* As0 = lds;
  uint16_t* Bs0 = lds + kTileElems;
  uint16_t* As1 = lds + 2 * kTileElems;
  uint16_t* Bs1 = lds + 3 * kTileElems;
  __shared__ int s_cum[1025];
  __shared__ int s_tmp[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int e, m0, n0, seg_lo, seg_hi, klen;
  if constexpr (kEpi == EPI_WGRAD) {
    const int tm = (p.wg_m + kBM - 1) / kBM, tn = (p.wg_n + kBN - 1) / kBN;
    const int per_e = tm * tn;
    e = blockIdx.x / per_e;
    if (e >= p.E) return;
    const int local = blockIdx.x - e * per_e;
    m0 = (local / tn) * kBM;
    n0 = (local % tn) * kBN;
    seg_lo = p.offsets[e];
    seg_hi = p.offsets[e + 1];
    klen = seg_hi - seg_lo;
  } else {
    tile_prefix<kGT>(p.offsets, p.E, kBM, p.ntn, s_cum, s_tmp);
    const int total = s_cum[p.E];
    if (static_cast<int>(blockIdx.x) >= total) return;
    const TileIdx ti = tile_decode(p.offsets, p.E, kBM, xcd_remap(blockIdx.x, total), s_cum);
    e = ti.e;
    seg_lo = ti.lo;
    seg_hi = ti.hi;
    m0 = seg_lo + ti.mt * kBM;
    n0 = ti.nt * kBN;
    klen = p.K;
  }

  const uint16_t* bexp = p.b + static_cast<size_t>(e) * p.b_estride;
  const int last_row = seg_hi - 1;
  auto arow = [&](int r) { const int g = m0 + r; return g <= last_row ? g : last_row; };
  auto load = [&](RegsK& ra, RegsK& rb, int k0) {
    if constexpr (kEpi == EPI_DGRAD2) {
      // A = dY rows (K = d contiguous); B = W2[e] (d x F): element (k=n, r=f)
      load_kcontig(ra, p.a, p.lda, arow, k0, klen);
      load_kstrided(rb, bexp, p.ldb, 0, klen, n0, p.F, k0);
    } else if constexpr (kEpi == EPI_DGRAD1) {
      // A = dH rows (K = 2F contiguous); B = W1[e] (2F x d): element (k=j, r=col)
      load_kcontig(ra, p.a, p.lda, arow, k0, klen);
      load_kstrided(rb, bexp, p.ldb, 0, klen, n0, p.d, k0);
    } else {
      // WGRAD: both operands K-strided over the expert's token rows
      load_kstrided(ra, p.a, p.lda, seg_lo, klen, m0, p.wg_m, k0);
      load_kstrided(rb, p.b, p.ldb, seg_lo, klen, n0, p.wg_n, k0);
    }
  };
  auto store = [&](const RegsK& ra, const RegsK& rb, uint16_t* As, uint16_t* Bs) {
    if constexpr (kEpi == EPI_WGRAD) store_kstrided(ra, As); else store_kcontig(ra, As);
    store_kstrided(rb, Bs);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (klen + kBK - 1) / kBK;
  if (nk > 0) {
    RegsK ra, rb;
    load(ra, rb, 0);
    store(ra, rb, As0, Bs0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const bool odd = kt & 1;
      uint16_t* Ac = odd ? As1 : As0;
      uint16_t* Bc = odd ? Bs1 : Bs0;
      const bool more = kt + 1 < nk;
      if (more) load(ra, rb, (kt + 1) * kBK);
      mfma_tile(Ac, Bc, acc, wm, wn, lane);
      if (more) store(ra, rb, odd ? As0 : As1, odd ? Bs0 : Bs1);
      __syncthreads();
    }
  }

  // ---------------- epilogue ------------------------------------------------
  const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int trow = wm * 64 + mi * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if constexpr (kEpi == EPI_WGRAD) {
        const int row = m0 + trow;
        if (row >= p.wg_m) continue;
        float* dst = p.outf + static_cast<size_t>(e) * p.outf_estride + static_cast<size_t>(row) * p.wg_n;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int col = n0 + c * 64 + wn * 32 + r32;
          if (col < p.wg_n) {
            const float v = acc[mi][c][r];
            dst[col] = p.accumulate ? dst[col] + v : v;
          }
        }
      } else {
        const int row = m0 + trow;
        if (row >= seg_hi) continue;
        const size_t rowz = static_cast<size_t>(row);
        if constexpr (kEpi == EPI_DGRAD2) {
          const float s = p.scale ? p.scale[row] : 1.0f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int f = n0 + c * 64 + wn * 32 + r32;
            if (f < p.F) {
              const float da = acc[mi][c][r] * s;
              const float g = bf16_to_f32(p.gu_in[rowz * 2 * p.F + f]);
              const float u = bf16_to_f32(p.gu_in[rowz * 2 * p.F + p.F + f]);
              const float sg = sigmoidf_(g);
              const float sl = g * sg;
              const float dg = da * u * sg * (1.0f + g * (1.0f - sg));
              const float du = da * sl;
              p.out[rowz * 2 * p.F + f] = f32_to_bf16(dg);
              p.out[rowz * 2 * p.F + p.F + f] = f32_to_bf16(du);
              p.out2[rowz * p.F + f] = f32_to_bf16(s * siluf_(g) * u);
            }
          }
        } else {  // EPI_DGRAD1
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int n = n0 + c * 64 + wn * 32 + r32;
            if (n < p.d) p.out[rowz * p.d + n] = f32_to_bf16(acc[mi][c][r]);
          }
        }
      }
    }
  }
}

}  // namespace moe

using namespace moe;

moe_status moe_grouped_check(moe_dtype dt, int64_t N, int64_t d, int64_t F, int32_t E) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (N < 0 || d < 1 || F < 1 || E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if (N >= (int64_t(1) << 31) || d >= (int64_t(1) << 20) || F >= (int64_t(1) << 20))
    return MOE_ERR_SHAPE;
  // buffer descriptors address one expert's weights with 32-bit byte offsets
  if (2 * F * d * 2 >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (d % 8 || F % 8) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

extern "C" size_t moe_grouped_swiglu_bwd_workspace_size(int64_t N, int64_t F, moe_dtype dt,
                                                        int32_t recompute) {
  if (N < 0 || F < 1) return 0;
  // dH [N, 2F] + A*scale [N, F] (+ recomputed G,U [N, 2F])
  const size_t per_row = static_cast<size_t>(F) * (3 + (recompute ? 2 : 0)) * elt_size(dt);
  return static_cast<size_t>(N) * per_row + 1024;
}

static size_t round_up256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

extern "C" moe_status moe_grouped_swiglu_bwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                             int64_t d, int64_t F, int32_t E,
                                             const void* dy_perm, const void* x_perm,
                                             const void* w1, const void* w2,
                                             const int32_t* expert_offsets, const void* gu_save,
                                             const float* row_scale, int32_t accumulate,
                                             void* dx_perm, float* dw1, float* dw2, void* ws,
                                             size_t ws_bytes) {
  moe_status st = moe_grouped_check(dt, N, d, F, E);
  if (st != MOE_OK) return st;
  if (dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!dy_perm || !x_perm || !w1 || !w2 || !expert_offsets || !dx_perm || !dw1 || !dw2)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(dy_perm) || !aligned16(x_perm) || !aligned16(w1) || !aligned16(w2) ||
      !aligned16(expert_offsets) || !aligned16(gu_save) || !aligned16(row_scale) ||
      !aligned16(dx_perm) || !aligned16(dw1) || !aligned16(dw2) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  const int recompute = gu_save == nullptr;
  if (!ws || ws_bytes < moe_grouped_swiglu_bwd_workspace_size(N, F, dt, recompute))
    return MOE_ERR_WORKSPACE;

  uint8_t* wsb = static_cast<uint8_t*>(ws);
  uint16_t* dH = reinterpret_cast<uint16_t*>(wsb);
  size_t off = round_up256(static_cast<size_t>(N) * 2 * F * 2);
  uint16_t* As = reinterpret_cast<uint16_t*>(wsb + off);
  off += round_up256(static_cast<size_t>(N) * F * 2);
  const uint16_t* gu = static_cast<const uint16_t*>(gu_save);
  hipError_t err = hipSuccess;
  if (recompute && N > 0) {
    uint16_t* gu_r = reinterpret_cast<uint16_t*>(wsb + off);
    // fc1 again: its SwiGLU output goes to As (overwritten below), G,U to gu_r
    err = launch_grouped_fwd_bf16(stream, N, d, F, E, x_perm, w1, w2, expert_offsets, nullptr,
                                  nullptr, gu_r, As, false);
    gu = gu_r;
  }
  const size_t lds = 4 * kTileElems * sizeof(uint16_t);
  if (err == hipSuccess) err = allow_lds(gg_kernel<EPI_DGRAD2>, lds);
  if (err == hipSuccess) err = allow_lds(gg_kernel<EPI_DGRAD1>, lds);
  if (err == hipSuccess) err = allow_lds(gg_kernel<EPI_WGRAD>, lds);
  if (err == hipSuccess && N > 0) {
    // fc2 dgrad + SwiGLU backward: dH, A*scale
    GGParams p{};
    p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = expert_offsets;
    p.ntn = (int)((F + kBN - 1) / kBN);
    p.a = static_cast<const uint16_t*>(dy_perm); p.lda = (int)d;
    p.b = static_cast<const uint16_t*>(w2); p.ldb = (int)F; p.b_estride = static_cast<size_t>(d) * F;
    p.K = (int)d; p.scale = row_scale; p.gu_in = gu; p.out = dH; p.out2 = As;
    err = launch(gg_kernel<EPI_DGRAD2>, dim3(tiles_bound(N, E, kBM) * p.ntn), dim3(kGT), lds,
                 stream, p);
  }
  if (err == hipSuccess && N > 0) {
    // fc1 dgrad: dX = dH W1[e]
    GGParams p{};
    p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = expert_offsets;
    p.ntn = (int)((d + kBN - 1) / kBN);
    p.a = dH; p.lda = (int)(2 * F);
    p.b = static_cast<const uint16_t*>(w1); p.ldb = (int)d; p.b_estride = static_cast<size_t>(2 * F) * d;
    p.K = (int)(2 * F); p.out = static_cast<uint16_t*>(dx_perm);
    err = launch(gg_kernel<EPI_DGRAD1>, dim3(tiles_bound(N, E, kBM) * p.ntn), dim3(kGT), lds,
                 stream, p);
  }
  if (err == hipSuccess) {
    // fc2 wgrad: dW2[e] (d x F) = dY^T (A*scale)
    GGParams p{};
    p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = expert_offsets;
    p.a = static_cast<const uint16_t*>(dy_perm); p.lda = (int)d;
    p.b = As; p.ldb = (int)F;
    p.wg_m = (int)d; p.wg_n = (int)F; p.outf = dw2; p.outf_estride = static_cast<size_t>(d) * F;
    p.accumulate = accumulate;
    const int tiles = (int)(((d + kBM - 1) / kBM) * ((F + kBN - 1) / kBN)) * E;
    err = launch(gg_kernel<EPI_WGRAD>, dim3(tiles), dim3(kGT), lds, stream, p);
  }
  if (err == hipSuccess) {
    // fc1 wgrad: dW1[e] (2F x d) = dH^T X
    GGParams p{};
    p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = expert_offsets;
    p.a = dH; p.lda = (int)(2 * F);
    p.b = static_cast<const uint16_t*>(x_perm); p.ldb = (int)d;
    p.wg_m = (int)(2 * F); p.wg_n = (int)d; p.outf = dw1; p.outf_estride = static_cast<size_t>(2 * F) * d;
    p.accumulate = accumulate;
    const int tiles = (int)(((2 * F + kBM - 1) / kBM) * ((d + kBN - 1) / kBN)) * E;
    err = launch(gg_kernel<EPI_WGRAD>, dim3(tiles), dim3(kGT), lds, stream, p);
  }
  return hip_status(err);
}
