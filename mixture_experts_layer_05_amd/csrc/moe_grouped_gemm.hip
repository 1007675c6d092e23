// Grouped SwiGLU expert FFN: forward (fc1 + SwiGLU, fc2 + row scale) and
// backward (fc2 dgrad + SwiGLU backward, fc1 dgrad, fc2 / fc1 wgrad).
//
// Passages: "Megatron-Bridge 深度剖析", section "计算融合 / Grouped GEMM" (all
// experts' GEMMs in one launch over segments of different length, expert
// weights stored back to back), section "权重映射策略" (GatedMLPMapping:
// linear_fc1 = [gate_proj; up_proj], (2*ffn, hidden)), "Motivation" (SwiGLU
// experts: gate_proj, up_proj, down_proj), "通信隐藏与混合精度 / TP 通信重叠"
// (backward dgrad and wgrad GEMMs) and "其他融合优化"
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
//   * an operand whose K runs along memory rows ("K-strided": weights in
//     dgrad, activations in wgrad) is read as 4 (k) x 8 (row) blocks of
//     16-byte loads and transposed in registers (v_perm) before the LDS
//     write, so every GEMM of the forward and backward uses the same core;
//   * tiles over ragged expert segments are enumerated on the device from
//     expert_offsets (no host synchronisation): per expert its row tiles
//     ceil(n_e / 128) x column tiles, row tiles fastest so tiles sharing a
//     weight panel are issued back to back;
//   * epilogues fuse SwiGLU (gate and up columns of the same f sit in the
//     same lane: the B tile holds 64 gate rows then the 64 matching up rows),
//     the routing-weight row scale, the SwiGLU backward and the fp32
//     (optionally accumulating) weight-gradient store.
//   Deterministic: each output element is produced by one workgroup with a
//   fixed K order; no atomics.
#include "moe_internal.h"

namespace moe {

constexpr int kGT = 256;          // threads per workgroup
constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLDK = 72;          // LDS row pitch in bf16 elements
constexpr int kTileElems = 128 * kLDK;

enum Epi { EPI_FC1 = 0, EPI_FC2 = 1, EPI_DGRAD2 = 2, EPI_DGRAD1 = 3, EPI_WGRAD = 4 };

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
  uint16_t* out;                  // FC1: A [N,F]; FC2: Y [N,d]; DGRAD2: dH [N,2F]; DGRAD1: dX
  uint16_t* out2;                 // FC1: gu_save or NULL; DGRAD2: A*scale [N,F]
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

// Token-tiled tile lookup: tile -> (expert, row tile, column tile).
// Builds, in LDS, the cumulative tile count over experts.
struct TileIdx { int e, mt, nt, lo, hi; bool valid; };

__device__ TileIdx token_tile(const GGParams& p, int* s_cum /*[E+1]*/, int* s_tmp) {
  const int tid = threadIdx.x;
  // per thread up to 4 consecutive experts
  int loc[4], sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    int t = 0;
    if (e < p.E) {
      const int n = p.offsets[e + 1] - p.offsets[e];
      t = (n > 0 ? (n + kBM - 1) / kBM : 0) * p.ntn;
    }
    loc[q] = t;
    sum += t;
  }
  // block exclusive scan
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
  for (int q = 0; q < 4; ++q) {
    const int e = tid * 4 + q;
    if (e < p.E) s_cum[e] = run;
    run += loc[q];
  }
  if (tid == kGT - 1) s_cum[p.E] = v + add;
  __syncthreads();
  TileIdx ti;
  const int tile = blockIdx.x;
  ti.valid = tile < s_cum[p.E];
  if (!ti.valid) return ti;
  // largest e with s_cum[e] <= tile (and a non-empty expert)
  int lo = 0, hi = p.E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int local = tile - s_cum[e];
  ti.e = e;
  ti.lo = p.offsets[e];
  ti.hi = p.offsets[e + 1];
  const int mts = (ti.hi - ti.lo + kBM - 1) / kBM;
  ti.nt = local / mts;
  ti.mt = local - ti.nt * mts;
  return ti;
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
    const TileIdx ti = token_tile(p, s_cum, s_tmp);
    if (!ti.valid) return;
    e = ti.e;
    seg_lo = ti.lo;
    seg_hi = ti.hi;
    m0 = seg_lo + ti.mt * kBM;
    n0 = ti.nt * (kEpi == EPI_FC1 ? 64 : kBN);
    klen = p.K;
  }

  const uint16_t* bexp = p.b + static_cast<size_t>(e) * p.b_estride;
  const int last_row = seg_hi - 1;
  auto arow = [&](int r) { const int g = m0 + r; return g <= last_row ? g : last_row; };
  auto brow_fc1 = [&](int r) {
    // rows 0..63: gate rows n0+r; rows 64..127: up rows F+n0+r-64
    const int f = n0 + (r & 63);
    const int fc = f < p.F ? f : p.F - 1;
    return (r < 64) ? fc : p.F + fc;
  };
  auto brow_fc2 = [&](int r) { const int n = n0 + r; return n < p.d ? n : p.d - 1; };

  auto load = [&](RegsK& ra, RegsK& rb, int k0) {
    if constexpr (kEpi == EPI_FC1) {
      load_kcontig(ra, p.a, p.lda, arow, k0, klen);
      load_kcontig(rb, bexp, p.ldb, brow_fc1, k0, klen);
    } else if constexpr (kEpi == EPI_FC2) {
      load_kcontig(ra, p.a, p.lda, arow, k0, klen);
      load_kcontig(rb, bexp, p.ldb, brow_fc2, k0, klen);
    } else if constexpr (kEpi == EPI_DGRAD2) {
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
    if constexpr (kEpi == EPI_DGRAD2 || kEpi == EPI_DGRAD1 || kEpi == EPI_WGRAD)
      store_kstrided(rb, Bs);
    else
      store_kcontig(rb, Bs);
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
        if constexpr (kEpi == EPI_FC1) {
          const int f = n0 + wn * 32 + r32;
          if (f < p.F) {
            const float g = acc[mi][0][r], u = acc[mi][1][r];
            p.out[rowz * p.F + f] = f32_to_bf16(siluf_(g) * u);
            if (p.out2) {
              p.out2[rowz * 2 * p.F + f] = f32_to_bf16(g);
              p.out2[rowz * 2 * p.F + p.F + f] = f32_to_bf16(u);
            }
          }
        } else if constexpr (kEpi == EPI_FC2) {
          const float s = p.scale ? p.scale[row] : 1.0f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const int n = n0 + c * 64 + wn * 32 + r32;
            if (n < p.d) p.out[rowz * p.d + n] = f32_to_bf16(acc[mi][c][r] * s);
          }
        } else if constexpr (kEpi == EPI_DGRAD2) {
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

// ---------------------------------------------------------------------------
// fp32 path (MOE_F32): LDS-tiled FMA, 64 x 64 x 16 tiles, 4 x 4 per thread.
// Same tile enumeration and epilogue semantics as the bf16 engine.
// ---------------------------------------------------------------------------
constexpr int kFM = 64, kFN = 64, kFK = 16;

template <int kEpi>
__global__ __launch_bounds__(256) void gg_f32_kernel(int E, int F, int d, int K, int ntn,
                                                     const int32_t* __restrict__ offsets,
                                                     const float* __restrict__ a, int lda,
                                                     const float* __restrict__ b, int ldb,
                                                     size_t b_estride, const float* __restrict__ scale,
                                                     float* __restrict__ out, float* __restrict__ out2) {
  __shared__ float As[kFK][kFM + 4];
  __shared__ float Bs[kFK][kFN + 4];
  __shared__ int s_cum[1025];
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x;
  // tile lookup (row tiles of 64)
  {
    int loc[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      int t = 0;
      if (e < E) {
        const int n = offsets[e + 1] - offsets[e];
        t = (n > 0 ? (n + kFM - 1) / kFM : 0) * ntn;
      }
      loc[q] = t;
      sum += t;
    }
    const int lane = tid & 63, wave = tid >> 6;
    int v = sum;
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(v, o, kWave);
      if (lane >= o) v += u;
    }
    if (lane == 63) s_tmp[wave] = v;
    __syncthreads();
    int add = 0;
    for (int w = 0; w < wave; ++w) add += s_tmp[w];
    int run = v + add - sum;
    for (int q = 0; q < 4; ++q) {
      const int e = tid * 4 + q;
      if (e < E) s_cum[e] = run;
      run += loc[q];
    }
    if (tid == 255) s_cum[E] = v + add;
    __syncthreads();
  }
  const int tile = blockIdx.x;
  if (tile >= s_cum[E]) return;
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_cum[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int seg_lo = offsets[e], seg_hi = offsets[e + 1];
  const int mts = (seg_hi - seg_lo + kFM - 1) / kFM;
  const int local = tile - s_cum[e];
  const int nt = local / mts, mt = local - nt * mts;
  const int m0 = seg_lo + mt * kFM;
  const float* bexp = b + static_cast<size_t>(e) * b_estride;

  const int ty = tid >> 4, tx = tid & 15;
  // B-tile rows held by this thread: FC1 {2tx, 2tx+1, 32+2tx, 33+2tx}; FC2 4tx..4tx+3
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bcol[j] = (kEpi == EPI_FC1) ? ((j >> 1) * 32 + 2 * tx + (j & 1)) : (4 * tx + j);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kFK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;          // 0..1023
      const int r = c >> 4, kk = c & 15;    // 64 rows x 16 k
      const int k = k0 + kk;
      int ar = m0 + r;
      if (ar > seg_hi - 1) ar = seg_hi - 1;
      As[kk][r] = k < K ? a[static_cast<size_t>(ar) * lda + k] : 0.0f;
      int br;
      if constexpr (kEpi == EPI_FC1) {
        int f = nt * 32 + (r & 31);
        if (f > F - 1) f = F - 1;
        br = r < 32 ? f : F + f;
      } else {
        br = nt * kFN + r;
        if (br > d - 1) br = d - 1;
      }
      Bs[kk][r] = k < K ? bexp[static_cast<size_t>(br) * ldb + k] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][bcol[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= seg_hi) continue;
    const size_t rowz = static_cast<size_t>(row);
    if constexpr (kEpi == EPI_FC1) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int f = nt * 32 + 2 * tx + j;
        if (f < F) {
          const float g = acc[i][j], u = acc[i][j + 2];
          out[rowz * F + f] = siluf_(g) * u;
          if (out2) {
            out2[rowz * 2 * F + f] = g;
            out2[rowz * 2 * F + F + f] = u;
          }
        }
      }
    } else {
      const float s = scale ? scale[row] : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * kFN + 4 * tx + j;
        if (n < d) out[rowz * d + n] = acc[i][j] * s;
      }
    }
  }
}

inline int tiles_bound(int64_t N, int E, int bm) {
  return static_cast<int>((N + bm - 1) / bm + E);
}

}  // namespace moe

using namespace moe;

static moe_status check_common(moe_dtype dt, int64_t N, int64_t d, int64_t F, int32_t E) {
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (N < 0 || d < 1 || F < 1 || E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if (N >= (int64_t(1) << 31) || d >= (int64_t(1) << 24) || F >= (int64_t(1) << 24))
    return MOE_ERR_SHAPE;
  if (d % 8 || F % 8) return MOE_ERR_ALIGNMENT;
  return MOE_OK;
}

extern "C" size_t moe_grouped_swiglu_fwd_workspace_size(int64_t N, int64_t F, moe_dtype dt) {
  if (N < 0 || F < 1) return 0;
  return static_cast<size_t>(N) * F * elt_size(dt) + 256;
}

extern "C" size_t moe_grouped_swiglu_bwd_workspace_size(int64_t N, int64_t F, moe_dtype dt,
                                                        int32_t recompute) {
  if (N < 0 || F < 1) return 0;
  // dH [N, 2F] + A*scale [N, F] (+ recomputed G,U [N, 2F])
  const size_t per_row = static_cast<size_t>(F) * (3 + (recompute ? 2 : 0)) * elt_size(dt);
  return static_cast<size_t>(N) * per_row + 1024;
}

static size_t round_up256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

static hipError_t launch_fwd_bf16(hipStream_t stream, int64_t N, int64_t d, int64_t F, int32_t E,
                                  const void* x_perm, const void* w1, const void* w2,
                                  const int32_t* offsets, const float* row_scale, void* y_perm,
                                  void* gu_save, uint16_t* a_buf, bool run_fc2) {
  const size_t lds = 4 * kTileElems * sizeof(uint16_t);
  hipError_t err = allow_lds(gg_kernel<EPI_FC1>, lds);
  if (err != hipSuccess) return err;
  GGParams p{};
  p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = offsets;
  // fc1: C[N, (gate,up) F] = X W1^T, fused SwiGLU
  p.ntn = (int)((F + 63) / 64);
  p.a = static_cast<const uint16_t*>(x_perm); p.lda = (int)d;
  p.b = static_cast<const uint16_t*>(w1); p.ldb = (int)d; p.b_estride = static_cast<size_t>(2 * F) * d;
  p.K = (int)d;
  p.out = a_buf; p.out2 = static_cast<uint16_t*>(gu_save);
  err = launch(gg_kernel<EPI_FC1>, dim3(tiles_bound(N, E, kBM) * p.ntn), dim3(kGT), lds, stream, p);
  if (err != hipSuccess || !run_fc2) return err;
  // fc2: Y[N, d] = A W2^T * row_scale
  err = allow_lds(gg_kernel<EPI_FC2>, lds);
  if (err != hipSuccess) return err;
  GGParams q{};
  q.E = E; q.F = (int)F; q.d = (int)d; q.offsets = offsets;
  q.ntn = (int)((d + kBN - 1) / kBN);
  q.a = a_buf; q.lda = (int)F;
  q.b = static_cast<const uint16_t*>(w2); q.ldb = (int)F; q.b_estride = static_cast<size_t>(d) * F;
  q.K = (int)F;
  q.scale = row_scale;
  q.out = static_cast<uint16_t*>(y_perm);
  return launch(gg_kernel<EPI_FC2>, dim3(tiles_bound(N, E, kBM) * q.ntn), dim3(kGT), lds, stream, q);
}

extern "C" moe_status moe_grouped_swiglu_fwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                             int64_t d, int64_t F, int32_t E,
                                             const void* x_perm, const void* w1, const void* w2,
                                             const int32_t* expert_offsets,
                                             const float* row_scale, void* y_perm,
                                             void* gu_save, void* ws, size_t ws_bytes) {
  moe_status st = check_common(dt, N, d, F, E);
  if (st != MOE_OK) return st;
  if (!x_perm || !w1 || !w2 || !expert_offsets || !y_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(w1) || !aligned16(w2) || !aligned16(expert_offsets) ||
      !aligned16(row_scale) || !aligned16(y_perm) || !aligned16(gu_save) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_grouped_swiglu_fwd_workspace_size(N, F, dt)) return MOE_ERR_WORKSPACE;
  if (N == 0) return MOE_OK;
  if (dt == MOE_BF16) {
    return hip_status(launch_fwd_bf16(stream, N, d, F, E, x_perm, w1, w2, expert_offsets,
                                      row_scale, y_perm, gu_save, static_cast<uint16_t*>(ws),
                                      true));
  }
  float* a_buf = static_cast<float*>(ws);
  const int ntn1 = (int)((F + 31) / 32);
  hipError_t err = launch(gg_f32_kernel<EPI_FC1>, dim3(tiles_bound(N, E, kFM) * ntn1), dim3(256), 0,
                          stream, E, (int)F, (int)d, (int)d, ntn1, expert_offsets,
                          static_cast<const float*>(x_perm), (int)d, static_cast<const float*>(w1),
                          (int)d, static_cast<size_t>(2 * F) * d, (const float*)nullptr, a_buf,
                          static_cast<float*>(gu_save));
  if (err == hipSuccess) {
    const int ntn2 = (int)((d + kFN - 1) / kFN);
    err = launch(gg_f32_kernel<EPI_FC2>, dim3(tiles_bound(N, E, kFM) * ntn2), dim3(256), 0, stream,
                 E, (int)F, (int)d, (int)F, ntn2, expert_offsets, (const float*)a_buf, (int)F,
                 static_cast<const float*>(w2), (int)F, static_cast<size_t>(d) * F, row_scale,
                 static_cast<float*>(y_perm), (float*)nullptr);
  }
  return hip_status(err);
}

extern "C" moe_status moe_grouped_swiglu_bwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                             int64_t d, int64_t F, int32_t E,
                                             const void* dy_perm, const void* x_perm,
                                             const void* w1, const void* w2,
                                             const int32_t* expert_offsets, const void* gu_save,
                                             const float* row_scale, int32_t accumulate,
                                             void* dx_perm, float* dw1, float* dw2, void* ws,
                                             size_t ws_bytes) {
  moe_status st = check_common(dt, N, d, F, E);
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
    err = launch_fwd_bf16(stream, N, d, F, E, x_perm, w1, w2, expert_offsets, nullptr, nullptr,
                          gu_r, As, false);
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
