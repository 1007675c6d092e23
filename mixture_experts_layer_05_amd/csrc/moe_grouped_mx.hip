// MXFP8 grouped SwiGLU forward: the expert GEMMs with microscaled FP8 E4M3
// operands on gfx950's block-scaled MFMA.
//
// Passages: "Megatron-Bridge 深度剖析", section "FP8 训练" (E4M3, scale
// factors, FP8 doubles the matrix rate and halves the traffic of the grouped
// GEMM that BF16 leaves memory-bound), and the section on future directions
// (MXFP8: finer-grained scale factors).  Format (the OCP microscaling one):
// E4M3 elements (largest finite 448), one E8M0 power-of-two scale per 32
// consecutive values along the reduction dimension,
//     X = 2^(floor(log2 amax) - 8),  q = RNE(clamp(v / X, -448, 448)).
//
//   * mx_quant_rows_kernel: bf16 rows -> E4M3 codes [R, K] + scales laid out
//     [K/512][R][16] (a row's scales of 4 consecutive 128-wide K tiles are 16
//     consecutive bytes, so a gathered row brings 4 K tiles' scales in one
//     16-byte read);
//   * mx_pack_kernel: expert weights -> codes in the tile-packed layout of
//     the bf16 path with 128-wide K tiles ([e][panel][K tile][256 rows][128
//     bytes], gate/up panels for fc1) + scales [e][panel][K tile][256][4];
//   * ggmx_kernel: the persistent grouped GEMM of moe_grouped_fwd.hip with
//     byte-wide operands: 256 x 256 tiles, 8 wavefronts of 128 x 64, each
//     K tile 128 values (one 128-byte line per staged row), two 2-slot rings
//     with the weights' 1 KB of scales per slot (130 KB) and two 4 KB
//     buffers of token-row scales, each filled once per 4 K tiles.  v_mfma_scale_f32_32x32x64
//     _f8f6f4 takes 32 bytes of a row per lane: lanes r and r + 32 hold
//     bytes 0-15 (k 0-15 and 16-31: the first 32-value block) and 16-31 (the
//     second block), and lane r + 32 b supplies the scale of row r's block b
//     (checked on the GPU with an in-bounds probe).  fc1's epilogue computes
//     A = silu(G) U and quantises it per row and 32 columns for fc2 (scale
//     from the two lanes holding the block); fc2's writes bf16 rows scaled by
//     the routing weight.  A K tile moves 66 KB into LDS for twice the FLOPs
//     of a bf16 K tile.
#include <algorithm>

#include "moe_gemm_common.h"
#include "moe_sched.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kMxBM = 256, kMxBN = 256;          // tile rows (tokens) x weight rows
constexpr int kMxBK = 128;                       // K values (= bytes) per K tile
constexpr int kMxWaves = 8, kMxThreads = 512;    // 2 x 4 waves of 128 x 64 (256 registers each)
constexpr int kMxRB = 4, kMxCB = 2;              // 32 x 32 blocks per wave
constexpr int kMxTile = kMxBM * kMxBK;           // bytes of one operand tile
constexpr int kMxSlot = 2 * kMxTile + 1024;      // A, B, B scales
constexpr int kMxGroup = 4;                      // K tiles per group of row scales
constexpr int kMxSgBuf = kMxBM * 4 * kMxGroup;   // one group's row scales (4 KB)
constexpr int kMxLds = 2 * kMxSlot + 2 * kMxSgBuf;
constexpr int kMxScanInts = 1040 + 64;

// K tiles and sizes of the packed weights (panels of 256 rows; fc1 panels
// hold 128 gate rows and the matching 128 up rows)
inline int64_t mx_panels(int64_t rows, int gated) {
  return gated ? (rows / 2 + kMxBN / 2 - 1) / (kMxBN / 2) : (rows + kMxBN - 1) / kMxBN;
}
inline int64_t mx_ktiles(int64_t K) { return (K + kMxBK - 1) / kMxBK; }
inline int64_t mx_sgroups(int64_t K) { return (K + kMxBK * kMxGroup - 1) / (kMxBK * kMxGroup); }

__device__ __forceinline__ int mx_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// E8M0 scale code of a block with largest magnitude amax (0 for amax 0)
__device__ __forceinline__ int mx_scale_code(float amax) {
  if (!(amax > 0.0f)) return 0;
  const int e = ilogbf(amax) - 8 + 127;
  return e < 0 ? 0 : (e > 254 ? 254 : e);
}

// four fp32 values times 2^(127 - code), clamped to +-448, rounded to E4M3
// (round to nearest even) -> 4 code bytes
__device__ __forceinline__ uint32_t mx_pack4(float a, float b, float c, float d, int code) {
  const int s = 127 - code;
  const float x0 = fminf(fmaxf(ldexpf(a, s), -448.0f), 448.0f);
  const float x1 = fminf(fmaxf(ldexpf(b, s), -448.0f), 448.0f);
  const float x2 = fminf(fmaxf(ldexpf(c, s), -448.0f), 448.0f);
  const float x3 = fminf(fmaxf(ldexpf(d, s), -448.0f), 448.0f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<uint32_t>(w);
}

// One thread per 32-value block of a bf16 row: R rows of K values; the
// scale slots of the last group past K get 0.  Block b's scale byte sits at
// [b / 16][r][b % 16].
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(int64_t R, int K,
                                                            const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
  const int nb = K / 32, nbg = (K + 511) / 512 * 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= R * nbg) return;
  const int64_t r = i / nbg;
  const int b = static_cast<int>(i - r * nbg);
  if (b >= nb) {
    scales[(static_cast<int64_t>(b / 16) * R + r) * 16 + (b & 15)] = 0;
    return;
  }
  const u32x4* src = reinterpret_cast<const u32x4*>(x + r * K + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = src[q];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      v[8 * q + 2 * t] = bf16lo(w[t]);
      v[8 * q + 2 * t + 1] = bf16hi(w[t]);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(v[t]));
  const int code = mx_scale_code(amax);
  u32x4 o[2];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    o[q / 4][q % 4] = mx_pack4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], code);
  u32x4* dst = reinterpret_cast<u32x4*>(codes + r * K + b * 32);
  dst[0] = o[0];
  dst[1] = o[1];
  scales[(static_cast<int64_t>(b / 16) * R + r) * 16 + (b & 15)] = static_cast<uint8_t>(code);
}

// One thread per 32-value block of a packed weight row: quantise and place.
__global__ __launch_bounds__(256) void mx_pack_kernel(int64_t total, int rows, int K, int gated,
                                                      int npanel, int nkt,
                                                      const uint16_t* __restrict__ w,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  const int j = static_cast<int>(i & 3);              // block in the K tile
  int64_t q = i >> 2;
  const int r = static_cast<int>(q % kMxBN);
  q /= kMxBN;
  const int kt = static_cast<int>(q % nkt);
  q /= nkt;
  const int t = static_cast<int>(q % npanel);
  const int64_t e = q / npanel;
  int row;
  if (gated) {
    const int F = rows / 2, h = kMxBN / 2;
    const int f = t * h + (r < h ? r : r - h);
    row = f < F ? (r < h ? f : F + f) : -1;
  } else {
    row = t * kMxBN + r;
    row = row < rows ? row : -1;
  }
  const int k0 = kt * kMxBK + j * 32;
  float v[32];
#pragma unroll
  for (int t2 = 0; t2 < 32; ++t2) v[t2] = 0.0f;
  if (row >= 0 && k0 < K) {
    const u32x4* src = reinterpret_cast<const u32x4*>(w + (e * rows + row) * K + k0);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const u32x4 ww = src[qq];
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        v[8 * qq + 2 * t2] = bf16lo(ww[t2]);
        v[8 * qq + 2 * t2 + 1] = bf16hi(ww[t2]);
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int t2 = 0; t2 < 32; ++t2) amax = fmaxf(amax, fabsf(v[t2]));
  const int code = mx_scale_code(amax);
  u32x4 o[2];
#pragma unroll
  for (int qq = 0; qq < 8; ++qq)
    o[qq / 4][qq % 4] = mx_pack4(v[4 * qq], v[4 * qq + 1], v[4 * qq + 2], v[4 * qq + 3], code);
  const int64_t tile = (e * npanel + t) * nkt + kt;
  u32x4* dst = reinterpret_cast<u32x4*>(codes + (tile * kMxBN + r) * kMxBK + j * 32);
  dst[0] = o[0];
  dst[1] = o[1];
  scales[(tile * kMxBN + r) * 4 + j] = static_cast<uint8_t>(code);
}

enum MxEpi { MX_FC1 = 0, MX_FC2 = 1 };

struct MxParams {
  int E, F, d, K, ntn, nkt;
  const int32_t* offsets;
  const uint8_t* a;            // codes: fc1 token rows [a_rows, K] (gathered), fc2 A [N, K]
  const uint8_t* as;           // scales [ceil(nkt / 4)][a_rows or N][16]
  int a_rows;                  // rows indexed by the scale layout (T for fc1 gathers, N otherwise)
  const int32_t* gather;       // fc1: source row of each row, or NULL
  const uint8_t* b;            // packed weight codes
  const uint8_t* bs;           // packed weight scales
  int64_t b_estride;           // bytes of one expert's packed codes
  const float* scale;          // fc2 row scale or NULL
  uint8_t* out_q;              // fc1: A codes [N, F]
  uint8_t* out_s;              // fc1: A scales [ceil(F / 512)][N][16]
  uint16_t* out;               // fc2: Y [N, d] bf16
  int N;
  int* counter;                // this launch's 8 tile counters, one per XCD (zero at launch)
};

struct MxTile {
  TileIdx ti;
  __amdgpu_buffer_rsrc_t ra, rb, rsa, rsb;
  int vo[8];                   // per-lane byte offsets of the data loads (4 A, 4 B)
  int vs;                      // per-lane offset of the scale load (waves 0-3: A rows; wave 4: B)
  int j;                       // the tile's position in this workgroup's walk
  int L;                       // the tile's index in the cost order
};

template <int kEpi>
__device__ __forceinline__ void ggmx_body(const MxParams& p) {
  extern __shared__ __align__(16) uint8_t lds[];
  int* s_cum = reinterpret_cast<int*>(lds + kMxLds);
  int* s_tmp = s_cum + 1040;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;      // wm: 128-row half, wn: 64-column quarter
  const int r32 = lane & 31, h = lane >> 5;
  const int K = p.K, nk = p.nkt;

  const int ng = (nk + kMxGroup - 1) / kMxGroup;  // row-scale groups per tile
  // this XCD's range of tiles (workgroup b runs on XCD b mod 8); its
  // workgroups take tiles pos and pos + G of the range first, then one fetch
  // from the XCD's counter per tile started
  const int xcd = static_cast<int>(blockIdx.x & 7), pos = static_cast<int>(blockIdx.x >> 3);
  const int G = static_cast<int>(gridDim.x >> 3);
  tile_prefix<kMxThreads>(p.offsets, p.E, kMxBM, p.ntn, s_cum, s_tmp);
  const XcdRange xr = xcd_range(s_cum[p.E], xcd);
  const int total = xr.xcnt;
  if (pos >= total) return;

  // data loads: block bb = wave + 8 j (j = 0..3) of 8 rows x 128 bytes;
  // lane l: row 8 bb + l / 8, physical chunk l % 8 = logical chunk ^ swizzle
  const int lr = lane >> 3, pc = lane & 7;
  int rowl[4], kcl[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bb = wave + kMxWaves * j;
    rowl[j] = bb * 8 + lr;
    kcl[j] = pc ^ mx_swz(rowl[j]);
  }
  const bool gath = p.gather != nullptr;

  auto setup = [&](int j, int L, MxTile& st) {
    st.j = j;
    st.L = L;
    st.ti = tile_decode(p.offsets, p.E, kMxBM, p.ntn, xr.xbeg + L, s_cum);
    const TileIdx& ti = st.ti;
    const int m0 = ti.m0, last = ti.mend - 1 - m0;
    st.ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(gath ? p.a : p.a + static_cast<size_t>(m0) * K), 0,
        (gath ? p.a_rows : ti.mend - m0) * K, kRsrcWord3);
    st.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.b + ti.e * p.b_estride), 0,
                                              static_cast<int>(p.b_estride), kRsrcWord3);
    st.rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.as), 0, ng * p.a_rows * 16,
                                               kRsrcWord3);
    st.rsb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(p.bs + ti.e * (p.b_estride / kMxBK) * 4), 0,
        static_cast<int>(p.b_estride / kMxBK * 4), kRsrcWord3);
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const int r = rowl[j2];
      const int src = r > last ? -1 : gath ? p.gather[m0 + r] : r;
      st.vo[j2] = src >= 0 && (!gath || src < p.a_rows) ? src * K + kcl[j2] * 16 : kOob;
      st.vo[4 + j2] = (ti.nt * nk * kMxBN + r) * kMxBK + kcl[j2] * 16;
    }
    if (wave < 4) {                     // A scales: one row per lane, 16 bytes (4 K tiles)
      const int r = wave * 64 + lane;
      const int src = r > last ? -1 : gath ? p.gather[m0 + r] : m0 + r;
      st.vs = src >= 0 && src < p.a_rows ? src * 16 : kOob;
    } else {                            // wave 4: the B scales' 1 KB, 16 bytes per lane
      st.vs = (ti.nt * nk * kMxBN) * 4 + lane * 16;
    }
  };
  auto slot_base = [&](int slot) { return lds + slot * kMxSlot; };
  auto issue = [&](const MxTile& st, int kt, int slot) {
    uint8_t* sl = slot_base(slot);
    const int k0 = kt * kMxBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int bb = wave + kMxWaves * j;
      const int va = (k0 + kcl[j] * 16 < K) ? st.vo[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, (lds_void*)(sl + bb * 1024), 16, va, k0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rb, (lds_void*)(sl + kMxTile + bb * 1024), 16,
                                               st.vo[4 + j], kt * kMxBN * kMxBK, 0, 0);
    }
    if (wave < 4) {
      if (kt % kMxGroup == 0) {         // the row scales of K tiles kt .. kt + 3
        const int gi = st.j * ng + kt / kMxGroup;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            st.rsa, (lds_void*)(lds + 2 * kMxSlot + (gi & 1) * kMxSgBuf + wave * 1024), 16, st.vs,
            kt / kMxGroup * p.a_rows * 16, 0, 0);
      }
    } else if (wave == 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rsb, (lds_void*)(sl + 2 * kMxTile), 16,
                                               st.vs, kt * kMxBN * 4, 0, 0);
  };

  // operand rows of this wave
  int a_rd[kMxRB], b_rd[kMxCB];
#pragma unroll
  for (int i = 0; i < kMxRB; ++i) a_rd[i] = wm * 128 + i * 32 + r32;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if constexpr (kEpi == MX_FC1) b_rd[c] = (c == 0 ? 0 : kMxBN / 2) + wn * 32 + r32;
    else b_rd[c] = wn * 64 + c * 32 + r32;
  }
  auto rd16 = [&](const uint8_t* base, int r, int chunk) {
    return *reinterpret_cast<const u32x4*>(base + r * kMxBK + ((chunk ^ mx_swz(r)) << 4));
  };

  f32x16 acc[kMxRB][kMxCB];
  auto compute = [&](int slot, int nrb, int gi, int kq) {
    const uint8_t* As = slot_base(slot);
    const uint8_t* Bs = As + kMxTile;
    const uint32_t* Ssb = reinterpret_cast<const uint32_t*>(As + 2 * kMxTile);
    const uint32_t* Ssa = reinterpret_cast<const uint32_t*>(lds + 2 * kMxSlot + (gi & 1) * kMxSgBuf);
    uint32_t sb[kMxCB], sa[kMxRB];
#pragma unroll
    for (int c = 0; c < kMxCB; ++c) sb[c] = Ssb[b_rd[c]];
#pragma unroll
    for (int i = 0; i < kMxRB; ++i) sa[i] = Ssa[a_rd[i] * kMxGroup + kq];
#pragma unroll
    for (int j = 0; j < 2; ++j) {                 // two 64-value MFMA steps per K tile
      i32x8 bv[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 lo = rd16(Bs, b_rd[c], 4 * j + h), hi = rd16(Bs, b_rd[c], 4 * j + 2 + h);
        bv[c] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                      (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      const int sh = 8 * (2 * j + h);
#pragma unroll
      for (int rb = 0; rb < kMxRB; ++rb) {
        if (rb < nrb) {
          const u32x4 lo = rd16(As, a_rd[rb], 4 * j + h), hi = rd16(As, a_rd[rb], 4 * j + 2 + h);
          const i32x8 av = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                            (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          const int sca = static_cast<int>((sa[rb] >> sh) & 255);
#pragma unroll
          for (int c = 0; c < 2; ++c)
            acc[rb][c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bv[c], av, acc[rb][c], 0, 0, 0, static_cast<int>((sb[c] >> sh) & 255), 0, sca);
        }
      }
    }
  };

  auto live_blocks = [&](const TileIdx& ti) {
    const int rows = ti.mend - ti.m0 - wm * 128;
    return rows <= 0 ? 0 : min(kMxRB, (rows + 31) >> 5);
  };

  // epilogues (staged in the free slot)
  auto epilogue = [&](const TileIdx& ti, int nrb, int free_slot) {
    uint8_t* st = slot_base(free_slot);
    const int m0 = ti.m0;
    if constexpr (kEpi == MX_FC1) {
      // A = silu(G) U of this wave's 32 columns, quantised per row (one block):
      // lane (r32, h) holds columns 8 qq + 4 h + i; its partner r32 + 32 - 32 h
      // the other 16
      const int n0 = ti.nt * (kMxBN / 2);
#pragma unroll
      for (int rb = 0; rb < kMxRB; ++rb) {
        if (rb >= nrb) continue;
        const int lrow = wm * 128 + rb * 32 + r32;
        float a[16];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float g = acc[rb][0][i];
          a[i] = g * sigmoid_fast(g) * acc[rb][1][i];
          amax = fmaxf(amax, fabsf(a[i]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
        const int code = mx_scale_code(amax);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int cb = wn * 32 + 8 * qq + 4 * h;           // byte (= column) in the tile row
          *reinterpret_cast<uint32_t*>(st + lrow * kMxBK + (((cb >> 4) ^ mx_swz(lrow)) << 4) + (cb & 15)) =
              mx_pack4(a[4 * qq], a[4 * qq + 1], a[4 * qq + 2], a[4 * qq + 3], code);
        }
        if (h == 0) st[2 * kMxTile + lrow * 4 + wn] = static_cast<uint8_t>(code);
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      // codes: 256 rows x 128 bytes, 16 bytes per lane; scales: 4 bytes per row
#pragma unroll
      for (int i = tid; i < kMxBM * 8; i += kMxThreads) {
        const int lr2 = i >> 3, ch = i & 7;
        const int row = m0 + lr2, col = n0 + ch * 16;
        if (row < ti.mend && col < p.F)
          *reinterpret_cast<u32x4*>(p.out_q + static_cast<size_t>(row) * p.F + col) =
              *reinterpret_cast<const u32x4*>(st + lr2 * kMxBK + ((ch ^ mx_swz(lr2)) << 4));
      }
      if (tid < kMxBM && m0 + tid < ti.mend) {
        uint32_t sc = *reinterpret_cast<const uint32_t*>(st + 2 * kMxTile + tid * 4);
        // blocks past F: zero scale (their codes are not read: fc2's K ends at F)
        const int nvalid = (p.F - n0) / 32;
        if (nvalid < 4) sc &= nvalid <= 0 ? 0u : (0xffffffffu >> (32 - 8 * nvalid));
        const int kt2 = n0 / kMxBK;           // fc2's K tile
        *reinterpret_cast<uint32_t*>(
            p.out_s + (static_cast<size_t>(kt2 / kMxGroup) * p.N + m0 + tid) * 16 + 4 * (kt2 % kMxGroup)) = sc;
      }
    } else {
      // Y rows (bf16, routing-weight scaled) through two 32 KB halves of the
      // free slot, 128 rows per pass, 512-byte rows, chunks XOR-swizzled
      const int n0 = ti.nt * kMxBN;
      const int wrow0 = wm * 128;
#pragma unroll
      for (int ps = 0; ps < 2; ++ps) {
        if (wm == ps) {
#pragma unroll
          for (int rb = 0; rb < kMxRB; ++rb) {
            if (rb >= nrb) continue;
            const int lp = wrow0 - ps * 128 + rb * 32 + r32;
            const int row = m0 + wrow0 + rb * 32 + r32;
            const float sc = (p.scale && row < ti.mend) ? p.scale[row] : 1.0f;
            uint8_t* srow = st + (lp >> 6) * kMxTile + (lp & 63) * 512;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) {
                const int nb = (wn * 64 + c * 32 + 8 * qq + 4 * h) * 2;   // byte in the row
                const f32x16& Y = acc[rb][c];
                *reinterpret_cast<u32x2*>(srow + ((((nb >> 4) ^ (lp & 15))) << 4) + (nb & 15)) =
                    pack4_bf16(Y[4 * qq] * sc, Y[4 * qq + 1] * sc, Y[4 * qq + 2] * sc,
                               Y[4 * qq + 3] * sc);
              }
            }
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int i = tid; i < 128 * 32; i += kMxThreads) {
          const int lp = i >> 5, ch = i & 31;
          const int row = m0 + ps * 128 + lp, col = n0 + ch * 8;
          if (row < ti.mend && col < p.d)
            *reinterpret_cast<u32x4*>(p.out + static_cast<size_t>(row) * p.d + col) =
                *reinterpret_cast<const u32x4*>(st + (lp >> 6) * kMxTile + (lp & 63) * 512 +
                                                ((ch ^ (lp & 15)) << 4));
        }
        if (ps == 0) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      }
    }
  };

  MxTile cur, nxt;
  setup(0, pos, cur);
  __syncthreads();
  issue(cur, 0, 0);
  bool has_nxt = pos + G < total;
  if (has_nxt) setup(1, pos + G, nxt);
  int* s_fetch = s_tmp + 32;
  int g = 0;
#pragma unroll 1
  for (int j = 0;; ++j) {
    const int nrb = live_blocks(cur.ti);
    int fetched = 0;
    if (has_nxt && tid == 0) fetched = atomicAdd(p.counter + xcd, 1);   // the tile after nxt
#pragma unroll
    for (int i = 0; i < kMxRB; ++i)
#pragma unroll
      for (int c = 0; c < kMxCB; ++c) acc[i][c] = f32x16{};
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt, ++g) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + 1 < nk) issue(cur, kt + 1, (g + 1) & 1);
      else if (has_nxt) issue(nxt, 0, (g + 1) & 1);
      compute(g & 1, nrb, j * ng + kt / kMxGroup, kt % kMxGroup);
    }
    if (tid == 0) *s_fetch = 2 * G + fetched;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    epilogue(cur.ti, nrb, (g - 1) & 1);
    if (!has_nxt) break;
    const int L2 = *s_fetch;
    cur = nxt;
    has_nxt = L2 < total;
    if (has_nxt) setup(j + 2, L2, nxt);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int kEpi>
__global__ __launch_bounds__(kMxThreads, 1) void ggmx_kernel(MxParams p) {
  ggmx_body<kEpi>(p);
}

__global__ void zero_counters_kernel(int* __restrict__ c, int n) {
  if (static_cast<int>(threadIdx.x) < n) c[threadIdx.x] = 0;
}

hipError_t launch_zero_counters(hipStream_t stream, int* c, int n) {
  return launch(zero_counters_kernel, dim3(1), dim3(64), 0, stream, c, n);
}

static unsigned mx_grid(int64_t tiles) {
  const int64_t cus = device_cu_count();
  const int64_t g = std::min<int64_t>(cus, (tiles + 7) / 8 * 8);
  return static_cast<unsigned>(std::max<int64_t>(8, g / 8 * 8));
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_quantize_mx_scales_size(int64_t R, int64_t K) {
  if (R < 1 || K < 1) return 0;
  return static_cast<size_t>(mx_sgroups(K) * R * 16);
}

extern "C" moe_status moe_quantize_mx(hipStream_t stream, int64_t R, int64_t K, const void* x,
                                      void* codes, void* scales) {
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (R < 1 || K < 1 || R >= (int64_t(1) << 31) || K >= (int64_t(1) << 20)) return MOE_ERR_SHAPE;
  if (K % 32) return MOE_ERR_ALIGNMENT;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_ALIGNMENT;
  if (mx_sgroups(K) * R * 16 >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  const int64_t n = R * mx_sgroups(K) * 16;
  return hip_status(launch(mx_quant_rows_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                           dim3(256), 0, stream, R, (int)K, static_cast<const uint16_t*>(x),
                           static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales)));
}

extern "C" size_t moe_pack_weights_mx_size(int32_t E, int64_t rows, int64_t K, int32_t gated,
                                           int32_t scales) {
  if (E < 1 || rows < 1 || K < 1 || (gated && rows % 2)) return 0;
  const int64_t per = mx_panels(rows, gated ? 1 : 0) * mx_ktiles(K) * kMxBN;
  return static_cast<size_t>(E * per * (scales ? 4 : kMxBK));
}

extern "C" moe_status moe_pack_weights_mx(hipStream_t stream, int32_t E, int64_t rows, int64_t K,
                                          int32_t gated, const void* w, void* w_codes,
                                          void* w_scales) {
  if (!w || !w_codes || !w_scales) return MOE_ERR_INVALID_ARG;
  if (E < 1 || rows < 1 || K < 1 || (gated && rows % 2)) return MOE_ERR_SHAPE;
  if (rows >= (int64_t(1) << 20) || K >= (int64_t(1) << 20)) return MOE_ERR_SHAPE;
  if (K % 32) return MOE_ERR_ALIGNMENT;
  if (!aligned16(w) || !aligned16(w_codes) || !aligned16(w_scales)) return MOE_ERR_ALIGNMENT;
  const int g = gated ? 1 : 0;
  const int64_t np = mx_panels(rows, g), nkt = mx_ktiles(K);
  const int64_t total = static_cast<int64_t>(E) * np * nkt * kMxBN * 4;
  return hip_status(launch(mx_pack_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                           dim3(256), 0, stream, total, (int)rows, (int)K, g, (int)np, (int)nkt,
                           static_cast<const uint16_t*>(w), static_cast<uint8_t*>(w_codes),
                           static_cast<uint8_t*>(w_scales)));
}

extern "C" size_t moe_grouped_swiglu_fwd_mx_workspace_size(int64_t N, int64_t F) {
  if (N < 0 || F < 1) return 0;
  const size_t q = (static_cast<size_t>(N) * F + 255) & ~static_cast<size_t>(255);
  return q + static_cast<size_t>(mx_sgroups(F) * std::max<int64_t>(N, 1) * 16) + 256;
}

extern "C" moe_status moe_grouped_swiglu_fwd_mx(hipStream_t stream, int64_t N, int64_t d,
                                                int64_t F, int32_t E, int64_t T,
                                                const void* xq, const void* xs,
                                                const int32_t* row_token, const void* w1q,
                                                const void* w1s, const void* w2q,
                                                const void* w2s, const int32_t* expert_offsets,
                                                const float* row_scale, void* y_perm, void* ws,
                                                size_t ws_bytes) {
  if (!xq || !xs || !w1q || !w1s || !w2q || !w2s || !expert_offsets || !y_perm)
    return MOE_ERR_INVALID_ARG;
  if (N < 0 || d < 1 || F < 1 || E < 1 || E > 1024) return MOE_ERR_SHAPE;
  if (N >= (int64_t(1) << 31) || d >= (int64_t(1) << 20) || F >= (int64_t(1) << 20))
    return MOE_ERR_SHAPE;
  if (d % 32 || F % 32) return MOE_ERR_ALIGNMENT;
  const int64_t rows_a = row_token ? T : N;
  if (row_token && T < 1) return MOE_ERR_SHAPE;
  const int64_t b1 = mx_panels(2 * F, 1) * mx_ktiles(d) * kMxBN * kMxBK;
  const int64_t b2 = mx_panels(d, 0) * mx_ktiles(F) * kMxBN * kMxBK;
  // byte offsets in 32 bits: one expert's packed codes, the token rows, A
  if (b1 >= (int64_t(1) << 31) || b2 >= (int64_t(1) << 31) || rows_a * d >= (int64_t(1) << 31) ||
      N * F >= (int64_t(1) << 31) || mx_sgroups(d) * rows_a * 16 >= (int64_t(1) << 31) ||
      mx_sgroups(F) * N * 16 >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  if (!aligned16(xq) || !aligned16(xs) || !aligned16(row_token) || !aligned16(w1q) ||
      !aligned16(w1s) || !aligned16(w2q) || !aligned16(w2s) || !aligned16(expert_offsets) ||
      !aligned16(row_scale) || !aligned16(y_perm) || !aligned16(ws))
    return MOE_ERR_ALIGNMENT;
  if (!ws || ws_bytes < moe_grouped_swiglu_fwd_mx_workspace_size(N, F)) return MOE_ERR_WORKSPACE;
  if (N == 0) return MOE_OK;
  const size_t lds = kMxLds + kMxScanInts * sizeof(int);
  hipError_t err = allow_lds(ggmx_kernel<MX_FC1>, lds);
  if (err == hipSuccess) err = allow_lds(ggmx_kernel<MX_FC2>, lds);
  if (err != hipSuccess) return MOE_ERR_HIP;
  uint8_t* aq = static_cast<uint8_t*>(ws);
  uint8_t* as = aq + ((static_cast<size_t>(N) * F + 255) & ~static_cast<size_t>(255));
  // the two launches' tile counters (8 each) sit after A's scales, in the workspace's slack
  int* counters = reinterpret_cast<int*>(as + mx_sgroups(F) * N * 16);
  err = launch_zero_counters(stream, counters, 16);
  if (err != hipSuccess) return MOE_ERR_HIP;
  MxParams p{};
  p.E = E; p.F = (int)F; p.d = (int)d; p.K = (int)d; p.N = (int)N;
  p.ntn = (int)((F + kMxBN / 2 - 1) / (kMxBN / 2));
  p.nkt = (int)mx_ktiles(d);
  p.offsets = expert_offsets;
  p.a = static_cast<const uint8_t*>(xq); p.as = static_cast<const uint8_t*>(xs);
  p.a_rows = (int)rows_a; p.gather = row_token;
  p.b = static_cast<const uint8_t*>(w1q); p.bs = static_cast<const uint8_t*>(w1s);
  p.b_estride = b1;
  p.out_q = aq; p.out_s = as;
  p.counter = counters;
  const int64_t tiles1 = (N + kMxBM - 1) / kMxBM + E;
  err = launch(ggmx_kernel<MX_FC1>, dim3(mx_grid(tiles1 * p.ntn)), dim3(kMxThreads), lds, stream, p);
  if (err != hipSuccess) return MOE_ERR_HIP;
  MxParams q{};
  q.E = E; q.F = (int)F; q.d = (int)d; q.K = (int)F; q.N = (int)N;
  q.ntn = (int)((d + kMxBN - 1) / kMxBN);
  q.nkt = (int)mx_ktiles(F);
  q.offsets = expert_offsets;
  q.a = aq; q.as = as; q.a_rows = (int)N; q.gather = nullptr;
  q.b = static_cast<const uint8_t*>(w2q); q.bs = static_cast<const uint8_t*>(w2s);
  q.b_estride = b2;
  q.scale = row_scale;
  q.counter = counters + 8;
  q.out = static_cast<uint16_t*>(y_perm);
  return hip_status(launch(ggmx_kernel<MX_FC2>, dim3(mx_grid(tiles1 * q.ntn)), dim3(kMxThreads), lds,
                           stream, q));
}
