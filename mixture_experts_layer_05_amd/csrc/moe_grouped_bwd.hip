// Grouped SwiGLU expert FFN, backward: fc2 dgrad + SwiGLU backward, fc1
// dgrad, fc2 and fc1 wgrad.
//
// Passages: "Megatron-Bridge 深度剖析", section "计算融合 / Grouped GEMM" (one
// grouped launch over all experts' segments), "通信隐藏与混合精度 / TP 通信重叠"
// (the backward's dgrad and wgrad GEMMs) and "其他融合优化"
// (gradient_accumulation_fusion: fp32 weight-gradient accumulation).
//
// bf16 engines (gfx950):
//   * dgrad (ggb_kernel): workgroup = 8 wavefronts (2 x 4), output tile
//     128 x 256, wave tile 64 x 64 = 2 x 2 v_mfma_f32_32x32x16_bf16
//     accumulators; a 3-deep ring of 32-wide K tiles filled global -> LDS
//     directly (no staging registers), two workgroups per CU, so one's
//     epilogue overlaps the other's K loop;
//   * wgrad (ggw_persistent_kernel): 256 x 256 tiles, 16 wavefronts, a
//     2-slot ring of 64-wide K tiles, one persistent workgroup per CU taking
//     tiles longest first (see its comment);
//   * a K-contiguous operand (dY and dH rows in dgrad) is staged as in the
//     forward: [row][32 k] with XOR-swizzled 16-byte chunks, read with
//     ds_read_b128;
//   * a K-strided operand (the weights in dgrad; both operands in wgrad,
//     whose K is the expert's token rows) is staged as it lies in memory,
//     [k][columns], and read with ds_read_b64_tr_b16, which transposes
//     4 x 4 blocks of 16-bit elements across each 16-lane group: lane p of
//     a group addresses k row p / 4, columns 4 (p % 4) .. +3, and receives
//     column p at 4 consecutive k.  Two such reads give one MFMA operand
//     (8 k for one row/column).  Chunk c of k row k sits at position
//     c ^ 4 (k % 4), so the 4 k rows x 64 bytes of each half-wave's read
//     fall on 64 distinct banks;
//   * K tails: a K-contiguous chunk past K gets an offset past the buffer
//     (reads zero); a K-strided operand's buffer descriptor is rebuilt per K
//     tile to cover exactly the K rows left, so rows past K (the next
//     expert's tokens in wgrad) read zero;
//   * dgrad tiles over ragged expert segments are decoded on the device from
//     expert_offsets and handed to XCDs in contiguous ranges; a wave whose
//     32-row blocks lie past the segment skips their MFMAs.  wgrad tiles are
//     per expert (an empty expert yields zeros);
//   * epilogues fuse the SwiGLU backward (dG = dA U silu'(G), dU = dA
//     silu(G)) with A * row_scale for the fc2 wgrad, and the fp32
//     (optionally accumulating) weight-gradient store.
//   Deterministic: each output element is produced by one workgroup with a
//   fixed K order.  The one atomic, the wgrad's tile counter, decides which
//   workgroup computes a tile, not how it is computed.
#include <algorithm>

#include "moe_sched.h"

namespace moe {

constexpr int kWM = 2, kWN = 4, kRB = 2, kCB = 2;
constexpr int kGT = 64 * kWM * kWN;           // threads per workgroup
constexpr int kWaves = kWM * kWN;
constexpr int kBM = kWM * kRB * 32;           // 128: rows of the A operand
constexpr int kBN = kWN * kCB * 32;           // 256: rows of the B operand
constexpr int kBK = 32;
constexpr int kStages = 3;
constexpr int kATileE = kBM * kBK;            // bf16 per stage
constexpr int kBTileE = kBN * kBK;
constexpr int kStageE = kATileE + kBTileE;
constexpr int kALoads = kATileE / 512 / kWaves;   // 1 KB blocks per wave per K tile
constexpr int kBLoads = kBTileE / 512 / kWaves;
constexpr int kLoads = kALoads + kBLoads;
static_assert(kALoads == 1 && kBLoads == 2, "block split");
// loads per wave per K tile x (kStages - 2) tiles left in flight
#define MOE_BWD_VMCNT 3
static_assert(MOE_BWD_VMCNT == kLoads * (kStages - 2), "ring wait count");
#define MOE_STR2(x) #x
#define MOE_STR(x) MOE_STR2(x)
constexpr size_t kBwdLds = kStages * kStageE * sizeof(uint16_t);


enum Epi { EPI_DGRAD2 = 2, EPI_DGRAD1 = 3 };

struct GGParams {
  int E, F, d;
  int K;                          // contraction length
  int ntn;                        // column tiles per row tile
  const int32_t* offsets;         // [E+1]
  const uint16_t* a;              // A operand (rows of C): token rows [N, K]
  int lda;
  const uint16_t* b;              // B operand (columns of C): weights [E][K, ldb]
  int ldb;
  size_t b_estride;
  const float* scale;             // [N] row scale or NULL (DGRAD2)
  const uint16_t* gu_in;          // [N, 2F] (DGRAD2)
  uint16_t* out;                  // DGRAD2: dH [N,2F]; DGRAD1: dX [N,d]
  uint16_t* out2;                 // DGRAD2: A*scale [N,F]
  int* zero;                      // 2 ints set to zero by workgroup 0 (or NULL): the
                                  // following wgrad launches' tile counters
};

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((ext_vector_type(8))) short i16x8;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// row-layout staged element offset of row r, 16-byte chunk kc
__device__ __forceinline__ int swz(int r, int kc) { return r * kBK + ((kc ^ swz_f(r)) << 3); }

// MFMA operand (lane l: row R + l % 32, k = 16 kk + 8 (l / 32) .. +7) from a
// row-layout staged tile
__device__ __forceinline__ bf16x8 frag_row(const uint16_t* T, int R, int kk, int lane) {
  return *reinterpret_cast<const bf16x8*>(T + swz(R + (lane & 31), 2 * kk + (lane >> 5)));
}

// Per-lane part of a transposed read's LDS offset for the operand rows
// starting at R (a multiple of 32) of a [kBK][kW] staged tile: k row
// 8 (l / 32) + (l % 16) / 4, column R + 16 ((l / 16) % 2) + 4 (l % 4),
// chunk XOR 4 (k % 4) with k % 4 = (l % 16) / 4.
template <int kW>
__device__ __forceinline__ int tr_base(int R, int lane) {
  const int q = lane & 15, g = lane >> 4;
  const int krow = 8 * (g >> 1) + (q >> 2);
  const int col = R + 16 * (g & 1) + 4 * (q & 3);
  return krow * kW + ((((col >> 3) ^ ((q >> 2) << 2))) << 3) + (col & 7);
}
// the same operand as frag_row, from a [kBK][kW] staged tile
template <int kW>
__device__ __forceinline__ bf16x8 frag_tr(const uint16_t* T, int base, int kk) {
  const uint16_t* p0 = T + base + 16 * kk * kW;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * kW));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// One dgrad output tile: rows [m0, min(m0 + kBM, hi)) of expert e's segment
// [lo, hi), output columns from n0.  kNRB = live 32-row blocks of this wave.
template <int kEpi, int kNRB>
__device__ __forceinline__ void ggb_tile(const GGParams& p, int e, int lo, int hi, int m0, int n0,
                                         uint16_t* s_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / kWN, wn = wave % kWN;
  const int r32 = lane & 31, h = lane >> 5;
  const int K = p.K;

  // --- A operand loads: block `wave` of the A tile ([128 rows][32 k], 16
  // rows per block), one descriptor over the tile's rows
  const i32x4 rs_a = buf_desc(p.a + static_cast<size_t>(m0) * p.lda, min(hi - m0, kBM) * p.lda * 2);
  const int r_a = wave * 16 + (lane >> 2);
  const int kcl_a = (lane & 3) ^ swz_f(r_a);
  const int vo_a = (min(r_a, hi - 1 - m0) * p.lda + kcl_a * 8) * 2;   // rows past the segment: dropped
  // --- B operand loads: blocks wave, wave + 8 of the [32 k][256 columns] tile
  const uint16_t* b_kbase = p.b + static_cast<size_t>(e) * p.b_estride;
  int vo_b[kBLoads];
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int krow = (wave + kWaves * j) * 2 + (lane >> 5);   // 512-byte k rows, 2 per block
    const int lc = (lane & 31) ^ ((krow & 3) << 2);
    vo_b[j] = (krow * p.ldb + n0 + 8 * lc) * 2;
  }

  const int nk = (K + kBK - 1) / kBK;
  // K tiles past the end (the ring's last kStages - 1 issues) load nothing:
  // an empty descriptor or an out-of-range offset reads zero without a
  // memory access, and the loads still count for the ring's fixed waits
  auto issue = [&](int kt) {
    const bool past = kt >= nk;
    const int t = min(kt, nk - 1);
    const int k0 = t * kBK;
    const int krows = past ? 0 : min(kBK, K - k0);
    uint16_t* st = s_lds + (kt % kStages) * kStageE;
    dma16(rs_a, st + wave * 512, (!past && k0 + kcl_a * 8 < K) ? vo_a : kOob, k0 * 2);
    const i32x4 rb = buf_desc(b_kbase + static_cast<size_t>(k0) * p.ldb, krows * p.ldb * 2);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
      dma16(rb, st + kATileE + (wave + kWaves * j) * 512, vo_b[j], 0);
  };

  // this wave's operand read offsets (B, transposed reads)
  int b_tr[kCB];
#pragma unroll
  for (int c = 0; c < kCB; ++c) b_tr[c] = tr_base<kBN>(wn * kCB * 32 + c * 32, lane);

  constexpr int kAccRB = kNRB > 0 ? kNRB : 1;
  f32x16 acc[kAccRB][kCB];
#pragma unroll
  for (int i = 0; i < kAccRB; ++i)
#pragma unroll
    for (int c = 0; c < kCB; ++c) acc[i][c] = f32x16{};

  auto compute = [&](int slot) {
    if constexpr (kNRB > 0) {
      const uint16_t* As = s_lds + slot * kStageE;
      const uint16_t* Bs = As + kATileE;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        bf16x8 bv[kCB];
#pragma unroll
        for (int c = 0; c < kCB; ++c) bv[c] = frag_tr<kBN>(Bs, b_tr[c], kk);
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb) {
          const bf16x8 av = frag_row(As, wm * kRB * 32 + rb * 32, kk, lane);
#pragma unroll
          for (int c = 0; c < kCB; ++c)
            acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[c], acc[rb][c], 0, 0, 0);
        }
      }
    }
  };

  // Ring as in the forward: tiles kt+1 .. kt+kStages-1 stay in flight while
  // tile kt is multiplied; the wait leaves the later tiles' loads in flight,
  // the bare barrier extends "tile kt landed" to all waves and frees the
  // slot about to be refilled.
  if (nk > 0) {
#pragma unroll
    for (int t = 0; t < kStages - 1; ++t) issue(t);
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      asm volatile("s_waitcnt vmcnt(" MOE_STR(MOE_BWD_VMCNT) ")\n\ts_barrier" ::: "memory");
      issue(kt + kStages - 1);
      compute(kt % kStages);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the ring (the empty tail loads)

  // ---------------- epilogue ------------------------------------------------
  // accumulator register r of lane l: A-operand row 8(r / 4) + 4(l / 32) +
  // r % 4, output column l % 32 (32 lanes write 32 consecutive columns).
  // (Taking the B block as the MFMAs' first operand instead, for 4
  // consecutive columns per lane and 8/16-byte accesses, measured slower
  // here: the SwiGLU backward's G, U reads then touch 32 rows per load.)
  if constexpr (kEpi == EPI_DGRAD2) {
    // fc2 dgrad + SwiGLU backward, staged through the free ring in four
    // passes of 32 rows (pass q: the waves with wm == q / 2 own their row
    // block q % 2): G and U come in as 16-byte vectors, each lane turns its
    // elements into dG, dU (in place) and A * scale (a third array), and the
    // results leave as 16-byte vectors.  Staged rows are padded to 264 bf16
    // so that the two half-waves (rows 4 apart) read disjoint banks.  Every
    // wave runs the same barriers.
    constexpr int kSR = 32, kSW = kBN + 8, kCh = kBN / 8;   // staged rows, padded width, chunks
    uint16_t* const GL = s_lds;
    uint16_t* const UL = s_lds + kSR * kSW;
    uint16_t* const AL = s_lds + 2 * kSR * kSW;
    static_assert(3 * kSR * kSW * 2 <= static_cast<int>(kBwdLds), "staging fits the ring");
    const int twoF = 2 * p.F;
    __syncthreads();                                     // every wave is done with the ring
#pragma unroll 1
    for (int q = 0; q < kBM / kSR; ++q) {
      const int r0 = m0 + q * kSR;
      // (1) G and U of rows r0 .. r0 + 31, columns n0 .. n0 + 255
#pragma unroll 1
      for (int i = tid; i < 2 * kSR * kCh; i += kGT) {
        const int arr = i / (kSR * kCh), rem = i % (kSR * kCh);
        const int row = rem / kCh, ch = rem % kCh;
        const int grow = r0 + row, f0 = n0 + ch * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (grow < hi && f0 < p.F)
          v = *reinterpret_cast<const u32x4*>(p.gu_in + static_cast<size_t>(grow) * twoF +
                                              (arr ? p.F : 0) + f0);
        *reinterpret_cast<u32x4*>((arr ? UL : GL) + row * kSW + ch * 8) = v;
      }
      __syncthreads();
      // (2) the owning waves: dG, dU in place, A * scale into AL
      if (wm == (q >> 1)) {
        const int rb = q & 1;
        if (rb < kNRB) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lrow = 8 * (r >> 2) + 4 * h + (r & 3);
            const int grow = r0 + lrow;
            const float sc = (p.scale && grow < hi) ? p.scale[grow] : 1.0f;
#pragma unroll
            for (int c = 0; c < kCB; ++c) {
              const int li = lrow * kSW + wn * kCB * 32 + c * 32 + r32;
              const float da = (rb == 0 ? acc[0][c][r] : acc[kAccRB - 1][c][r]) * sc;
              const float g = bf16_to_f32(GL[li]);
              const float u = bf16_to_f32(UL[li]);
              const float sg = sigmoid_fast(g);
              const float sl = g * sg;
              const u32x2 o = pack4_bf16(da * u * sg * (1.0f + g * (1.0f - sg)), da * sl,
                                         sc * sl * u, 0.0f);
              GL[li] = static_cast<uint16_t>(o[0]);
              UL[li] = static_cast<uint16_t>(o[0] >> 16);
              AL[li] = static_cast<uint16_t>(o[1]);
            }
            // one row at a time: keeps the staged reads from piling up in registers
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
      // (3) dG, dU to dH[row][f], dH[row][F + f]; A * scale to out2[row][f]
#pragma unroll 1
      for (int i = tid; i < 3 * kSR * kCh; i += kGT) {
        const int arr = i / (kSR * kCh), rem = i % (kSR * kCh);
        const int row = rem / kCh, ch = rem % kCh;
        const int grow = r0 + row, f0 = n0 + ch * 8;
        if (grow < hi && f0 < p.F) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(s_lds + arr * kSR * kSW + row * kSW + ch * 8);
          if (arr < 2)
            *reinterpret_cast<u32x4*>(p.out + static_cast<size_t>(grow) * twoF + (arr ? p.F : 0) + f0) = v;
          else
            *reinterpret_cast<u32x4*>(p.out2 + static_cast<size_t>(grow) * p.F + f0) = v;
        }
      }
      __syncthreads();
    }
  } else {                           // EPI_DGRAD1: dX rows, staged as 16-byte vectors
    constexpr int kSW = kBN + 8, kCh = kBN / 8;          // padded staged row (bf16), chunks
    static_assert(kBM * kSW * 2 <= static_cast<int>(kBwdLds), "staging fits the ring");
    __syncthreads();                                     // every wave is done with the ring
    if constexpr (kNRB > 0) {
#pragma unroll
      for (int rb = 0; rb < kNRB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lrow = wm * kRB * 32 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
          for (int c = 0; c < kCB; ++c)
            s_lds[lrow * kSW + wn * kCB * 32 + c * 32 + r32] =
                static_cast<uint16_t>(pack4_bf16(acc[rb][c][r], 0.f, 0.f, 0.f)[0]);
        }
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int i = tid; i < kBM * kCh; i += kGT) {
      const int row = i / kCh, ch = i % kCh;
      const int grow = m0 + row, n = n0 + ch * 8;
      if (grow < hi && n < p.d)
        *reinterpret_cast<u32x4*>(p.out + static_cast<size_t>(grow) * p.d + n) =
            *reinterpret_cast<const u32x4*>(s_lds + row * kSW + ch * 8);
    }
  }
}

template <int kEpi>
__global__ __launch_bounds__(kGT, 2) void ggb_kernel(GGParams p) {
  extern __shared__ __align__(16) uint16_t s_lds[];   // kStages x (A tile + B tile)
  __shared__ int s_cum[1025];
  __shared__ int s_tmp[kWaves];
  if (p.zero && blockIdx.x == 0 && threadIdx.x < 2) p.zero[threadIdx.x] = 0;
  tile_prefix<kGT>(p.offsets, p.E, kBM, p.ntn, s_cum, s_tmp);
  const int total = s_cum[p.E];
  if (static_cast<int>(blockIdx.x) >= total) return;
  const TileIdx ti = tile_decode(p.offsets, p.E, kBM, p.ntn, xcd_remap(blockIdx.x, total), s_cum);
  const int m0 = ti.m0;
  const int rows = ti.mend - m0 - (static_cast<int>(threadIdx.x >> 6) / kWN) * kRB * 32;
  const int nrb = rows <= 0 ? 0 : min(kRB, (rows + 31) >> 5);
  switch (nrb) {
    case 0: ggb_tile<kEpi, 0>(p, ti.e, ti.lo, ti.mend, m0, ti.nt * kBN, s_lds); break;
    case 1: ggb_tile<kEpi, 1>(p, ti.e, ti.lo, ti.mend, m0, ti.nt * kBN, s_lds); break;
    default: ggb_tile<kEpi, 2>(p, ti.e, ti.lo, ti.mend, m0, ti.nt * kBN, s_lds); break;
  }
}

// ---------------------------------------------------------------------------
// Persistent weight-gradient engine: dW[e] (+)= A_e^T B_e over expert e's
// token rows (K = the segment), both operands K-strided ([k][columns]).
// 256 x 256 output tiles, 16 wavefronts (4 x 4) of 64 x 64 (2 x 2
// accumulators), 64-wide K tiles in a 2-slot ring (A 32 KB + B 32 KB per
// slot), one workgroup per CU.  The next tile's first K tile is loaded while
// the current tile's last one is multiplied and while its epilogue stores
// the fp32 result straight from the accumulators (32 consecutive columns per
// row per store).  An empty expert runs one K tile of zeros, so its dW is
// written as zeros (or left as it is when accumulating).
//
// Schedule.  A tile's cost grows with its expert's row count, and routing
// makes those counts very unequal (one expert can hold a fifth of the rows,
// so its tiles cost most of a workgroup's fair share each).  Every
// workgroup ranks the experts by decreasing row count (ties by index) and
// lists the tiles in that order, each expert's tiles together (row tiles
// inner).  Workgroup b takes tiles b and b + grid, then fetches the next
// from one counter as it starts each tile: the most expensive tiles go
// first and the cheap ones fill the tail (longest-first list scheduling).
// When the caller gives scratch space, the tiles of the heaviest experts
// (more K steps than a workgroup's fair share of the launch) are split in
// two halves along K: the first half writes dW as usual, the second writes
// its partial tile to the scratch, and a second launch (ggw_fixup_kernel)
// adds it, so every element is still formed in a fixed order.  The
// heaviest expert's tiles would otherwise end the launch on their own
// when an expert has few output tiles.
constexpr int kPM = 256, kPN = 256, kPK = 64, kPWN = 4, kPRB = 2, kPCB = 2, kPWaves = 16;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPATileE = kPM * kPK, kPBTileE = kPN * kPK, kPSlotE = kPATileE + kPBTileE;
constexpr size_t kPRing = 2 * kPSlotE * sizeof(uint16_t);   // 128 KB
constexpr int kPLoads = kPATileE / 512 / kPWaves;          // 1 KB blocks per wave per operand (2)
constexpr int kPEpiSteps = 6;        // a tile's epilogue (256 KB of fp32 stores) in K steps
constexpr int kPMaxSplit = 256;      // split tiles per launch at most
constexpr size_t kPSplitMeta = 4096; // scratch header: count, then (e, mt, nt) per split tile
// LDS past the ring: expert order (1024 ints) and the fetch slot
constexpr size_t kPLds = kPRing + (1024 + 4) * sizeof(int);

// a descriptor the compiler cannot prove wave-uniform, moved to SGPRs
__device__ __forceinline__ i32x4 uniform4(i32x4 v) {
  return i32x4{__builtin_amdgcn_readfirstlane(v[0]), __builtin_amdgcn_readfirstlane(v[1]),
               __builtin_amdgcn_readfirstlane(v[2]), __builtin_amdgcn_readfirstlane(v[3])};
}

struct WgradParams {
  int E;
  const int32_t* offsets;    // [E+1]
  const uint16_t* a;         // [N, lda]: rows are k, columns the output rows m
  int lda;
  const uint16_t* b;         // [N, ldb]: columns the output columns n
  int ldb;
  float* outf;               // dW of expert 0, [out_m, out_n] fp32
  size_t outf_estride;
  int out_m, out_n;
  int mts, nts;              // 256-tiles per expert along m and n
  int accumulate;
  int* counter;              // tile counter, zero at launch
  int* split_meta;           // scratch header (NULL: no split) ...
  float* split_tiles;        // ... and split_cap partial 256 x 256 tiles after it
  int split_cap;
};

__device__ __forceinline__ int wgrad_nk(int K) { return K > 0 ? (K + kPK - 1) / kPK : 1; }

__global__ __launch_bounds__(kPThreads, 1) void ggw_persistent_kernel(WgradParams p) {
  extern __shared__ __align__(16) uint16_t s_lds[];
  int* s_order = reinterpret_cast<int*>(s_lds + kPRing / 2);   // rank -> expert (kept)
  int* s_fetch = s_order + 1024;
  int* s_K = reinterpret_cast<int*>(s_lds);   // [E] row counts, in the ring before its first load
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kPWN, wn = wave % kPWN;
  const int r32 = lane & 31, h = lane >> 5;
  const int E = p.E;
  const int per_e = p.mts * p.nts;
  const int total = per_e * E;

  // ---- expert order and split set (identical in every workgroup) --------
  for (int e = tid; e < E; e += kPThreads) s_K[e] = p.offsets[e + 1] - p.offsets[e];
  __syncthreads();
  for (int e = tid; e < E; e += kPThreads) {
    const int ke = s_K[e];
    int rank = 0;
    for (int f = 0; f < E; ++f) {
      const int kf = s_K[f];
      rank += (kf > ke || (kf == ke && f < e)) ? 1 : 0;
    }
    s_order[rank] = e;
  }
  __syncthreads();
  // split the experts (a prefix of the ranking) whose tiles hold more K
  // steps than the launch's cost per workgroup, as far as the scratch allows
  if (wave == 0) {
    float c = 0.0f;
    for (int e = lane; e < E; e += 64) c += static_cast<float>(wgrad_nk(s_K[e]) + kPEpiSteps);
    c = wave_sum(c) * static_cast<float>(per_e);
    const float share = c / static_cast<float>(gridDim.x);
    if (lane == 0) {
      int rs = 0;
      if (p.split_meta) {
        while (rs < E && (rs + 1) * per_e <= p.split_cap) {
          const int nk = wgrad_nk(s_K[s_order[rs]]);
          if (nk < 2 || static_cast<float>(nk) <= share) break;
          ++rs;
        }
      }
      *s_fetch = rs;
    }
  }
  __syncthreads();
  const int rs = *s_fetch;                       // split experts: ranks [0, rs)
  const int nsplit = rs * per_e;                 // split tiles, two halves each
  const int total_list = 2 * nsplit + (E - rs) * per_e;
  if (p.split_meta && blockIdx.x == 0) {         // the list of split tiles for the fixup
    for (int o = tid; o < nsplit; o += kPThreads) {
      const int r = o / per_e, local = o - r * per_e;
      const int nt = local / p.mts;
      p.split_meta[1 + 3 * o] = s_order[r];
      p.split_meta[2 + 3 * o] = local - nt * p.mts;
      p.split_meta[3 + 3 * o] = nt;
    }
    if (tid == 0) p.split_meta[0] = nsplit;
  }
  __syncthreads();              // s_fetch is reused below; s_K (in the ring) is read above
  if (static_cast<int>(blockIdx.x) >= total_list) return;   // uniform over the workgroup

  struct Tile {
    int e, lo, kbeg, kend, nk, m0, n0, part, ord;   // part -1: whole K; 0, 1: halves
  };
  auto setup = [&](int gl) {    // gl: index in the tile list
    Tile t;
    int r, local;
    if (gl < 2 * nsplit) {      // split tiles first: (tile, half) pairs
      t.ord = gl >> 1;
      t.part = gl & 1;
      r = t.ord / per_e;
      local = t.ord - r * per_e;
    } else {
      const int g2 = gl - 2 * nsplit;
      r = rs + g2 / per_e;
      local = g2 - (r - rs) * per_e;
      t.part = -1;
      t.ord = 0;
    }
    t.e = __builtin_amdgcn_readfirstlane(s_order[r]);
    const int nt = local / p.mts, mt = local - nt * p.mts;
    t.lo = __builtin_amdgcn_readfirstlane(p.offsets[t.e]);
    const int K = __builtin_amdgcn_readfirstlane(p.offsets[t.e + 1]) - t.lo;
    const int half = ((wgrad_nk(K) + 1) / 2) * kPK;
    t.kbeg = t.part == 1 ? half : 0;
    t.kend = t.part == 0 ? half : K;
    t.nk = wgrad_nk(t.kend - t.kbeg);
    t.m0 = mt * kPM;
    t.n0 = nt * kPN;
    return t;
  };
  // the wave's blocks: k rows 2 bb, 2 bb + 1 of a [64 k][256 columns] tile;
  // lane l fills 16-byte position l % 32 of k row 2 bb + l / 32 with chunk
  // (l % 32) ^ 4 (k % 4), the layout the transposed reads expect
  int krow[kPLoads], lcol[kPLoads];
#pragma unroll
  for (int j = 0; j < kPLoads; ++j) {
    const int bb = wave + kPWaves * j;
    krow[j] = 2 * bb + (lane >> 5);
    lcol[j] = 8 * ((lane & 31) ^ ((krow[j] & 3) << 2));
  }
  // K tile kt of tile t into ring slot `slot`; rows past the segment (and
  // every row of an empty expert) read zero through the descriptors' size
  auto issue = [&](const Tile& t, int kt, int slot) {
    const int k0 = t.kbeg + kt * kPK;
    const int krows = max(0, min(kPK, t.kend - k0));
    uint16_t* da = s_lds + slot * kPSlotE;
    uint16_t* db = da + kPATileE;
    const size_t r0 = static_cast<size_t>(t.lo) + (krows > 0 ? k0 : 0);   // (t.lo: in bounds)
    const i32x4 ra = uniform4(buf_desc(p.a + r0 * p.lda, krows * p.lda * 2));
    const i32x4 rb = uniform4(buf_desc(p.b + r0 * p.ldb, krows * p.ldb * 2));
#pragma unroll
    for (int j = 0; j < kPLoads; ++j)
      dma16(ra, da + (wave + kPWaves * j) * 512, (krow[j] * p.lda + t.m0 + lcol[j]) * 2, 0);
#pragma unroll
    for (int j = 0; j < kPLoads; ++j)
      dma16(rb, db + (wave + kPWaves * j) * 512, (krow[j] * p.ldb + t.n0 + lcol[j]) * 2, 0);
  };

  int a_tr[kPRB], b_tr[kPCB];
#pragma unroll
  for (int i = 0; i < kPRB; ++i) a_tr[i] = tr_base<kPM>(wm * kPRB * 32 + i * 32, lane);
#pragma unroll
  for (int c = 0; c < kPCB; ++c) b_tr[c] = tr_base<kPN>(wn * kPCB * 32 + c * 32, lane);

  f32x16 acc[kPRB][kPCB];
  auto compute = [&](int slot) {
    const uint16_t* As = s_lds + slot * kPSlotE;
    const uint16_t* Bs = As + kPATileE;
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 bv[kPCB];
#pragma unroll
      for (int c = 0; c < kPCB; ++c) bv[c] = frag_tr<kPN>(Bs, b_tr[c], kk);
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb) {
        const bf16x8 av = frag_tr<kPM>(As, a_tr[rb], kk);
#pragma unroll
        for (int c = 0; c < kPCB; ++c)
          acc[rb][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[c], acc[rb][c], 0, 0, 0);
      }
    }
  };
  // accumulator register r of lane l: output row 8 (r / 4) + 4 (l / 32) + r % 4
  // of the 32-row block, column l % 32
  auto epilogue = [&](const Tile& t) {
    if (t.part == 1) {          // second half: the partial tile, row-major 256 x 256
      float* dst = p.split_tiles + static_cast<size_t>(t.ord) * (kPM * kPN);
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * kPRB * 32 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
#pragma unroll
          for (int c = 0; c < kPCB; ++c) dst[row * kPN + wn * kPCB * 32 + c * 32 + r32] = acc[rb][c][r];
        }
      return;
    }
    float* dw = p.outf + static_cast<size_t>(t.e) * p.outf_estride;
    if (!p.accumulate) {
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = t.m0 + wm * kPRB * 32 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row >= p.out_m) continue;
          float* dst = dw + static_cast<size_t>(row) * p.out_n;
#pragma unroll
          for (int c = 0; c < kPCB; ++c) {
            const int col = t.n0 + wn * kPCB * 32 + c * 32 + r32;
            if (col < p.out_n) dst[col] = acc[rb][c][r];
          }
        }
      }
    } else {
      // dW += the tile: the old values of 8 elements at a time are loaded
      // branch-free (elements outside dW get an offset past the buffer: they
      // read zero and their stores are dropped) and waited for together; a
      // wait per element would also wait for every store before it
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc(dw, 0, p.out_m * p.out_n * 4, kRsrcWord3);
#pragma unroll
      for (int rb = 0; rb < kPRB; ++rb) {
#pragma unroll
        for (int r0 = 0; r0 < 16; r0 += 4) {
          int off[4][kPCB];
          float old[4][kPCB];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = t.m0 + wm * kPRB * 32 + rb * 32 + 8 * ((r0 + r) >> 2) + 4 * h + r;
#pragma unroll
            for (int c = 0; c < kPCB; ++c) {
              const int col = t.n0 + wn * kPCB * 32 + c * 32 + r32;
              off[r][c] = (row < p.out_m && col < p.out_n) ? (row * p.out_n + col) * 4 : kOob;
              old[r][c] = __builtin_bit_cast(
                  float, __builtin_amdgcn_raw_buffer_load_b32(rs, off[r][c], 0, 0));
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < kPCB; ++c) asm volatile("" ::"v"(old[r][c]));   // one wait
#pragma unroll
          for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int c = 0; c < kPCB; ++c)
              __builtin_amdgcn_raw_buffer_store_b32(
                  __builtin_bit_cast(uint32_t, old[r][c] + acc[rb][c][r0 + r]), rs, off[r][c], 0, 0);
        }
      }
    }
  };

  const int G = static_cast<int>(gridDim.x);
  Tile cur = setup(blockIdx.x);
  bool has_nxt = static_cast<int>(blockIdx.x) + G < total_list;
  Tile nxt = has_nxt ? setup(blockIdx.x + G) : cur;
  issue(cur, 0, 0);
  int g = 0;                    // global K step: ring slot g & 1
#pragma unroll 1
  for (;;) {
    int fetched = 0;
    if (has_nxt && tid == 0) fetched = atomicAdd(p.counter, 1);   // the tile after nxt
#pragma unroll
    for (int i = 0; i < kPRB; ++i)
#pragma unroll
      for (int c = 0; c < kPCB; ++c) acc[i][c] = f32x16{};
#pragma unroll 1
    for (int kt = 0; kt < cur.nk; ++kt, ++g) {
      // this wave's loads (and the last epilogue's stores) have landed; the
      // barrier makes K tile g visible and frees slot (g + 1) & 1
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + 1 < cur.nk) issue(cur, kt + 1, (g + 1) & 1);
      else if (has_nxt) issue(nxt, 0, (g + 1) & 1);
      compute(g & 1);
    }
    if (tid == 0) *s_fetch = 2 * G + fetched;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int L2 = *s_fetch;
    epilogue(cur);
    if (!has_nxt) break;
    cur = nxt;
    has_nxt = L2 < total_list;
    if (has_nxt) nxt = setup(L2);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// dW[e] tile (mt, nt) += the second half's partial, for each split tile
// listed by ggw_persistent_kernel: kFixBlocks workgroups per tile, 16 rows
// each, one 16-byte vector per thread and row group (out_n % 8 == 0, so a
// vector is wholly inside or outside the matrix).
constexpr int kFixBlocks = kPM / 16;
__global__ __launch_bounds__(256) void ggw_fixup_kernel(const int* __restrict__ meta,
                                                        const float* __restrict__ tiles,
                                                        float* __restrict__ dw, size_t estride,
                                                        int out_m, int out_n) {
  const int o = blockIdx.x / kFixBlocks, part = blockIdx.x % kFixBlocks;
  if (o >= meta[0]) return;
  const int e = meta[1 + 3 * o], m0 = meta[2 + 3 * o] * kPM, n0 = meta[3 + 3 * o] * kPN;
  const float4* src = reinterpret_cast<const float4*>(tiles + static_cast<size_t>(o) * (kPM * kPN));
  float* d = dw + static_cast<size_t>(e) * estride;
  constexpr int kVecRow = kPN / 4;                   // 64 vectors per tile row
  float4 v[4], w[4];
  int idx[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {                      // rows part * 16 + 4u + threadIdx.x / 64
    const int i = part * 16 * kVecRow + u * 256 + threadIdx.x;
    const int r = i / kVecRow, c = (i - r * kVecRow) * 4;
    idx[u] = (m0 + r < out_m && n0 + c < out_n) ? (m0 + r) * out_n + n0 + c : -1;
    v[u] = src[i];
    if (idx[u] >= 0) w[u] = *reinterpret_cast<const float4*>(d + idx[u]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (idx[u] >= 0) {
      float4 t = w[u];
      t.x += v[u].x; t.y += v[u].y; t.z += v[u].z; t.w += v[u].w;
      *reinterpret_cast<float4*>(d + idx[u]) = t;
    }
}

static unsigned wgrad_grid(int64_t tiles) {   // one workgroup per CU, at most one per tile
  return static_cast<unsigned>(std::max<int64_t>(1, std::min<int64_t>(device_cu_count(), tiles)));
}

// dW[e] (out_m x out_n) (+)= A[seg e]^T B[seg e] for every expert e.
// (counter: one int, zero when the launch starts; split: scratch of
// split_bytes for the K-split of the heaviest experts' tiles, or NULL)
static hipError_t launch_wgrad(hipStream_t stream, int32_t E, const int32_t* offsets,
                               const uint16_t* a, int lda, const uint16_t* b, int ldb, float* dw,
                               int out_m, int out_n, int accumulate, int* counter, void* split,
                               size_t split_bytes) {
  WgradParams p{};
  const size_t tile_bytes = static_cast<size_t>(kPM) * kPN * sizeof(float);
  const int cap = split && split_bytes > kPSplitMeta
                      ? static_cast<int>(std::min<size_t>(kPMaxSplit,
                                                          (split_bytes - kPSplitMeta) / tile_bytes))
                      : 0;
  if (cap > 0) {
    p.split_meta = static_cast<int*>(split);
    p.split_tiles = reinterpret_cast<float*>(static_cast<uint8_t*>(split) + kPSplitMeta);
    p.split_cap = cap;
  }
  p.E = E; p.offsets = offsets;
  p.a = a; p.lda = lda; p.b = b; p.ldb = ldb;
  p.outf = dw; p.outf_estride = static_cast<size_t>(out_m) * out_n;
  p.out_m = out_m; p.out_n = out_n;
  p.mts = (out_m + kPM - 1) / kPM;
  p.nts = (out_n + kPN - 1) / kPN;
  p.accumulate = accumulate;
  p.counter = counter;
  hipError_t err = allow_lds(ggw_persistent_kernel, kPLds);
  if (err == hipSuccess)
    err = launch(ggw_persistent_kernel, dim3(wgrad_grid(static_cast<int64_t>(p.mts) * p.nts * E)),
                 dim3(kPThreads), kPLds, stream, p);
  if (err == hipSuccess && cap > 0)
    err = launch(ggw_fixup_kernel, dim3(static_cast<unsigned>(cap * kFixBlocks)), dim3(256), 0, stream,
                 (const int*)p.split_meta, (const float*)p.split_tiles, dw, p.outf_estride, out_m,
                 out_n);
  return err;
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
  // with no rows (N = 0) the row buffers may be empty (NULL); dW is still written
  if (!w1 || !w2 || !expert_offsets || !dw1 || !dw2 || (N > 0 && (!dy_perm || !x_perm || !dx_perm)))
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
  // the two wgrad launches' tile counters sit in the workspace's slack; fc1
  // dgrad's first workgroup zeroes them (a kernel when there are no rows)
  int* counters = reinterpret_cast<int*>(
      wsb + off + (recompute ? round_up256(static_cast<size_t>(N) * 2 * F * 2) : 0));
  if (err == hipSuccess && N == 0) err = launch_zero_counters(stream, counters, 2);
  const size_t lds = kBwdLds;
  if (err == hipSuccess) err = allow_lds(ggb_kernel<EPI_DGRAD2>, lds);
  if (err == hipSuccess) err = allow_lds(ggb_kernel<EPI_DGRAD1>, lds);
  if (err == hipSuccess && N > 0) {
    // fc2 dgrad + SwiGLU backward: dH, A*scale
    GGParams p{};
    p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = expert_offsets;
    p.ntn = (int)((F + kBN - 1) / kBN);
    p.a = static_cast<const uint16_t*>(dy_perm); p.lda = (int)d;
    p.b = static_cast<const uint16_t*>(w2); p.ldb = (int)F; p.b_estride = static_cast<size_t>(d) * F;
    p.K = (int)d; p.scale = row_scale; p.gu_in = gu; p.out = dH; p.out2 = As;
    err = launch(ggb_kernel<EPI_DGRAD2>, dim3(tiles_bound(N, E, kBM) * p.ntn), dim3(kGT), lds,
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
    p.zero = counters;
    err = launch(ggb_kernel<EPI_DGRAD1>, dim3(tiles_bound(N, E, kBM) * p.ntn), dim3(kGT), lds,
                 stream, p);
  }
  if (err == hipSuccess)      // fc1 wgrad: dW1[e] (2F x d) = dH^T X
    err = launch_wgrad(stream, E, expert_offsets, dH, (int)(2 * F),
                       static_cast<const uint16_t*>(x_perm), (int)d, dw1, (int)(2 * F), (int)d,
                       accumulate, counters + 1, nullptr, 0);
  if (err == hipSuccess)      // fc2 wgrad: dW2[e] (d x F) = dY^T (A*scale); dH is free now
    err = launch_wgrad(stream, E, expert_offsets, static_cast<const uint16_t*>(dy_perm), (int)d,
                       As, (int)F, dw2, (int)d, (int)F, accumulate, counters, dH,
                       static_cast<size_t>(N) * 2 * F * 2);
  return hip_status(err);
}
