// Grouped SwiGLU expert FFN, forward: fc1 + SwiGLU, then fc2 + row scale.
//
// Passages: "Megatron-Bridge 深度剖析", section "计算融合 / Grouped GEMM" (all
// experts' GEMMs in one launch over segments of different length, expert
// weights stored back to back), section "权重映射策略" (GatedMLPMapping:
// linear_fc1 = [gate_proj; up_proj], (2*ffn, hidden)) and "Motivation"
// (SwiGLU experts with gate_proj, up_proj, down_proj).
//
// bf16 kernel (gfx950), one tile shape per use (compile-time FwdCfg):
//   * expert GEMMs: one workgroup of 16 wavefronts (4 x 4) per CU = one
//     output tile of 256 token rows x 256 weight rows (fc1: 128 gate rows +
//     the 128 matching up rows; fc2: 256 output columns); each wave computes
//     64 x 64 as 4 x 4 blocks of v_mfma_f32_16x16x32_bf16 (the router
//     logits tile keeps 32 x 32 x 16 blocks); K tiles are
//     64 wide, so every staged row segment is one whole 128-byte cache line
//     (a 32-wide K tile fetches half lines, which measured 1.5x slower from
//     L2 into LDS), in a 2-deep ring (128 KB);
//   * router logits (few output columns, many K slabs): two workgroups of
//     8 wavefronts (2 x 4) per CU, tiles of 128 x 256, a 3-deep ring of
//     32-wide K tiles (72 KB each), so that the small GEMM still fills the
//     chip;
//   * operand tiles go global -> LDS directly (buffer_load_dwordx4 ... lds):
//     no staging registers; each 1 KB block is 16 rows x 64 bytes (32-wide
//     K) or 8 rows x 128 bytes (64-wide K);
//   * the LDS layout is [row][16-byte chunks] with the chunk index XOR a
//     function of the row (f = (r1 ^ r3) | r2 << 1 for 4 chunks, (r mod 8)
//     ^ r3 for 8 chunks; r_i = bit i of the row): lane l of a block fetches
//     the chunk that lands at position l, and the MFMA operand reads (16 or
//     32 consecutive rows, one chunk) and the block writes are free of bank
//     conflicts with 32 or 64 banks;
//   * addresses are a buffer descriptor, a loop-invariant per-lane offset
//     and a scalar K offset; a chunk past K gets an offset past the end of
//     the buffer, which reads as zero, so K tails need no branches;
//   * a wave whose 32-row blocks lie past the end of the expert's segment
//     skips their MFMAs, and so does a wave whose columns all lie past the
//     output (the last column tile's padding, whose weight rows are not
//     read);
//   * tiles are decoded on the device from expert_offsets and handed to
//     XCDs in contiguous ranges (the row tiles sharing a weight panel run
//     together on one XCD and share its L2);
//   * fc1's epilogue computes silu(G) * U in registers (gate and up of the
//     same f land in the same lane); fc2's multiplies by the row's routing
//     weight.
#include <algorithm>

#include "moe_gemm_common.h"

namespace moe {

// Tile configuration: WM x WN MFMA wavefronts, each owning RB x CB blocks of
// 32 x 32 outputs, out of W wavefronts that all load (W >= WM * WN; the
// others only load); LDS rings of BK-wide K tiles, S deep for the token rows
// (A) and SB >= S deep for the weights (B); WG workgroups per CU.
template <int WM, int WN, int RB, int CB, int S, int BK, int WG, int W = WM * WN, int SB = S>
struct FwdCfg {
  static constexpr int kWM = WM, kWN = WN, kRB = RB, kCB = CB, kStages = S, kBK = BK, kWgPerCu = WG;
  static constexpr int kStagesB = SB;
  static constexpr int kThreads = 64 * W;
  static constexpr int kWaves = W;
  static constexpr int kBM = WM * RB * 32;            // token rows per tile
  static constexpr int kBN = WN * CB * 32;            // weight rows per tile
  static constexpr int kChunks = BK / 8;              // 16-byte chunks per staged row
  static constexpr int kRowsPerBlk = 64 / kChunks;    // staged rows per 1 KB block
  static constexpr int kATileE = kBM * BK;            // bf16 per ring slot
  static constexpr int kBTileE = kBN * BK;
  static constexpr int kStageE = kATileE + kBTileE;
  static constexpr int kABlocks = kBM / kRowsPerBlk;   // 1 KB blocks per ring slot
  static constexpr int kBBlocks = kBN / kRowsPerBlk;
  static constexpr int kLoads = (kABlocks + kBBlocks) / W;   // per wave per K tile
  static constexpr int kALoads = kABlocks / W;                // the first kALoads are A
  static constexpr int kBLoads = kBBlocks / W;
  // Per K tile kt a wave issues A(kt + S - 1), then B(kt + SB - 1); the
  // prologue issues the earlier ones in the same interleaved order, so B(kt)
  // always precedes A(kt).  Loads a wave may leave in flight when K tile kt
  // must have landed (loads complete in issue order): everything issued
  // after A(kt), or after B(kt) when the rings are equally deep.
  static constexpr int kRingWait = SB > S ? kBLoads + kLoads * (S - 2) : kLoads * (S - 2);
  static constexpr size_t kLdsBytes =
      (static_cast<size_t>(S) * kATileE + static_cast<size_t>(SB) * kBTileE) * sizeof(uint16_t);
  static_assert(BK == 32 || BK == 64, "K tile");
  static_assert(S >= 2 && SB >= S, "ring depth");
  static_assert(kABlocks % W == 0 && kBBlocks % W == 0 && W >= WM * WN && W <= 16,
                "blocks per wave");
  static_assert(kLdsBytes <= 160 * 1024, "LDS");
  static_assert(CB % 2 == 0, "fc1 pairs gate and up column blocks");
  static_assert(kLdsBytes >= (1040 + 64) * sizeof(int), "tile-decode scratch fits the ring");
  static_assert(RB == 2 || RB == 4, "live-row dispatch");
};

// Expert GEMMs.  Measured on MI355X (fc1 + fc2, bf16) against 128 x 256
// tiles with two workgroups per CU and a 3-deep ring of 32-wide K tiles:
// 2 to 9% faster on the 128- and 32-expert shapes with 256 to 1024 rows per
// expert, equal on the 128-expert shape with ragged segments.  A deeper ring
// for the weights (160 KB) and software L2 prefetch of the weight rows were
// no faster.  (Overridable at build time for tuning sweeps.)
#ifndef MOE_FWD_WM
#define MOE_FWD_WM 4
#define MOE_FWD_WN 4
#define MOE_FWD_RB 2
#define MOE_FWD_CB 2
#define MOE_FWD_STAGES 2
#define MOE_FWD_BK 64
#define MOE_FWD_WG_PER_CU 1
#endif
#ifndef MOE_FWD_W
#define MOE_FWD_W (MOE_FWD_WM * MOE_FWD_WN)
#endif
#ifndef MOE_FWD_SB
#define MOE_FWD_SB MOE_FWD_STAGES
#endif
using GemmCfg = FwdCfg<MOE_FWD_WM, MOE_FWD_WN, MOE_FWD_RB, MOE_FWD_CB, MOE_FWD_STAGES, MOE_FWD_BK,
                       MOE_FWD_WG_PER_CU, MOE_FWD_W, MOE_FWD_SB>;
// Router logits: 128 token rows x 128 experts per tile (the expert count of
// the 128-expert models: no padded weight rows), 64-wide K, K split into
// slabs of at least eight K tiles (see router_ksplit) so that the small GEMM
// has about one workgroup per CU, and a 4-deep ring (one workgroup per CU).
using RouterCfg = FwdCfg<2, 2, 2, 2, 4, 64, 1>;

enum FwdEpi { FWD_FC1 = 0, FWD_FC2 = 1, FWD_LOGITS = 2 };

struct FwdParams {
  int E, F, d, K, ntn;
  const int32_t* offsets;                     // [E+1], or NULL: one group of rows1 rows
  int rows1;
  const uint16_t* a;                          // token rows [N, K], or [a_rows, K] when gathering
  int lda;
  const int32_t* gather;                      // [N]: source row of each row, or NULL (row r is a[r])
  int a_rows;                                 // rows of a when gathering
  const uint16_t* b;                          // weights, expert-major
  int ldb;
  size_t b_estride;
  int packed_b;                               // b is tile-packed (pack_b_kernel); nkt K tiles
  int nkt;
  const float* scale;                         // FC2: [N] row scale; LOGITS: [d] column bias (or NULL)
  uint16_t* out;                              // FC1: A [N, F]; FC2: Y [N, d]
  uint16_t* out2;                             // FC1: [G | U] [N, 2F] or NULL
  float* outf;                                // LOGITS: z [N, d] fp32 (d = output columns)
  int ksplit;                                 // K split into gridDim.y slabs (LOGITS)
  size_t outf_split;                          // LOGITS: elements between slabs
  const uint16_t* gate_w;                     // LOGITS: [K] shared-gate weights, or NULL
  float* gate_out;                            // LOGITS: [ksplit][rows1] x . gate_w per slab
  int32_t* zero_i32;                          // LOGITS: zero_n ints zeroed by workgroup 0, or NULL
  int zero_n;
};

// chunk permutation of staged row r (see the file comment)
template <int kChunks>
__device__ __forceinline__ int swz_row(int r) {
  return kChunks == 4 ? swz_f(r) : ((r & 7) ^ ((r >> 3) & 1));
}

// One output tile.  kNRB = live 32-row blocks of this wave (0..RB).
template <class C, int kEpi, int kNRB>
__device__ __forceinline__ void ggf_tile(const FwdParams& p, const TileIdx& ti, uint16_t* s_lds) {
  constexpr int kWN = C::kWN, kRB = C::kRB, kCB = C::kCB, kWaves = C::kWaves;
  constexpr int kBM = C::kBM, kBN = C::kBN, kBK = C::kBK, kChunks = C::kChunks;
  constexpr int kStages = C::kStages, kStagesB = C::kStagesB, kLoads = C::kLoads;
  constexpr int kALoads = C::kALoads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int r32 = lane & 31, h = lane >> 5;
  constexpr int nbn = kEpi == FWD_FC1 ? kBN / 2 : kBN;   // output columns per tile
  // accumulator layout (see the epilogue): row per lane for the bf16
  // outputs, column per lane for the fp32 logits
  constexpr bool kSwap = kEpi != FWD_LOGITS;
  const int m0 = ti.m0;
  const int n0 = ti.nt * nbn;
  const int K = p.K;

  // buffer descriptors: this tile's token rows (all of a when gathering),
  // this expert's weights
  const bool gath = p.gather != nullptr;
  const __amdgpu_buffer_rsrc_t rs_a = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(gath ? p.a : p.a + static_cast<size_t>(m0) * p.lda), 0,
      (gath ? p.a_rows : ti.mend - m0) * p.lda * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_b = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.b + static_cast<size_t>(ti.e) * p.b_estride), 0,
      static_cast<int>(p.b_estride * 2), kRsrcWord3);

  // Load j of this wave fills block wave + kWaves j of the slot: A blocks
  // first, then B blocks (which one is uniform per wave).  Lane l of a block
  // writes LDS position l, i.e. row kRowsPerBlk blk + l / kChunks, physical
  // chunk l % kChunks, so it fetches logical chunk (l % kChunks) ^ swz_row(row).
  const int lr = lane / kChunks, pc = lane % kChunks;
  const int last = ti.mend - 1 - m0;
  int vo[kLoads], kcl[kLoads], dsto[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool isa = j < kALoads;
    const int bb = isa ? wave + kWaves * j : wave + kWaves * (j - kALoads);
    const int r = bb * C::kRowsPerBlk + lr;
    const int kc = pc ^ swz_row<kChunks>(r);
    kcl[j] = kc;
    dsto[j] = bb * 512;
    if (isa) {
      // rows past the tile, and gathered rows outside [0, a_rows), read zero
      const int src = r > last ? -1 : gath ? p.gather[m0 + r] : r;
      vo[j] = src >= 0 && (!gath || src < p.a_rows) ? (src * p.lda + kc * 8) * 2 : kOob;
    } else if (p.packed_b) {
      // tile ti.nt of this expert's packed weights, row r; the K tile is
      // the scalar offset (one contiguous kBN x kBK block per K tile)
      vo[j] = ((ti.nt * p.nkt * kBN + r) * kBK + kc * 8) * 2;
    } else {
      int wr;
      if constexpr (kEpi == FWD_FC1) {        // B rows: gate half, then the matching up half
        int f = n0 + (r % (kBN / 2));
        f = f < p.F ? f : p.F - 1;
        wr = r < kBN / 2 ? f : p.F + f;
      } else {
        wr = n0 + r;
        wr = wr < p.d ? wr : p.d - 1;
      }
      vo[j] = (wr * p.ldb + kc * 8) * 2;
    }
  }
  // K tiles [kt_lo, kt_hi) of this workgroup (all of them unless K is split)
  const int nk_all = (K + kBK - 1) / kBK;
  const int kchunk = (nk_all + p.ksplit - 1) / p.ksplit;
  const int kt_lo = min(nk_all, static_cast<int>(blockIdx.y) * kchunk);
  const int kt_hi = min(nk_all, kt_lo + kchunk);

  // Router logits with a shared-expert gate: the first column tile of each
  // row block also forms x . gate_w over its K slab from the token rows
  // already staged for the MFMAs (two threads per row, four 16-byte chunks
  // each per K tile).  The slab's gate weights go to LDS behind the rings,
  // 1 KB per direct load, issued before the ring's own loads, so the ring's
  // first wait and barrier cover them.  (The top-k kernel sums the slabs.)
  constexpr bool kGateOk = kEpi == FWD_LOGITS && C::kThreads == 2 * kBM && kChunks == 8;
  const bool do_gate = kGateOk && p.gate_w != nullptr && ti.nt == 0;
  uint16_t* const s_gw = s_lds + C::kLdsBytes / 2;      // [kchunk * kBK] bf16
  float gsum = 0.0f;
  if constexpr (kGateOk) {
    if (do_gate) {
      const __amdgpu_buffer_rsrc_t rs_g = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(p.gate_w), 0, K * 2, kRsrcWord3);   // past K: zeros
      const int nblk = ((kt_hi - kt_lo) * kBK * 2 + 1023) / 1024;
      for (int b = wave; b < nblk; b += kWaves)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_g, (lds_void*)(s_gw + b * 512), 16,
                                                 kt_lo * kBK * 2 + b * 1024 + lane * 16, 0, 0, 0);
    }
  }

  // LDS: the A ring (kStages slots), then the B ring (kStagesB slots)
  uint16_t* const ring_b = s_lds + kStages * C::kATileE;
  // fetch the A (token rows) or B (weights) part of K tile kt (clamped to
  // the last one) into its ring slot
  auto issue_a = [&](int kt) {
    const int t = min(kt, kt_hi - 1);
    const int k0 = t * kBK;
    uint16_t* st = s_lds + ((kt - kt_lo) % kStages) * C::kATileE;
#pragma unroll
    for (int j = 0; j < kALoads; ++j) {
      const int v = (k0 + kcl[j] * 8 < K) ? vo[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_a, (lds_void*)(st + dsto[j]), 16, v, k0 * 2,
                                               0, 0);
    }
  };
  auto issue_b = [&](int kt) {
    const int t = min(kt, kt_hi - 1);
    const int k0 = t * kBK;
    uint16_t* st = ring_b + ((kt - kt_lo) % kStagesB) * C::kBTileE;
    const int sb = p.packed_b ? t * (kBN * kBK * 2) : k0 * 2;
#pragma unroll
    for (int j = kALoads; j < kLoads; ++j) {
      const int v = (k0 + kcl[j] * 8 < K) ? vo[j] : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_b, (lds_void*)(st + dsto[j]), 16, v, sb, 0, 0);
    }
  };

  // this wave's operand rows in the staged tiles
  int a_rd[kRB], b_rd[kCB];
#pragma unroll
  for (int i = 0; i < kRB; ++i) a_rd[i] = wm * kRB * 32 + i * 32 + r32;
#pragma unroll
  for (int c = 0; c < kCB; ++c) {
    if constexpr (kEpi == FWD_FC1) {          // gate blocks, then the matching up blocks
      const int cc = c % (kCB / 2);
      b_rd[c] = (c < kCB / 2 ? 0 : kBN / 2) + wn * (kCB / 2) * 32 + cc * 32 + r32;
    } else {
      b_rd[c] = wn * kCB * 32 + c * 32 + r32;
    }
  }
  // staged element offset of row r, 16-byte chunk kc
  auto swz = [](int r, int kc) { return r * kBK + ((kc ^ swz_row<kChunks>(r)) << 3); };

  constexpr int kAccRB = kNRB > 0 ? kNRB : 1;
  f32x16 acc[kAccRB][kCB];
#pragma unroll
  for (int i = 0; i < kAccRB; ++i)
#pragma unroll
    for (int c = 0; c < kCB; ++c) acc[i][c] = f32x16{};

  auto compute = [&](int kt) {
    if constexpr (kNRB > 0) {
      const uint16_t* As = s_lds + ((kt - kt_lo) % kStages) * C::kATileE;
      const uint16_t* Bs = ring_b + ((kt - kt_lo) % kStagesB) * C::kBTileE;
#pragma unroll
      for (int kk = 0; kk < kBK / 16; ++kk) {
        const int ck = 2 * kk + h;
        bf16x8 bv[kCB];
#pragma unroll
        for (int c = 0; c < kCB; ++c) bv[c] = *reinterpret_cast<const bf16x8*>(Bs + swz(b_rd[c], ck));
#pragma unroll
        for (int rb = 0; rb < kNRB; ++rb) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(As + swz(a_rd[rb], ck));
#pragma unroll
          for (int c = 0; c < kCB; ++c)
            acc[rb][c] = kSwap
                             ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[c], av, acc[rb][c], 0, 0, 0)
                             : __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[c], acc[rb][c], 0, 0, 0);
        }
      }
    }
  };

  // this thread's part of the gate dot product for K tile kt: row tid / 2,
  // chunks 4 (tid % 2) .. +3 of the staged A tile
  auto gate_step = [&](int kt) {
    if constexpr (kGateOk) {
      const uint16_t* As = s_lds + ((kt - kt_lo) % kStages) * C::kATileE;
      const int r = tid >> 1;
      const uint16_t* gw = s_gw + (kt - kt_lo) * kBK;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kc = 4 * (tid & 1) + q;
        const u32x4 a = *reinterpret_cast<const u32x4*>(As + swz(r, kc));
        const u32x4 w = *reinterpret_cast<const u32x4*>(gw + kc * 8);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (through scalars: a bit_cast of a vector element itself reads
          // element 0 whatever the index, with this compiler)
          const uint32_t ae = a[e], we = w[e];
          gsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, ae),
                                                 __builtin_bit_cast(bf16x2v, we), gsum, false);
        }
      }
    }
  };

  // Rings: A tiles kt+1 .. kt+kStages-1 and B tiles kt+1 .. kt+kStagesB-1
  // stay in flight while tile kt is multiplied.  The wait leaves the later
  // tiles' loads in flight (kRingWait), the barrier extends "tile kt landed"
  // to all waves and guarantees that the slots about to be refilled (tile
  // kt-1's) are no longer read.  The barrier is the bare s_barrier (LDS is
  // coherent inside the CU): a __syncthreads fence would wait for every load
  // in flight.
  if (kt_lo < kt_hi) {
#pragma unroll
    for (int v = 1 - kStagesB; v < 0; ++v) {      // the same order as the loop's issues
      if (v + kStages - 1 >= 0) issue_a(kt_lo + v + kStages - 1);
      issue_b(kt_lo + v + kStagesB - 1);
    }
#pragma unroll 1
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C::kRingWait) : "memory");
      issue_a(kt + kStages - 1);
      issue_b(kt + kStagesB - 1);
      compute(kt);
      if (do_gate) gate_step(kt);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // drain the clamped extra loads
  if constexpr (kGateOk) {
    if (do_gate) {
      // the row = its low half's sum + its high half's sum
      const float other = __shfl_xor(gsum, 1, kWave);
      const int r = tid >> 1;
      if ((tid & 1) == 0 && m0 + r < ti.mend)
        p.gate_out[blockIdx.y * static_cast<size_t>(p.rows1) + m0 + r] = gsum + other;
    }
  }

  // ---------------- epilogue ------------------------------------------------
  // fc1 / fc2: the MFMAs take the weight block as their first operand, so
  // accumulator register 4q + i of lane l holds token row l % 32 of the
  // block and output column 8q + 4(l / 32) + i: four consecutive columns per
  // lane, staged in LDS as one 8-byte (bf16) write.  Logits: register r of
  // lane l holds token row 8(r / 4) + 4(l / 32) + r % 4 and column l % 32
  // (32 lanes write 128 contiguous bytes of fp32).
  if constexpr (kEpi == FWD_LOGITS) {
    if constexpr (kNRB > 0) {
    float* dst = p.outf + blockIdx.y * p.outf_split;
    // This lane's columns' bias, loaded and waited for before the first
    // store, with no branch around the loads (a descriptor of 0 bytes when
    // there is no bias, or for slabs past the first; columns past d read
    // zero): a load still pending at a store's operand would be waited for
    // there with vmcnt(0), which also waits for every store before it (one
    // round trip per store).
    const bool has_bias = p.scale != nullptr && blockIdx.y == 0;
    const __amdgpu_buffer_rsrc_t rs_bias = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(p.scale), 0, has_bias ? p.d * 4 : 0, kRsrcWord3);
    float bias[kCB];
#pragma unroll
    for (int c = 0; c < kCB; ++c) {
      const int n = n0 + wn * kCB * 32 + c * 32 + r32;
      bias[c] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs_bias, n * 4, 0, 0));
    }
#pragma unroll
    for (int c = 0; c < kCB; ++c) asm volatile("" ::"v"(bias[c]));   // the one wait, here
#pragma unroll
    for (int rb = 0; rb < kNRB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * kRB * 32 + rb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row >= ti.mend) continue;
#pragma unroll
        for (int c = 0; c < kCB; ++c) {
          const int n = n0 + wn * kCB * 32 + c * 32 + r32;
          if (n < p.d) dst[static_cast<size_t>(row) * p.d + n] = acc[rb][c][r] + bias[c];
        }
      }
    }
    }
  } else {
    // fc1 (A = silu(G) U) and fc2 (Y, row-scaled): the bf16 tile goes through
    // LDS (the ring is idle now) and leaves as 16-byte lanes over whole rows,
    // 8 full 128-byte lines per store instruction; stored straight from the
    // MFMA layout, one instruction would touch 32 rows with 16 bytes each.
    constexpr int kCols = nbn;                    // output columns of the tile
    constexpr int kSRow = kCols * 2 + 16;         // staged row bytes; the pad spreads rows over banks
    constexpr int kPass = kBM * kSRow <= static_cast<int>(C::kLdsBytes) ? 1 : 2;
    constexpr int kPR = kBM / kPass;              // tile rows per pass
    static_assert(kPR * kSRow <= static_cast<int>(C::kLdsBytes) && kPR % (kRB * 32) == 0,
                  "staging fits the ring");
    constexpr int kChunksRow = kCols / 8;         // 16-byte chunks per staged row
    uint8_t* const stg = reinterpret_cast<uint8_t*>(s_lds);
    const int limit = kEpi == FWD_FC1 ? p.F : p.d;
    const int wrow0 = wm * kRB * 32;              // this wave's first row in the tile
    __syncthreads();                              // every wave is done with the ring
#pragma unroll
    for (int ps = 0; ps < kPass; ++ps) {
      if constexpr (kNRB > 0) {
        if (wrow0 / kPR == ps) {
#pragma unroll
          for (int rb = 0; rb < kNRB; ++rb) {
            const int lrow = wrow0 - ps * kPR + rb * 32 + r32;
            const int row = m0 + wrow0 + rb * 32 + r32;
            uint8_t* srow = stg + lrow * kSRow;
            if constexpr (kEpi == FWD_FC1) {
              const size_t rowz = static_cast<size_t>(row);
#pragma unroll
              for (int c = 0; c < kCB / 2; ++c) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int fl = wn * (kCB / 2) * 32 + c * 32 + 8 * q + 4 * h;   // in the tile
                  const f32x16& G = acc[rb][c];
                  const f32x16& U = acc[rb][c + kCB / 2];
                  float a4[4];
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const float g = G[4 * q + i];
                    a4[i] = g * sigmoid_fast(g) * U[4 * q + i];
                  }
                  *reinterpret_cast<u32x2*>(srow + fl * 2) = pack4_bf16(a4[0], a4[1], a4[2], a4[3]);
                  const int f = n0 + fl;
                  if (p.out2 && row < ti.mend && f < p.F) {
                    uint16_t* gu = p.out2 + rowz * 2 * p.F;
                    *reinterpret_cast<u32x2*>(gu + f) =
                        pack4_bf16(G[4 * q], G[4 * q + 1], G[4 * q + 2], G[4 * q + 3]);
                    *reinterpret_cast<u32x2*>(gu + p.F + f) =
                        pack4_bf16(U[4 * q], U[4 * q + 1], U[4 * q + 2], U[4 * q + 3]);
                  }
                }
              }
            } else {  // FWD_FC2
              const float sc = (p.scale && row < ti.mend) ? p.scale[row] : 1.0f;
#pragma unroll
              for (int c = 0; c < kCB; ++c) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const int nl = wn * kCB * 32 + c * 32 + 8 * q + 4 * h;
                  const f32x16& Y = acc[rb][c];
                  *reinterpret_cast<u32x2*>(srow + nl * 2) =
                      pack4_bf16(Y[4 * q] * sc, Y[4 * q + 1] * sc, Y[4 * q + 2] * sc,
                                 Y[4 * q + 3] * sc);
                }
              }
            }
          }
        }
      }
      __syncthreads();
      // rows past the segment and columns past F / d are not stored (F and d
      // are multiples of 8: a 16-byte chunk is wholly in or out)
#pragma unroll
      for (int i = tid; i < kPR * kChunksRow; i += C::kThreads) {
        const int lr = i / kChunksRow, ch = i - lr * kChunksRow;
        const int row = m0 + ps * kPR + lr;
        const int col = n0 + ch * 8;
        if (row < ti.mend && col < limit)
          *reinterpret_cast<u32x4*>(p.out + static_cast<size_t>(row) * limit + col) =
              *reinterpret_cast<const u32x4*>(stg + lr * kSRow + ch * 16);
      }
      if (ps + 1 < kPass) __syncthreads();
    }
  }
}

template <class C, int kEpi>
__global__ __launch_bounds__(C::kThreads, C::kWgPerCu) void ggf_kernel(FwdParams p) {
  // kStages x (A tile + B tile); the tile-decode scratch lives in the same
  // memory before the ring starts
  extern __shared__ __align__(16) uint16_t s_lds[];
  int* s_cum = reinterpret_cast<int*>(s_lds);
  int* s_tmp = s_cum + 1040;
  if (p.zero_i32 && blockIdx.x == 0 && blockIdx.y == 0)   // (the next kernel's counters)
    for (int i = threadIdx.x; i < p.zero_n; i += C::kThreads) p.zero_i32[i] = 0;
  TileIdx ti;
  if (p.offsets) {
    tile_prefix<C::kThreads>(p.offsets, p.E, C::kBM, p.ntn, s_cum, s_tmp);
    const int total = s_cum[p.E];
    if (static_cast<int>(blockIdx.x) >= total) return;
    ti = tile_decode(p.offsets, p.E, C::kBM, p.ntn, xcd_remap(blockIdx.x, total), s_cum);
    __syncthreads();   // every wave has decoded its tile before the ring overwrites s_cum
  } else {
    const int total = ((p.rows1 + C::kBM - 1) / C::kBM) * p.ntn;
    if (static_cast<int>(blockIdx.x) >= total) return;
    ti = tile_decode_one(p.rows1, C::kBM, p.ntn, xcd_remap(blockIdx.x, total));
  }
  // live 32-row blocks of this wave's rows
  const int rows = ti.mend - ti.m0 -
                   (static_cast<int>(threadIdx.x >> 6) / C::kWN) * C::kRB * 32;
  const int nrb = rows <= 0 ? 0 : min(C::kRB, (rows + 31) >> 5);
  if constexpr (C::kRB == 2) {
    switch (nrb) {
      case 0: ggf_tile<C, kEpi, 0>(p, ti, s_lds); break;
      case 1: ggf_tile<C, kEpi, 1>(p, ti, s_lds); break;
      default: ggf_tile<C, kEpi, 2>(p, ti, s_lds); break;
    }
  } else {
    switch (nrb) {
      case 0: ggf_tile<C, kEpi, 0>(p, ti, s_lds); break;
      case 1: ggf_tile<C, kEpi, 1>(p, ti, s_lds); break;
      case 2: ggf_tile<C, kEpi, 2>(p, ti, s_lds); break;
      case 3: ggf_tile<C, kEpi, 3>(p, ti, s_lds); break;
      default: ggf_tile<C, kEpi, 4>(p, ti, s_lds); break;
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent expert GEMMs (fc1, fc2; bf16): one workgroup per CU walks its
// share of the tiles with one 2-slot ring that runs across tile boundaries.
// The next tile's first K tile is loaded while the current tile's last one
// is multiplied, its decode and row gathers are done while the current tile
// runs, and the current tile's epilogue overlaps those loads; the per-tile
// prologue and the workgroup turnaround of the one-tile-per-workgroup launch
// disappear.  Tiles, their staging and their epilogue math are those of
// ggf_tile, so the results are bit-identical to it.
//
// Schedule: workgroup b sits on XCD b % 8 (round-robin dispatch); each XCD
// owns a contiguous range of logical tiles (the row tiles that share a
// weight panel are neighbours) and its workgroups take them round robin.
// ---------------------------------------------------------------------------
constexpr int kScanInts = 1040 + 64;    // tile_prefix scratch (E <= 1024)

// One tile's addressing: its decode, buffer descriptors and per-lane offsets.
template <int kLoads>
struct PersistTile {
  TileIdx ti;
  __amdgpu_buffer_rsrc_t ra, rb;
  int vo[kLoads];
};

template <class C, int kEpi>
__device__ __forceinline__ void ggfp_body(const FwdParams& p) {
  static_assert(kEpi == FWD_FC1 || kEpi == FWD_FC2, "expert GEMMs only");
  static_assert(C::kStages == 2 && C::kStagesB == 2, "2-slot rings");
  constexpr int kWN = C::kWN, kRB = C::kRB, kCB = C::kCB, kWaves = C::kWaves;
  constexpr int kBM = C::kBM, kBN = C::kBN, kBK = C::kBK, kChunks = C::kChunks;
  constexpr int kLoads = C::kLoads, kALoads = C::kALoads;
  constexpr int nbn = kEpi == FWD_FC1 ? kBN / 2 : kBN;   // output columns per tile
  extern __shared__ __align__(16) uint16_t s_lds[];
  int* s_cum = reinterpret_cast<int*>(s_lds + C::kLdsBytes / 2);   // past the rings
  int* s_tmp = s_cum + 1040;
  uint16_t* const ring_a = s_lds;
  uint16_t* const ring_b = s_lds + 2 * C::kATileE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Waves are dealt to the SIMDs round robin (SIMD = wave mod 4).  With 4 x 4
  // waves, wave (wm, wn) sits on SIMD (wm + wn) mod 4, so the dead row blocks
  // of a short tile (one wm) and the dead column blocks of the last column
  // tile (the high wn) are spread over all four SIMDs.
  const int wm = C::kWM == 4 && kWN == 4 ? wave >> 2 : wave / kWN;
  const int wn = C::kWM == 4 && kWN == 4 ? ((wave & 3) - wm) & 3 : wave % kWN;
  const int r16 = lane & 15, q4 = lane >> 4;
  const int K = p.K;
  const int nk = (K + kBK - 1) / kBK;

  tile_prefix<C::kThreads>(p.offsets, p.E, kBM, p.ntn, s_cum, s_tmp);
  const int total = s_cum[p.E];
  const int g8 = static_cast<int>(gridDim.x >> 3);
  const int xcd = static_cast<int>(blockIdx.x & 7), pos = static_cast<int>(blockIdx.x >> 3);
  const int q = total >> 3, rq = total & 7;
  const int xbeg = xcd * q + min(xcd, rq), xcnt = q + (xcd < rq ? 1 : 0);
  const int ntiles = xcnt > pos ? (xcnt - pos + g8 - 1) / g8 : 0;
  if (ntiles == 0) return;                       // uniform over the workgroup

  // tile-invariant: the staged row, chunk and LDS block of each load
  const int lr = lane / kChunks, pc = lane % kChunks;
  int kcl[kLoads], dsto[kLoads], rowl[kLoads];
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool isa = j < kALoads;
    const int bb = isa ? wave + kWaves * j : wave + kWaves * (j - kALoads);
    const int r = bb * C::kRowsPerBlk + lr;
    rowl[j] = r;
    kcl[j] = pc ^ swz_row<kChunks>(r);
    dsto[j] = bb * 512;
  }
  const bool gath = p.gather != nullptr;

  // per-tile addressing: decode, descriptors, per-lane source offsets
  using TileState = PersistTile<kLoads>;
  auto setup = [&](int j, TileState& st) {
    st.ti = tile_decode(p.offsets, p.E, kBM, p.ntn, xbeg + pos + j * g8, s_cum);
    const TileIdx& ti = st.ti;
    const int m0 = ti.m0, n0 = ti.nt * nbn, last = ti.mend - 1 - m0;
    st.ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(gath ? p.a : p.a + static_cast<size_t>(m0) * p.lda), 0,
        (gath ? p.a_rows : ti.mend - m0) * p.lda * 2, kRsrcWord3);
    st.rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.b + static_cast<size_t>(ti.e) * p.b_estride), 0,
        static_cast<int>(p.b_estride * 2), kRsrcWord3);
#pragma unroll
    for (int j2 = 0; j2 < kLoads; ++j2) {
      const int r = rowl[j2], kc = kcl[j2];
      if (j2 < kALoads) {
        const int src = r > last ? -1 : gath ? p.gather[m0 + r] : r;
        st.vo[j2] = src >= 0 && (!gath || src < p.a_rows) ? (src * p.lda + kc * 8) * 2 : kOob;
      } else {
        // weight rows past the output (the last column tile's padding) are
        // not read: an offset past the buffer reads zero, with no traffic
        const int f = kEpi == FWD_FC1 ? n0 + (r % (kBN / 2)) : n0 + r;
        const bool dead = f >= (kEpi == FWD_FC1 ? p.F : p.d);
        const int wr = kEpi == FWD_FC1 && r >= kBN / 2 ? p.F + f : f;
        st.vo[j2] = dead ? kOob
                         : p.packed_b ? ((ti.nt * p.nkt * kBN + r) * kBK + kc * 8) * 2
                                      : (wr * p.ldb + kc * 8) * 2;
      }
    }
  };
  // K tile kt of tile st into ring slot `slot`
  auto issue = [&](const TileState& st, int kt, int slot) {
    const int k0 = kt * kBK;
    const int sb = p.packed_b ? kt * (kBN * kBK * 2) : k0 * 2;
    uint16_t* da = ring_a + slot * C::kATileE;
    uint16_t* db = ring_b + slot * C::kBTileE;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int v = (k0 + kcl[j] * 8 < K) ? st.vo[j] : kOob;
      if (j < kALoads)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(st.ra, (lds_void*)(da + dsto[j]), 16, v, k0 * 2,
                                                 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(st.rb, (lds_void*)(db + dsto[j]), 16, v, sb, 0, 0);
    }
  };

  // The MFMAs are v_mfma_f32_16x16x32_bf16: a wave's 32-row / 32-column
  // blocks (the tiling, the live-block counts) are each 2 x 2 blocks of 16;
  // lane l reads 8 bf16 of K (16-byte chunk 4 kk + l / 16) of row l mod 16 of
  // a block, and holds output columns 4 (l / 16) .. + 3 of row l mod 16.
  // (Against 32 x 32 x 16 in a dense probe of the same loop: 3-7% faster,
  // with the shader clock higher.)
  constexpr int kR16 = 2 * kRB, kC16 = 2 * kCB;
  // Every block starts at a multiple of 16 rows and the chunk swizzle
  // depends on the row mod 16 only, so one lane offset per K sub-step
  // addresses the same row of every block; the blocks differ by constants.
  int lane_off[kBK / 32];
#pragma unroll
  for (int kk = 0; kk < kBK / 32; ++kk)
    lane_off[kk] = r16 * kBK + (((4 * kk + q4) ^ swz_row<kChunks>(r16)) << 3);
  const int a_row0 = wm * kRB * 32;
  auto b_row0 = [&](int c16) {   // first row of this wave's 16-row block c16 of B
    const int c = c16 >> 1, half = c16 & 1;
    if constexpr (kEpi == FWD_FC1)
      return (c < kCB / 2 ? 0 : kBN / 2) + wn * (kCB / 2) * 32 + (c % (kCB / 2)) * 32 + half * 16;
    else
      return wn * kCB * 32 + c * 32 + half * 16;
  };

  f32x4 acc[kR16][kC16];
  // A wave with any live row block multiplies all of its blocks (rows past
  // the segment are zero in LDS): no branch inside the K step, so the next
  // block's fragment can be read while this block's MFMAs run.
  auto compute = [&](int slot, int nrb) {
    if (nrb == 0) return;
    const uint16_t* As = ring_a + slot * C::kATileE + a_row0 * kBK;
    const uint16_t* Bs = ring_b + slot * C::kBTileE;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      bf16x8 bv[kC16], av[2];
#pragma unroll
      for (int c = 0; c < kC16; ++c)
        bv[c] = *reinterpret_cast<const bf16x8*>(Bs + b_row0(c) * kBK + lane_off[kk]);
      av[0] = *reinterpret_cast<const bf16x8*>(As + lane_off[kk]);
#pragma unroll
      for (int i = 0; i < kR16; ++i) {
        if (i + 1 < kR16)
          av[(i + 1) & 1] = *reinterpret_cast<const bf16x8*>(As + (i + 1) * 16 * kBK + lane_off[kk]);
#pragma unroll
        for (int c = 0; c < kC16; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[c], av[i & 1], acc[i][c], 0, 0, 0);
        if (i + 1 < kR16) __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Epilogue staging without padding: a staged row is kCols bf16, its
  // 16-byte chunk c stored at c ^ (row mod 16); rows go to the two ring
  // slots not being filled (region 0: A slot, region 1: B slot, 32 KB each).
  constexpr int kCols = nbn;
  constexpr int kRowB = kCols * 2;                     // staged row bytes
  constexpr int kRR = 32768 / kRowB;                   // rows per region
  constexpr int kPassRows = 2 * kRR;
  constexpr int kPass = (kBM + kPassRows - 1) / kPassRows;
  constexpr int kChunksRow = kCols / 8;
  static_assert(C::kATileE * 2 == 32768 && C::kBTileE * 2 == 32768, "32 KB ring slots");
  static_assert(kPassRows % (kRB * 32) == 0 && kBM % kPassRows == 0, "waves stage whole passes");
  const int limit = kEpi == FWD_FC1 ? p.F : p.d;
  auto epilogue = [&](const TileIdx& ti, int nrb, int free_slot) {
    const int m0 = ti.m0, n0 = ti.nt * nbn;
    uint8_t* reg0 = reinterpret_cast<uint8_t*>(ring_a + free_slot * C::kATileE);
    uint8_t* reg1 = reinterpret_cast<uint8_t*>(ring_b + free_slot * C::kBTileE);
    auto staged = [&](int lp, int byte) -> uint8_t* {   // row lp of the pass, byte offset
      const int rr = lp % kRR;
      uint8_t* base = lp < kRR ? reg0 : reg1;
      return base + rr * kRowB + ((((byte >> 4) ^ (rr & 15))) << 4) + (byte & 15);
    };
    const int wrow0 = wm * kRB * 32;
    // the lane's row and column within a 16 x 16 block, re-derived here from
    // an opaque copy of the lane index so that the staging addresses are
    // formed per tile instead of being hoisted and kept live through the
    // K loop (they would push its registers past the 128 of 4 waves per SIMD)
    int le = lane;
    asm volatile("" : "+v"(le));
    const int r16 = le & 15, q4 = le >> 4;
    // fc2: the row scales of this lane's rows, loaded (branch-free: a
    // descriptor over the tile's rows, 0 bytes when there is no scale) and
    // waited for before the first pass: loaded inside a later pass, they
    // would be waited for with vmcnt(0) behind the earlier pass's stores
    float scl[kR16];
    if constexpr (kEpi == FWD_FC2) {
      const bool has_scale = p.scale != nullptr;
      const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(p.scale + (has_scale ? m0 : 0)), 0,
          has_scale ? (ti.mend - m0) * 4 : 0, kRsrcWord3);
#pragma unroll
      for (int i = 0; i < kR16; ++i) {
        const float v = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs_s, (wrow0 + i * 16 + r16) * 4, 0, 0));
        scl[i] = has_scale ? v : 1.0f;
      }
#pragma unroll
      for (int i = 0; i < kR16; ++i) asm volatile("" ::"v"(scl[i]));   // the one wait, here
    }
#pragma unroll
    for (int ps = 0; ps < kPass; ++ps) {
      if (wrow0 / kPassRows == ps) {
#pragma unroll
        for (int i = 0; i < kR16; ++i) {
          if ((i >> 1) >= nrb) continue;
          const int lp = wrow0 - ps * kPassRows + i * 16 + r16;
          if constexpr (kEpi == FWD_FC1) {
#pragma unroll
            for (int c16 = 0; c16 < kC16 / 2; ++c16) {   // G blocks; U is kC16 / 2 further
              const int fl = wn * (kCB / 2) * 32 + c16 * 16 + 4 * q4;
              const f32x4& G = acc[i][c16];
              const f32x4& U = acc[i][c16 + kC16 / 2];
              float a4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) a4[e] = G[e] * sigmoid_fast(G[e]) * U[e];
              *reinterpret_cast<u32x2*>(staged(lp, fl * 2)) = pack4_bf16(a4[0], a4[1], a4[2], a4[3]);
            }
          } else {
            const float sc = scl[i];
#pragma unroll
            for (int c16 = 0; c16 < kC16; ++c16) {
              const int nl = wn * kCB * 32 + c16 * 16 + 4 * q4;
              const f32x4& Y = acc[i][c16];
              *reinterpret_cast<u32x2*>(staged(lp, nl * 2)) =
                  pack4_bf16(Y[0] * sc, Y[1] * sc, Y[2] * sc, Y[3] * sc);
            }
          }
        }
      }
      // LDS only: a __syncthreads fence would also wait for the next tile's loads
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int i = tid; i < kPassRows * kChunksRow; i += C::kThreads) {
        const int lp = i / kChunksRow, ch = i - lp * kChunksRow;
        const int row = m0 + ps * kPassRows + lp;
        const int col = n0 + ch * 8;
        if (row < ti.mend && col < limit)
          *reinterpret_cast<u32x4*>(p.out + static_cast<size_t>(row) * limit + col) =
              *reinterpret_cast<const u32x4*>(staged(lp, ch * 16));
      }
      if (ps + 1 < kPass) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if constexpr (kEpi == FWD_FC1) {
      // G and U saved for the backward ([G | U] rows of 2F): staged like A,
      // one pass each, so they leave as 16-byte lanes over whole rows
      static_assert(kPass == 1, "one staging pass holds the fc1 tile");
      if (p.out2) {
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // staging free again
#pragma unroll
          for (int i = 0; i < kR16; ++i) {
            if ((i >> 1) >= nrb) continue;
            const int lp = wrow0 + i * 16 + r16;
#pragma unroll
            for (int c16 = 0; c16 < kC16 / 2; ++c16) {
              const int fl = wn * (kCB / 2) * 32 + c16 * 16 + 4 * q4;
              const f32x4& X = half ? acc[i][c16 + kC16 / 2] : acc[i][c16];
              *reinterpret_cast<u32x2*>(staged(lp, fl * 2)) = pack4_bf16(X[0], X[1], X[2], X[3]);
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          int t0 = tid;
          asm volatile("" : "+v"(t0));   // keep this loop's addressing out of the kernel preamble
#pragma unroll
          for (int i = t0; i < kPassRows * kChunksRow; i += C::kThreads) {
            const int lp = i / kChunksRow, ch = i - lp * kChunksRow;
            const int row = m0 + lp;
            const int col = n0 + ch * 8;
            if (row < ti.mend && col < p.F)
              *reinterpret_cast<u32x4*>(p.out2 + static_cast<size_t>(row) * 2 * p.F + half * p.F + col) =
                  *reinterpret_cast<const u32x4*>(staged(lp, ch * 16));
          }
        }
      }
    }
  };

  // live 32-row blocks of this wave; none when all its columns lie past the
  // output (the last column tile's padding): its MFMAs are skipped
  auto live_blocks = [&](const TileIdx& ti) {
    const int rows = ti.mend - ti.m0 - wm * kRB * 32;
    const int col0 = ti.nt * nbn + wn * (kEpi == FWD_FC1 ? kCB / 2 : kCB) * 32;
    if (col0 >= limit) return 0;
    return rows <= 0 ? 0 : min(kRB, (rows + 31) >> 5);
  };

  TileState cur, nxt;
  setup(0, cur);
  __syncthreads();              // s_cum (read by setup) is never overwritten; the ring is free
  issue(cur, 0, 0);
  if (ntiles > 1) setup(1, nxt);
  int g = 0;                    // global K step: ring slot g & 1
#pragma unroll 1
  for (int j = 0; j < ntiles; ++j) {
    const int nrb = live_blocks(cur.ti);
#pragma unroll
    for (int i = 0; i < kR16; ++i)
#pragma unroll
      for (int c = 0; c < kC16; ++c) acc[i][c] = f32x4{};
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt, ++g) {
      // everything this wave issued has landed (the ring's loads, the gathers
      // of the next tile's setup, the last epilogue's stores); the barrier
      // makes tile g visible and frees slot (g + 1) & 1
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
      if (kt + 1 < nk) issue(cur, kt + 1, (g + 1) & 1);
      else if (j + 1 < ntiles) issue(nxt, 0, (g + 1) & 1);
      compute(g & 1, nrb);
    }
    asm volatile("s_barrier" ::: "memory");   // every wave is done reading slot (g - 1) & 1
    epilogue(cur.ti, nrb, (g - 1) & 1);
    if (j + 1 < ntiles) {
      cur = nxt;
      if (j + 2 < ntiles) setup(j + 2, nxt);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class C, int kEpi>
__global__ __launch_bounds__(C::kThreads, 1) void ggfp_kernel(FwdParams p) {
  ggfp_body<C, kEpi>(p);
}

// ---------------------------------------------------------------------------
// fp32 path (MOE_F32): LDS-tiled FMA, 64 x 64 x 16 tiles, 4 x 4 outputs per
// thread, same tile enumeration and epilogue semantics.
// ---------------------------------------------------------------------------
constexpr int kFM = 64, kFN = 64, kFK = 16;

template <int kEpi>
__global__ __launch_bounds__(256) void ggf_f32_kernel(int E, int F, int d, int K, int ntn,
                                                      const int32_t* __restrict__ offsets,
                                                      const float* __restrict__ a, int lda,
                                                      const int32_t* __restrict__ gather,
                                                      int a_rows,
                                                      const float* __restrict__ b, int ldb,
                                                      size_t b_estride,
                                                      const float* __restrict__ scale,
                                                      float* __restrict__ out,
                                                      float* __restrict__ out2) {
  __shared__ float As[kFK][kFM + 4];
  __shared__ float Bs[kFK][kFN + 4];
  __shared__ int s_cum[1025];
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x;
  tile_prefix<256>(offsets, E, kFM, ntn, s_cum, s_tmp);
  const int total = s_cum[E];
  if (static_cast<int>(blockIdx.x) >= total) return;
  const TileIdx ti = tile_decode(offsets, E, kFM, ntn, blockIdx.x, s_cum);
  const int m0 = ti.m0;
  const int nt = ti.nt;
  const float* bexp = b + static_cast<size_t>(ti.e) * b_estride;

  const int ty = tid >> 4, tx = tid & 15;
  // B-tile rows of this thread: FC1 {2tx, 2tx+1, 32+2tx, 33+2tx}; FC2 4tx..4tx+3
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bcol[j] = (kEpi == FWD_FC1) ? ((j >> 1) * 32 + 2 * tx + (j & 1)) : (4 * tx + j);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kFK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;          // 64 rows x 16 k
      const int r = c >> 4, kk = c & 15;
      const int k = k0 + kk;
      int ar = m0 + r;
      if (ar > ti.mend - 1) ar = ti.mend - 1;
      if (gather) ar = gather[ar];            // outside [0, a_rows): a zero row
      As[kk][r] = k < K && ar >= 0 && (!gather || ar < a_rows)
                      ? a[static_cast<size_t>(ar) * lda + k] : 0.0f;
      int br;
      if constexpr (kEpi == FWD_FC1) {
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
    if (row >= ti.mend) continue;
    const size_t rowz = static_cast<size_t>(row);
    if constexpr (kEpi == FWD_FC1) {
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

// Tile-packed weights (the B operand of the expert GEMMs stored the way the
// forward stages it): for expert e, column tile t and K tile kt, one
// contiguous block of kBN rows x kBK columns,
//     packed[e][t][kt][r][c] = W[e][row(t, r)][kt kBK + c]   (0 past K or rows)
// with row(t, r) = t kBN + r for the second GEMM (W2 [E, d, F]) and, for the
// gated first GEMM (W1 [E, 2F, d]), gate rows t kBN/2 + r for r < kBN/2 and
// the matching up rows F + t kBN/2 + r - kBN/2 after them.  Each K tile of a
// weight panel is then one sequential 32 KB read instead of kBN rows of 128
// bytes at the row stride (measured on MI355X: 6.2-6.3 TB/s versus 4.4-4.8
// TB/s streamed from HBM).
constexpr int kPackBN = GemmCfg::kBN, kPackBK = GemmCfg::kBK;

inline int64_t pack_tiles(int64_t rows, int gated) {
  return gated ? (rows / 2 + kPackBN / 2 - 1) / (kPackBN / 2) : (rows + kPackBN - 1) / kPackBN;
}
inline int64_t pack_ktiles(int64_t K) { return (K + kPackBK - 1) / kPackBK; }
inline int64_t pack_expert_elems(int64_t rows, int64_t K, int gated) {
  return pack_tiles(rows, gated) * pack_ktiles(K) * kPackBN * kPackBK;
}

// one thread per 16-byte chunk of the packed output
__global__ __launch_bounds__(256) void pack_b_kernel(int64_t total, int rows, int K, int gated,
                                                     int ntile, int nkt,
                                                     const u32x4* __restrict__ w,
                                                     u32x4* __restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total) return;
  constexpr int kCh = kPackBK / 8;
  const int c8 = static_cast<int>(i % kCh);
  int64_t q = i / kCh;
  const int r = static_cast<int>(q % kPackBN);
  q /= kPackBN;
  const int kt = static_cast<int>(q % nkt);
  q /= nkt;
  const int t = static_cast<int>(q % ntile);
  const int64_t e = q / ntile;
  int row;
  if (gated) {
    const int F = rows / 2, h = kPackBN / 2;
    const int f = t * h + (r < h ? r : r - h);
    row = f < F ? (r < h ? f : F + f) : -1;
  } else {
    row = t * kPackBN + r;
    row = row < rows ? row : -1;
  }
  const int k = kt * kPackBK + c8 * 8;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row >= 0 && k < K) v = w[((e * rows + row) * K + k) / 8];
  out[i] = v;
}

// One workgroup per CU (at most one per tile), a multiple of the 8 XCDs.
static unsigned persistent_grid(int64_t tiles) {
  const int64_t cus = device_cu_count();
  const int64_t g = std::min<int64_t>(cus, (tiles + 7) / 8 * 8);
  return static_cast<unsigned>(std::max<int64_t>(8, g / 8 * 8));
}

hipError_t launch_grouped_fwd_bf16(hipStream_t stream, int64_t N, int64_t d, int64_t F, int32_t E,
                                   const void* x_perm, const void* w1, const void* w2,
                                   const int32_t* offsets, const float* row_scale, void* y_perm,
                                   void* gu_save, uint16_t* a_buf, bool run_fc2,
                                   const int32_t* gather, int64_t a_rows, bool packed) {
  using C = GemmCfg;
  FwdParams p{};
  p.E = E; p.F = (int)F; p.d = (int)d; p.offsets = offsets;
  // fc1: [G | U] = X W1^T with the SwiGLU epilogue; kBN / 2 f per tile
  p.ntn = (int)((F + C::kBN / 2 - 1) / (C::kBN / 2));
  p.a = static_cast<const uint16_t*>(x_perm); p.lda = (int)d;
  p.gather = gather; p.a_rows = (int)a_rows;
  p.b = static_cast<const uint16_t*>(w1); p.ldb = (int)d;
  p.b_estride = packed ? static_cast<size_t>(pack_expert_elems(2 * F, d, 1))
                       : static_cast<size_t>(2 * F) * d;
  p.packed_b = packed; p.nkt = (int)pack_ktiles(d);
  p.K = (int)d;
  p.out = a_buf; p.out2 = static_cast<uint16_t*>(gu_save);
  p.ksplit = 1;
  const size_t lds = C::kLdsBytes + kScanInts * sizeof(int);
  hipError_t err = allow_lds(ggfp_kernel<C, FWD_FC1>, lds);
  if (err == hipSuccess) err = allow_lds(ggfp_kernel<C, FWD_FC2>, lds);
  if (err == hipSuccess)
    err = launch(ggfp_kernel<C, FWD_FC1>, dim3(persistent_grid(tiles_bound(N, E, C::kBM) * p.ntn)),
                 dim3(C::kThreads), lds, stream, p);
  if (err != hipSuccess || !run_fc2) return err;
  // fc2: Y = (A W2^T) * row_scale; kBN output columns per tile
  FwdParams q{};
  q.E = E; q.F = (int)F; q.d = (int)d; q.offsets = offsets;
  q.ntn = (int)((d + C::kBN - 1) / C::kBN);
  q.a = a_buf; q.lda = (int)F;
  q.b = static_cast<const uint16_t*>(w2); q.ldb = (int)F;
  q.b_estride = packed ? static_cast<size_t>(pack_expert_elems(d, F, 0))
                       : static_cast<size_t>(d) * F;
  q.packed_b = packed; q.nkt = (int)pack_ktiles(F);
  q.K = (int)F;
  q.scale = row_scale;
  q.out = static_cast<uint16_t*>(y_perm);
  q.ksplit = 1;
  return launch(ggfp_kernel<C, FWD_FC2>, dim3(persistent_grid(tiles_bound(N, E, C::kBM) * q.ntn)),
                dim3(C::kThreads), lds, stream, q);
}

int router_ksplit(int64_t T, int64_t d, int32_t E) {
  // about one workgroup per CU, each slab at least 8 K tiles.  Measured on
  // MI355X (route call, us; ksplit 1 / 2 / 4 / 8): T=4096 d=2048 E=128
  // 38 / 31 / 29 / 31; T=8192 d=2688 E=128 46 / 36 / 34 / 47; T=16384
  // d=2048 E=256 63 / 76 / 99 / -.  Fewer slabs also shrink the fp32 slab
  // traffic that route_topk sums.
  using C = RouterCfg;
  const int64_t tiles = ((T + C::kBM - 1) / C::kBM) * ((E + C::kBN - 1) / C::kBN);
  const int64_t nk = (d + C::kBK - 1) / C::kBK;
  int64_t s = (256 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, nk / 8));
  return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(s, 16)));
}

static size_t router_lds(int64_t d, int ksplit, bool gate) {
  using C = RouterCfg;
  const int64_t kchunk = ((d + C::kBK - 1) / C::kBK + ksplit - 1) / ksplit;
  const size_t gbytes = (static_cast<size_t>(kchunk) * C::kBK * 2 + 1023) / 1024 * 1024;
  return C::kLdsBytes + (gate ? gbytes : 0);
}

bool router_gate_fused(int64_t T, int64_t d, int32_t E) {
  return router_lds(d, router_ksplit(T, d, E), true) <= 160 * 1024;
}

hipError_t launch_router_logits_bf16(hipStream_t stream, int64_t T, int64_t d, int32_t E,
                                    const void* x, const void* w_router, const float* bias,
                                    float* logits, int ksplit, const void* gate_w,
                                    float* gate_out, int32_t* zero_counts) {
  using C = RouterCfg;
  FwdParams p{};
  p.E = 1; p.F = 1; p.d = E; p.offsets = nullptr; p.rows1 = (int)T;
  p.ntn = (E + C::kBN - 1) / C::kBN;
  p.a = static_cast<const uint16_t*>(x); p.lda = (int)d;
  p.b = static_cast<const uint16_t*>(w_router); p.ldb = (int)d;
  p.b_estride = static_cast<size_t>(E) * d;
  p.K = (int)d;
  p.scale = bias;
  p.outf = logits;
  p.ksplit = ksplit;
  p.outf_split = static_cast<size_t>(T) * E;
  p.gate_w = static_cast<const uint16_t*>(gate_w);
  p.gate_out = gate_out;
  p.zero_i32 = zero_counts;
  p.zero_n = E;
  // the gate weights of one K slab sit behind the rings
  const size_t lds = router_lds(d, ksplit, gate_w != nullptr);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  hipError_t err = allow_lds(ggf_kernel<C, FWD_LOGITS>, lds);
  if (err != hipSuccess) return err;
  return launch(ggf_kernel<C, FWD_LOGITS>, dim3(tiles_bound(T, 1, C::kBM) * p.ntn, ksplit),
                dim3(C::kThreads), lds, stream, p);
}

}  // namespace moe

using namespace moe;

moe_status moe_grouped_check(moe_dtype dt, int64_t N, int64_t d, int64_t F, int32_t E);

extern "C" size_t moe_grouped_swiglu_fwd_workspace_size(int64_t N, int64_t F, moe_dtype dt) {
  if (N < 0 || F < 1) return 0;
  return static_cast<size_t>(N) * F * elt_size(dt) + 256;
}

// The forward, with row r of the first GEMM read from x[gather[r]] when
// gather is non-NULL (x then has T rows), else from x[r].
static moe_status grouped_fwd(hipStream_t stream, moe_dtype dt, int64_t N, int64_t d, int64_t F,
                              int32_t E, int64_t T, const void* x, const int32_t* gather,
                              const void* w1, const void* w2, const int32_t* expert_offsets,
                              const float* row_scale, void* y_perm, void* gu_save, void* ws,
                              size_t ws_bytes, bool packed = false) {
  moe_status st = moe_grouped_check(dt, N, d, F, E);
  if (st != MOE_OK) return st;
  if (packed && dt != MOE_BF16) return MOE_ERR_DTYPE;
  // packed per-expert blocks are addressed with 32-bit byte offsets
  if (packed && 2 * std::max(pack_expert_elems(2 * F, d, 1), pack_expert_elems(d, F, 0)) >=
                    (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  // with no rows (N = 0) the row buffers may be empty (NULL) and nothing runs
  if (!w1 || !w2 || !expert_offsets || (N > 0 && (!x || !y_perm))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(expert_offsets) ||
      !aligned16(row_scale) || !aligned16(y_perm) || !aligned16(gu_save) || !aligned16(ws) ||
      !aligned16(gather))
    return MOE_ERR_ALIGNMENT;
  if (N == 0) return MOE_OK;
  if (!ws || ws_bytes < moe_grouped_swiglu_fwd_workspace_size(N, F, dt)) return MOE_ERR_WORKSPACE;
  if (dt == MOE_BF16) {
    return hip_status(launch_grouped_fwd_bf16(stream, N, d, F, E, x, w1, w2, expert_offsets,
                                              row_scale, y_perm, gu_save,
                                              static_cast<uint16_t*>(ws), true, gather, T, packed));
  }
  float* a_buf = static_cast<float*>(ws);
  const int ntn1 = (int)((F + 31) / 32);
  hipError_t err = launch(ggf_f32_kernel<FWD_FC1>, dim3(tiles_bound(N, E, kFM) * ntn1), dim3(256),
                          0, stream, E, (int)F, (int)d, (int)d, ntn1, expert_offsets,
                          static_cast<const float*>(x), (int)d, gather, (int)T,
                          static_cast<const float*>(w1), (int)d, static_cast<size_t>(2 * F) * d,
                          (const float*)nullptr, a_buf, static_cast<float*>(gu_save));
  if (err == hipSuccess) {
    const int ntn2 = (int)((d + kFN - 1) / kFN);
    err = launch(ggf_f32_kernel<FWD_FC2>, dim3(tiles_bound(N, E, kFM) * ntn2), dim3(256), 0,
                 stream, E, (int)F, (int)d, (int)F, ntn2, expert_offsets, (const float*)a_buf,
                 (int)F, (const int32_t*)nullptr, 0, static_cast<const float*>(w2), (int)F,
                 static_cast<size_t>(d) * F, row_scale, static_cast<float*>(y_perm),
                 (float*)nullptr);
  }
  return hip_status(err);
}

extern "C" moe_status moe_grouped_swiglu_fwd(hipStream_t stream, moe_dtype dt, int64_t N,
                                             int64_t d, int64_t F, int32_t E,
                                             const void* x_perm, const void* w1, const void* w2,
                                             const int32_t* expert_offsets,
                                             const float* row_scale, void* y_perm,
                                             void* gu_save, void* ws, size_t ws_bytes) {
  return grouped_fwd(stream, dt, N, d, F, E, N, x_perm, nullptr, w1, w2, expert_offsets,
                     row_scale, y_perm, gu_save, ws, ws_bytes);
}

extern "C" moe_status moe_grouped_swiglu_fwd_gather(hipStream_t stream, moe_dtype dt, int64_t N,
                                                    int64_t d, int64_t F, int32_t E, int64_t T,
                                                    const void* x, const int32_t* row_token,
                                                    const void* w1, const void* w2,
                                                    const int32_t* expert_offsets,
                                                    const float* row_scale, void* y_perm,
                                                    void* gu_save, void* ws, size_t ws_bytes) {
  if (!row_token) return MOE_ERR_INVALID_ARG;
  if (T < 1) return MOE_ERR_SHAPE;
  // gathered rows are addressed from x's start with 32-bit byte offsets
  if (T * d * static_cast<int64_t>(elt_size(dt)) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  return grouped_fwd(stream, dt, N, d, F, E, T, x, row_token, w1, w2, expert_offsets, row_scale,
                     y_perm, gu_save, ws, ws_bytes);
}

extern "C" size_t moe_pack_weights_size(int32_t E, int64_t rows, int64_t K, int32_t gated) {
  if (E < 1 || rows < 1 || K < 1 || (gated && rows % 2)) return 0;
  return static_cast<size_t>(E) * pack_expert_elems(rows, K, gated ? 1 : 0) * sizeof(uint16_t);
}

extern "C" moe_status moe_pack_weights(hipStream_t stream, moe_dtype dt, int32_t E, int64_t rows,
                                       int64_t K, int32_t gated, const void* w, void* w_packed) {
  if (dt != MOE_BF16) return MOE_ERR_DTYPE;
  if (!w || !w_packed) return MOE_ERR_INVALID_ARG;
  if (E < 1 || rows < 1 || K < 1 || (gated && rows % 2)) return MOE_ERR_SHAPE;
  if (K % 8) return MOE_ERR_ALIGNMENT;
  if (rows >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(w_packed)) return MOE_ERR_ALIGNMENT;
  const int g = gated ? 1 : 0;
  const int64_t total = static_cast<int64_t>(E) * pack_expert_elems(rows, K, g) / 8;
  return hip_status(launch(pack_b_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                           dim3(256), 0, stream, total, (int)rows, (int)K, g,
                           (int)pack_tiles(rows, g), (int)pack_ktiles(K),
                           static_cast<const u32x4*>(w), static_cast<u32x4*>(w_packed)));
}

extern "C" moe_status moe_grouped_swiglu_fwd_packed(hipStream_t stream, moe_dtype dt, int64_t N,
                                                    int64_t d, int64_t F, int32_t E, int64_t T,
                                                    const void* x, const int32_t* row_token,
                                                    const void* w1_packed, const void* w2_packed,
                                                    const int32_t* expert_offsets,
                                                    const float* row_scale, void* y_perm,
                                                    void* gu_save, void* ws, size_t ws_bytes) {
  if (row_token) {
    if (T < 1) return MOE_ERR_SHAPE;
    if (T * d * static_cast<int64_t>(elt_size(dt)) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  } else {
    T = N;
  }
  return grouped_fwd(stream, dt, N, d, F, E, T, x, row_token, w1_packed, w2_packed,
                     expert_offsets, row_scale, y_perm, gu_save, ws, ws_bytes, true);
}
