// W4A4 NVFP4 GEMM for gfx950:  out[m, n] = g_a * g_w[seg(n)] * sum_k A[m,k] * W[n,k]
// with A and W given as E2M1 codes + one E4M3 scale per 16 elements
// (evolve.pub review of arXiv 2609.04098, "Scope & Claims"), the weight made
// of row segments that each keep their own global scale (the fused-GEMM
// global-scale mismatch, chatpaper.ai English abstract; evolve.pub review,
// "Key claims under review"), and an optional GDN gate epilogue
// (chatpaper.ai abstract, mechanism (ii)).
//
// Why fp16 MFMA on decoded operands.  gfx950's scaled MFMAs take one E8M0
// (power-of-two) scale per 32 elements; an E4M3 scale per 16 elements fits
// neither the block size nor the scale format, and folding it into the
// element needs 6 significand bits, which FP8/FP6/FP4 lack.  But
// e2m1 * e4m3 has <= 6 significant bits and lies in [2^-10, 2688], so it is
// EXACT in fp16 (11 bits, normal range 2^-14..65504).  Products of two such
// values have <= 12 bits and are exact in fp32; only the fp32 accumulation
// rounds.  The global scales are applied once, in the epilogue.
//
// Data path per workgroup (BM x BN output tile, BK = 128):
//   global -> LDS by LDS-DMA (buffer_load ... lds, no VGPR staging), raw
//   packed codes + scale bytes (0.5625 B per element, 3.6x less LDS traffic
//   than staging fp16), three stages so two tiles are in flight while one is
//   computed; each wave reads its fragments from LDS in MFMA lane order (one
//   16-byte read per lane, consecutive lanes consecutive addresses) and
//   decodes them in registers: 4 x v_cvt_scalef32_pk_f16_fp4 + 4 x
//   v_pk_mul_f16 per 8 elements; then v_mfma_f32_32x32x16_f16.
//   Large shapes whose K is a whole number of K tiles run gemm_kernel_pipe:
//   one wave per SIMD with 128x128 outputs each (a decoded fragment feeds
//   four MFMAs), software-pipelined across K tiles; other shapes run
//   gemm_kernel (two waves per SIMD for the 256-wide tiles, and the ragged
//   last K tile through registers).
//
// K order inside a 128-wide K tile.  The MFMA sums over its 16 k values, so
// any permutation of k that A and W share is allowed.  Lane (row, h) of a
// fragment feeds the k-values {64h + 8t + e : e < 8} at k-step t (t < 8),
// so one lane's codes for a whole tile are 32 contiguous bytes of its row,
// and its scales are 4 contiguous bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_util.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

using namespace dev;

constexpr int kBK = 128;              // K elements per tile
constexpr int kRowCodeBytes = kBK / 2;  // 64 code bytes per row per tile
constexpr int kRowScaleBytes = kBK / 16;  // 8 scale bytes per row per tile

// SCHED_VALU > 0: after each k-step's MFMAs, ask the scheduler to interleave
// them one by one with SCHED_VALU decode VALU ops (measured per config).
template <int BM_, int BN_, int WGM_, int WGN_, int SCHED_VALU>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WGM = WGM_, WGN = WGN_;
  static constexpr int kSchedValu = SCHED_VALU;
  static constexpr int kThreads = WGM * WGN * 64;
  static constexpr int kWavesPerSimd = kThreads / 256;  // one workgroup per CU
  static constexpr int TM = BM / WGM, TN = BN / WGN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;    // 32x32 fragments per wave
  static constexpr int kACode = BM * kRowCodeBytes;
  static constexpr int kBCode = BN * kRowCodeBytes;
  static constexpr int kAScale = BM * kRowScaleBytes;
  static constexpr int kBScale = BN * kRowScaleBytes;
  static constexpr int kStage = kACode + kBCode + kAScale + kBScale;
  // the pipelined kernel's stage: scales as 16 bytes per row (see AsyncLoader)
  static constexpr int kStageWide = kACode + kBCode + (BM + BN) * 16;
  static constexpr int kChunks = (BM + BN) * 4;  // 16-byte code chunks per stage
  static constexpr int kChunkIters = (kChunks + kThreads - 1) / kThreads;
  static constexpr int kScaleIters = (BM + BN + kThreads - 1) / kThreads;
  // waves per SIMD the pipelined kernel allows (two workgroups per CU when
  // the accumulators are few enough for two waves' registers)
  static constexpr int kPipeOcc = FM * FN <= 4 ? 2 : 1;
  static_assert(BM % (32 * WGM) == 0 && BN % (32 * WGN) == 0, "tile shape");
};

// LDS byte offset of 16-byte chunk q (0..3) of tile row `row`: fragment
// (row / 32) holds 2 KB = [chunk parity c][lane][16 B], lane = 32*(q/2) + row%32.
__device__ inline int code_slot(int row, int q) {
  return (row >> 5) * 2048 + (q & 1) * 1024 + ((((q >> 1) << 5) | (row & 31)) << 4);
}
// LDS byte offset of scale dword h (0..1) of tile row `row`: [fragment][lane][4 B].
__device__ inline int scale_slot(int row, int h) {
  return (row >> 5) * 256 + ((((h) << 5) | (row & 31)) << 2);
}

// Epilogue modes.  kEpiGate: GDN gate columns.  kEpiSwiglu: the tile's 256
// W rows are 128 gate rows and the 128 matching up rows (see w_row), and the
// epilogue writes h = silu(gate) * up for 128 columns of h.
enum { kEpiPlain = 0, kEpiGate = 1, kEpiSwiglu = 2 };

// Output columns covered by one tile.
template <class C, int EPI>
constexpr int tile_cols() { return EPI == kEpiSwiglu ? C::BN / 2 : C::BN; }

// Weight row feeding tile-local B row `row` (0..BN-1), clamped in range.
// kEpiSwiglu: wave column wn owns fragments FN*wn .. FN*wn+FN-1; its first
// FN/2 fragments hold gate rows and the others the up rows of the same h
// columns, so each lane ends with gate and up accumulators side by side.
template <class C, int EPI>
__device__ inline int w_row(const GemmArgs& p, int n0, int n_hi, int row) {
  if constexpr (EPI == kEpiSwiglu) {
    constexpr int TN = C::BN / C::WGN;
    const int f = row >> 5, wn = f / C::FN, j = f % C::FN;
    const bool up = j >= C::FN / 2;
    const int hl = wn * (TN / 2) + (up ? j - C::FN / 2 : j) * 32 + (row & 31);
    return (up ? p.ep.inter : 0) + min(n0 + hl, p.ep.inter - 1);
  } else {
    return min(n0 + row, n_hi - 1);
  }
}

// Asynchronous global -> LDS copy of one full K tile with gfx950's
// buffer_load ... lds (LDS DMA): no VGPR staging, no ds_write.  One
// instruction moves one 1 KB "group" = 64 lanes x 16 bytes, written to
// LDS at (group base + lane * 16); the group layout above makes lane l of
// fragment f, parity c, fetch 16 code bytes of row 32f + l%32 at chunk
// q = 2(l/32) + c.  Scale groups move 64 lanes x 4 bytes the same way.
// Waves split the groups round-robin.  Row offsets beyond M/N are clamped
// to the last row (results of those rows are never stored).  The K tile
// index enters as the uniform soffset, so the per-lane offsets are fixed.
//
// WIDE (the pipelined kernel): each scale copy moves 16 bytes per lane, one
// row's scale bytes of this K tile and the next (8 + 8), 64 rows per copy
// into [row][16 B]: half as many scale copies; the second 8 bytes are not
// used (past the last row they read beyond the buffer's end, which returns
// zeros).
template <class C, int EPI, bool WIDE = false>
struct AsyncLoader {
  static constexpr int kWaves = C::kThreads / 64;
  static constexpr int kScaleRows = WIDE ? 64 : 32;  // rows per scale copy
  static constexpr int kCodeGroups = (C::BM + C::BN) / 32 * 2;
  static constexpr int kScaleGroups = (C::BM + C::BN) / kScaleRows;
  static constexpr int kCodePer = (kCodeGroups + kWaves - 1) / kWaves;
  static constexpr int kScalePer = (kScaleGroups + kWaves - 1) / kWaves;
  i32x4 ra_c, ra_s, rw_c, rw_s;
  int cvoff[kCodePer], svoff[kScalePer];
  int clds[kCodePer], slds[kScalePer];  // wave-uniform LDS offsets in the stage
  bool cB[kCodePer], sB[kScalePer];

  __device__ __attribute__((always_inline)) void init(const GemmArgs& p, int m0, int n0, int n_hi, int wave,
                                                     int lane) {
    ra_c = buffer_rsrc(p.a_codes, (uint32_t)((int64_t)p.M * p.lda_c));
    ra_s = buffer_rsrc(p.a_scales, (uint32_t)((int64_t)p.M * p.lda_s));
    rw_c = buffer_rsrc(p.w_codes, (uint32_t)((int64_t)p.N * p.ldw_c));
    rw_s = buffer_rsrc(p.w_scales, (uint32_t)((int64_t)p.N * p.ldw_s));
#pragma unroll
    for (int i = 0; i < kCodePer; ++i) {
      int g = wave + i * kWaves;
      if (g >= kCodeGroups) g = 0;  // idle slot (never issued)
      const bool isB = g >= C::BM / 32 * 2;
      const int gg = isB ? g - C::BM / 32 * 2 : g;
      const int f = gg >> 1, c = gg & 1;
      const int row = f * 32 + (lane & 31), q = 2 * (lane >> 5) + c;
      const int grow = isB ? w_row<C, EPI>(p, n0, n_hi, row) : min(m0 + row, p.M - 1);
      cvoff[i] = (int)(grow * (isB ? p.ldw_c : p.lda_c)) + q * 16;
      clds[i] = (isB ? C::kACode : 0) + f * 2048 + c * 1024;
      cB[i] = isB;
    }
#pragma unroll
    for (int i = 0; i < kScalePer; ++i) {
      int g = wave + i * kWaves;
      if (g >= kScaleGroups) g = 0;
      const bool isB = g >= C::BM / kScaleRows;
      const int f = isB ? g - C::BM / kScaleRows : g;
      if constexpr (WIDE) {
        const int row = f * 64 + lane;
        const int grow = isB ? w_row<C, EPI>(p, n0, n_hi, row) : min(m0 + row, p.M - 1);
        svoff[i] = (int)(grow * (isB ? p.ldw_s : p.lda_s));
        slds[i] = C::kACode + C::kBCode + (isB ? C::BM * 16 : 0) + f * 1024;
      } else {
        const int row = f * 32 + (lane & 31), h = lane >> 5;
        const int grow = isB ? w_row<C, EPI>(p, n0, n_hi, row) : min(m0 + row, p.M - 1);
        svoff[i] = (int)(grow * (isB ? p.ldw_s : p.lda_s)) + h * 4;
        slds[i] = C::kACode + C::kBCode + (isB ? C::kAScale : 0) + f * 256;
      }
      sB[i] = isB;
    }
  }

  // Every wave issues exactly kCodePer + kScalePer copies per tile (idle
  // slots repeat group 0: identical bytes to identical LDS addresses), so
  // a fixed vmcnt tells how many tiles are still in flight.
  static constexpr int kPerTile = kCodePer + kScalePer;
  // Copy slot i alone (codes first, then scales): lets a caller spread one
  // tile's copies over several points of its instruction stream.
  __device__ __attribute__((always_inline)) void issue_slot(uint8_t* stage, int kt, int i) const {
    if (i < kCodePer) {
      const bool isB = kCodeSplit ? i * kWaves >= C::BM / 32 * 2 : cB[i];
      llvm_amdgcn_raw_buffer_load_lds(isB ? rw_c : ra_c, (lds_u32_ptr)(stage + clds[i]), 16, cvoff[i],
                                      kt * kRowCodeBytes, 0, 0);
    } else {
      const int j = i - kCodePer;
      const bool isB = kScaleSplit ? j * kWaves >= C::BM / kScaleRows : sB[j];
      llvm_amdgcn_raw_buffer_load_lds(isB ? rw_s : ra_s, (lds_u32_ptr)(stage + slds[j]), WIDE ? 16 : 4,
                                      svoff[j], kt * kRowScaleBytes, 0, 0);
    }
  }

  // When the waves split the A groups and all groups evenly (no idle
  // slots), slot i's operand (A or W) is the same for every wave and known
  // at compile time.
  static constexpr bool kCodeSplit = (C::BM / 32 * 2) % kWaves == 0 && kCodeGroups % kWaves == 0;
  static constexpr bool kScaleSplit = (C::BM / kScaleRows) % kWaves == 0 && kScaleGroups % kWaves == 0;
  __device__ __attribute__((always_inline)) void issue(uint8_t* stage, int kt) const {
#pragma unroll
    for (int i = 0; i < kCodePer; ++i) {
      const bool isB = kCodeSplit ? i * kWaves >= C::BM / 32 * 2 : cB[i];
      llvm_amdgcn_raw_buffer_load_lds(isB ? rw_c : ra_c, (lds_u32_ptr)(stage + clds[i]), 16, cvoff[i],
                                      kt * kRowCodeBytes, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kScalePer; ++i) {
      const bool isB = kScaleSplit ? i * kWaves >= C::BM / kScaleRows : sB[i];
      llvm_amdgcn_raw_buffer_load_lds(isB ? rw_s : ra_s, (lds_u32_ptr)(stage + slds[i]), WIDE ? 16 : 4,
                                      svoff[i], kt * kRowScaleBytes, 0, 0);
    }
  }
};

// The last K tile when K % 128 != 0, through registers: everything beyond K
// is zero (a zero code and a zero scale byte both decode to 0).
template <class C, int EPI>
struct TailLoader {
  static constexpr int kChunkIters = (C::kChunks + C::kThreads - 1) / C::kThreads;
  static constexpr int kScaleIters = (C::BM + C::BN + C::kThreads - 1) / C::kThreads;
  u32x4 chunk[kChunkIters];
  uint2 sc[kScaleIters];

  __device__ void load(const GemmArgs& p, int m0, int n0, int n_hi, int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int it = 0; it < kChunkIters; ++it) {
      const int id = it * C::kThreads + (int)threadIdx.x;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (id < C::kChunks) {
        const bool isB = id >= C::BM * 4;
        const int lid = isB ? id - C::BM * 4 : id;
        const int row = lid >> 2, q = lid & 3;
        const int grow = isB ? w_row<C, EPI>(p, n0, n_hi, row) : min(m0 + row, p.M - 1);
        const uint8_t* src = (isB ? p.w_codes + (int64_t)grow * p.ldw_c : p.a_codes + (int64_t)grow * p.lda_c) +
                             (k0 >> 1) + q * 16;
        const int rem = p.K - (k0 + q * 32);
        if (rem >= 32) {
          v = *reinterpret_cast<const u32x4*>(src);
        } else if (rem > 0) {  // rem == 16: the first 8 bytes only
          const uint2 h = *reinterpret_cast<const uint2*>(src);
          v[0] = h.x;
          v[1] = h.y;
        }
      }
      chunk[it] = v;
    }
    const int nb = (p.K >> 4) - kt * kRowScaleBytes;  // valid scale bytes in this tile (1..7)
#pragma unroll
    for (int it = 0; it < kScaleIters; ++it) {
      const int id = it * C::kThreads + (int)threadIdx.x;
      uint32_t lo = 0, hi = 0;
      if (id < C::BM + C::BN) {
        const bool isB = id >= C::BM;
        const int row = isB ? id - C::BM : id;
        const int grow = isB ? w_row<C, EPI>(p, n0, n_hi, row) : min(m0 + row, p.M - 1);
        const uint8_t* src = (isB ? p.w_scales + (int64_t)grow * p.ldw_s : p.a_scales + (int64_t)grow * p.lda_s) +
                             kt * kRowScaleBytes;
        for (int b = 0; b < nb; ++b) {
          const uint32_t byte = src[b];
          if (b < 4) lo |= byte << (8 * b);
          else hi |= byte << (8 * (b - 4));
        }
      }
      sc[it] = make_uint2(lo, hi);
    }
  }

  __device__ void store(uint8_t* stage) const {
#pragma unroll
    for (int it = 0; it < kChunkIters; ++it) {
      const int id = it * C::kThreads + (int)threadIdx.x;
      if (id < C::kChunks) {
        const bool isB = id >= C::BM * 4;
        const int lid = isB ? id - C::BM * 4 : id;
        *reinterpret_cast<u32x4*>(stage + (isB ? C::kACode : 0) + code_slot(lid >> 2, lid & 3)) = chunk[it];
      }
    }
#pragma unroll
    for (int it = 0; it < kScaleIters; ++it) {
      const int id = it * C::kThreads + (int)threadIdx.x;
      if (id < C::BM + C::BN) {
        const bool isB = id >= C::BM;
        const int row = isB ? id - C::BM : id;
        uint8_t* reg = stage + C::kACode + C::kBCode + (isB ? C::kAScale : 0);
        *reinterpret_cast<uint32_t*>(reg + scale_slot(row, 0)) = sc[it].x;
        *reinterpret_cast<uint32_t*>(reg + scale_slot(row, 1)) = sc[it].y;
      }
    }
  }
};

// Row stride (bytes) of a bf16 output tile staged in LDS: 16 bytes of
// padding move rows 4 apart (one MFMA lane group) off each other's banks.
template <int COLS>
constexpr int staged_row_bytes() { return COLS * 2 + 16; }

// Copy a staged bf16 tile [rows][cols] to global memory, 16 bytes per lane,
// rows at m0 (< M), columns at n0 (< n_hi); row starts 16-byte aligned.
template <int ROWS, int COLS, int THREADS>
__device__ inline void store_staged_tile(const uint8_t* tile, int m0, int n0, int M, int n_hi, uint16_t* out,
                                         int64_t ld_out) {
  constexpr int kChunksPerRow = COLS / 8;
  for (int c = (int)threadIdx.x; c < ROWS * kChunksPerRow; c += THREADS) {
    const int row = c / kChunksPerRow, col = (c % kChunksPerRow) * 8;
    const int m = m0 + row, n = n0 + col;
    if (m >= M || n >= n_hi) continue;
    const uint4 v = *reinterpret_cast<const uint4*>(tile + row * staged_row_bytes<COLS>() + col * 2);
    uint16_t* dst = out + (int64_t)m * ld_out + n;
    if (n + 8 <= n_hi) {
      store_stream16(dst, v.x, v.y, v.z, v.w);
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int q = 0; q < 8 && n + q < n_hi; ++q) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
    }
  }
}

// The tile's scaled accumulators as bf16 into LDS, then coalesced stores.
template <class C>
__device__ __attribute__((always_inline)) inline void stage_bf16_and_store(
    floatx16 (&acc)[C::FM][C::FN], int fm0, int fn0, int lane, uint8_t* smem, int m0, int n0, int M,
    int n_hi, uint16_t* out, int64_t ld_out) {
  constexpr int kRow = staged_row_bytes<C::BN>();
  barrier_lds();  // every wave is done reading the K tiles' stages
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = (fm0 + i) * 32 + 4 * (lane >> 5) + 8 * (r >> 2) + (r & 3);
        const int nl = (fn0 + j) * 32 + (lane & 31);
        *reinterpret_cast<uint16_t*>(smem + ml * kRow + nl * 2) = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
      }
  barrier_lds();
  store_staged_tile<C::BM, C::BN, C::kThreads>(smem, m0, n0, M, n_hi, out, ld_out);
}

// Gated-MLP epilogue.  Lane (row, h column) holds the gate accumulator in
// fragment j and the up accumulator in fragment j + FN/2.  Each is scaled and
// rounded to bf16 exactly as the plain epilogue stores it, then
// h = bf16(silu(gate) * up) as the SiLU*mul kernel computes it, so h is bit
// for bit the unfused chain's.  Outputs: bf16 h, the amax of |h| (one
// atomic max per wave into partials[workgroup % n]), and/or h quantized
// with a static global scale: h is staged in LDS as bf16 [BM][BN/2] and
// each thread quantizes whole 16-element blocks of a row from there.
template <class C>
__device__ __attribute__((always_inline)) inline void swiglu_epilogue(
    const GemmArgs& p, floatx16 (&acc)[C::FM][C::FN], int m0, int n0, int fm0, int wn, int lane,
    uint8_t* smem) {
  static_assert(C::FN % 2 == 0, "gate and up fragments pair up");
  constexpr int FH = C::FN / 2;
  constexpr int TH = C::BN / C::WGN / 2;  // h columns per wave
  constexpr int kHCols = C::BN / 2;       // h columns per tile
  const float ga = *p.ep.a_g;
  const float sg = ga * p.ep.seg_g[0], su = ga * p.ep.seg_g[1];
  const bool quant = p.ep.hq_codes != nullptr;
  constexpr int kRow = staged_row_bytes<kHCols>();
  barrier_lds();  // every wave is done reading the last K tile
  // Two rows (r, r+1) of a lane's column at a time: one conversion rounds
  // gate and up of a row to bf16 together, one rounds the two h values,
  // and the amax runs on the two bf16 magnitudes as packed 16-bit
  // integers (|h| >= 0: float order is integer order).  Rows and columns
  // past the output are left out of the amax (partial tiles only).
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 amax2 = {0, 0};
  auto rows = [&](auto full_tag) __attribute__((always_inline)) {
    constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      const int ml = (fm0 + i) * 32 + 4 * (lane >> 5);
#pragma unroll
      for (int j = 0; j < FH; ++j) {
        const int hl = wn * TH + j * 32 + (lane & 31);
        const int hcol = n0 + hl;
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int mloc = ml + 8 * (r >> 2) + (r & 3);  // rows mloc, mloc + 1
          const uint32_t gu0 = pack_bf16x2(acc[i][j][r] * sg, acc[i][j + FH][r] * su);
          const uint32_t gu1 = pack_bf16x2(acc[i][j][r + 1] * sg, acc[i][j + FH][r + 1] * su);
          const float h0 = silu(__uint_as_float(gu0 << 16)) * __uint_as_float(gu0 & 0xFFFF0000u);
          const float h1 = silu(__uint_as_float(gu1 << 16)) * __uint_as_float(gu1 & 0xFFFF0000u);
          const uint32_t hh = pack_bf16x2(h0, h1);
          uint32_t keep = 0x7FFF7FFFu;
          if constexpr (!FULL) {
            const int m = m0 + mloc;
            keep = hcol < p.ep.inter ? (m < p.M ? 0x7FFFu : 0u) | (m + 1 < p.M ? 0x7FFF0000u : 0u) : 0u;
          }
          amax2 = __builtin_elementwise_max(amax2, __builtin_bit_cast(u16x2, hh & keep));
          *reinterpret_cast<uint16_t*>(smem + mloc * kRow + hl * 2) = (uint16_t)hh;
          *reinterpret_cast<uint16_t*>(smem + (mloc + 1) * kRow + hl * 2) = (uint16_t)(hh >> 16);
        }
      }
    }
  };
  if (m0 + C::BM <= p.M && n0 + kHCols <= p.ep.inter) rows(std::true_type{});
  else rows(std::false_type{});
  if (p.ep.partials != nullptr) {
    float amax = __uint_as_float((uint32_t)(amax2[0] > amax2[1] ? amax2[0] : amax2[1]) << 16);
    amax = wave_max(amax);  // |h| >= 0: float order is unsigned integer order
    if (lane == 0)
      atomicMax(reinterpret_cast<unsigned int*>(p.ep.partials) + blockIdx.x % p.ep.n_partials,
                __float_as_uint(amax));
  }
  barrier_lds();
  if (p.ep.h != nullptr)
    store_staged_tile<C::BM, kHCols, C::kThreads>(smem, m0, n0, p.M, p.ep.inter, p.ep.h, p.ep.ld_h);
  if (quant) {
    const float gh = *p.ep.hq_g;
    constexpr int kBlocksPerRow = kHCols / 16;
    for (int b = (int)threadIdx.x; b < C::BM * kBlocksPerRow; b += C::kThreads) {
      const int mloc = b / kBlocksPerRow, jb = b % kBlocksPerRow;
      const int m = m0 + mloc, h0 = n0 + jb * 16;
      if (m >= p.M || h0 >= p.ep.inter) continue;  // inter % 16 == 0: blocks are whole
      const uint16_t* src = reinterpret_cast<const uint16_t*>(smem + mloc * kRow + jb * 32);
      const uint4 q0 = *reinterpret_cast<const uint4*>(src);
      const uint4 q1 = *reinterpret_cast<const uint4*>(src + 8);
      const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      float v[16];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[2 * e] = __uint_as_float(w[e] << 16);
        v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
      uint2 c;
      const uint32_t sc = quantize_block16(v, gh, &c);
      store_stream8(p.ep.hq_codes + (int64_t)m * p.ep.hq_ld_codes + h0 / 2, c.x, c.y);
      store_stream1(p.ep.hq_scales + (int64_t)m * p.ep.hq_ld_scales + h0 / 16, (uint8_t)sc);
    }
  }
}

// The epilogue of one output tile from its accumulators: the gated-MLP
// epilogue, or per output column its segment's global scale (and gate).
template <class C, int EPI>
__device__ __attribute__((always_inline)) inline void finish_tile(
    const GemmArgs& p, floatx16 (&acc)[C::FM][C::FN], int m0, int n0, int n_hi, int fm0, int fn0, int wn,
    int lane, uint8_t* smem) {
  if constexpr (EPI == kEpiSwiglu) {
    swiglu_epilogue<C>(p, acc, m0, n0, fm0, wn, lane, smem);
    return;
  }

  const float ga = *p.ep.a_g;
  float colscale[C::FN], alog[C::FN], dtb[C::FN];
  int coln[C::FN], kind[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    const int n = n0 + (fn0 + j) * 32 + (lane & 31);
    coln[j] = n;
    int seg = 0;
    for (int s = 1; s < p.ep.n_seg; ++s) seg += (n >= p.ep.seg_off[s]) ? 1 : 0;
    colscale[j] = ga * p.ep.seg_g[seg];
    kind[j] = 0;
    alog[j] = 0.0f;
    dtb[j] = 0.0f;
    if constexpr (EPI == kEpiGate) {
      kind[j] = (seg == p.ep.b_seg) ? 1 : (seg == p.ep.a_seg ? 2 : 0);
      if (kind[j] == 2 && n < n_hi) {
        const int h = n - p.ep.seg_off[seg];
        alog[j] = expf(p.ep.A_log[h]);
        dtb[j] = p.ep.dt_bias[h];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) {
    // A lane holds one column of fragment j: each gate is evaluated only in
    // fragments where some lane's column needs it (wave-uniform branches).
    bool any_sig = false, any_dec = false;
    if constexpr (EPI == kEpiGate) {
      any_sig = __ballot(kind[j] == 1) != 0;
      any_dec = __ballot(kind[j] == 2) != 0;
    }
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = acc[i][j][r] * colscale[j];
        float v = x;
        if (any_sig || any_dec) {
          const float t = kind[j] == 2 ? x + dtb[j] : x;
          const ExpNeg en = exp_neg(fabsf(t));
          if (any_sig) v = kind[j] == 1 ? sigmoid_from(t, en) : v;
          if (any_dec) v = kind[j] == 2 ? decay_from(t, en, alog[j]) : v;
        }
        acc[i][j][r] = v;
      }
  }
  // bf16 output through LDS: the MFMA layout gives each lane one column of
  // 16 rows, so direct stores are 2-byte scatters (one instruction per
  // element); staged, every lane stores 16 contiguous bytes.
  if (p.out_bf16 && p.ld_out % 8 == 0 && ((uintptr_t)p.out & 15) == 0 && n0 % 8 == 0) {
    stage_bf16_and_store<C>(acc, fm0, fn0, lane, smem, m0, n0, p.M, n_hi,
                            reinterpret_cast<uint16_t*>(p.out), p.ld_out);
    return;
  }
  const bool full_tile = m0 + C::BM <= p.M && n0 + C::BN <= n_hi;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int mb = m0 + (fm0 + i) * 32 + 4 * (lane >> 5);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int n = coln[j];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (full_tile || (m < p.M && n < n_hi)) {
          const float v = acc[i][j][r];
          if (p.out_bf16)
            reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.ld_out + n] = (uint16_t)f32_to_bf16_bits(v);
          else
            reinterpret_cast<float*>(p.out)[(int64_t)m * p.ld_out + n] = v;
        }
      }
    }
  }
}

// One launch covers the output columns [n_lo, n_hi).  EPI = kEpiGate is
// launched only over the gate segments' columns, so the bulk of the output
// runs gate-free code; kEpiSwiglu covers the columns of h.
template <class C, int EPI>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kWavesPerSimd, C::kWavesPerSimd)))
void gemm_kernel(const GemmArgs p, int n_lo, int n_hi) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tiles_m = (p.M + C::BM - 1) / C::BM;
  constexpr int kCols = tile_cols<C, EPI>();
  const int tiles_n = (n_hi - n_lo + kCols - 1) / kCols;
  int tm, tn;
  tile_of((int)blockIdx.x, (int)gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = n_lo + tn * kCols;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int fm0 = wm * C::FM, fn0 = wn * C::FN;  // first fragment (of 32 rows/cols) in the tile

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // One K tile from LDS stage `st`: this wave's fragments (32 code bytes +
  // 4 scale bytes per lane each), then 8 k-steps in which the decode of
  // step t+1 overlaps the MFMAs of step t.  `prefetch` runs right after the
  // LDS reads (it issues the next tile's copy into the other stage).
  auto compute_tile = [&](const uint8_t* st, auto prefetch) {
    const uint8_t* sA = st;
    const uint8_t* sB = st + C::kACode;
    const uint8_t* sAs = st + C::kACode + C::kBCode;
    const uint8_t* sBs = sAs + C::kAScale;
    u32x4 ac[C::FM][2], bc[C::FN][2];
    uint32_t as[C::FM], bs[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
      ac[i][0] = *reinterpret_cast<const u32x4*>(sA + (fm0 + i) * 2048 + lane * 16);
      ac[i][1] = *reinterpret_cast<const u32x4*>(sA + (fm0 + i) * 2048 + 1024 + lane * 16);
      as[i] = *reinterpret_cast<const uint32_t*>(sAs + (fm0 + i) * 256 + lane * 4);
    }
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      bc[j][0] = *reinterpret_cast<const u32x4*>(sB + (fn0 + j) * 2048 + lane * 16);
      bc[j][1] = *reinterpret_cast<const u32x4*>(sB + (fn0 + j) * 2048 + 1024 + lane * 16);
      bs[j] = *reinterpret_cast<const uint32_t*>(sBs + (fn0 + j) * 256 + lane * 4);
    }
    prefetch();

    half2v sa2[C::FM], sb2[C::FN];
    half8 a_cur[C::FM], b_cur[C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) sa2[i] = scale_pair(as[i], 0);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) sb2[j] = scale_pair(bs[j], 0);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) a_cur[i] = decode8(ac[i][0][0], sa2[i]);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) b_cur[j] = decode8(bc[j][0][0], sb2[j]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      half8 a_nxt[C::FM], b_nxt[C::FN];
      if (t < 7) {
        const int u = t + 1;
        if ((u & 1) == 0) {  // k-steps 2v and 2v+1 share scale byte v
#pragma unroll
          for (int i = 0; i < C::FM; ++i) sa2[i] = scale_pair(as[i], u >> 1);
#pragma unroll
          for (int j = 0; j < C::FN; ++j) sb2[j] = scale_pair(bs[j], u >> 1);
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a_nxt[i] = decode8(ac[i][u >> 2][u & 3], sa2[i]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b_nxt[j] = decode8(bc[j][u >> 2][u & 3], sb2[j]);
      }
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a_cur[i], b_cur[j], acc[i][j], 0, 0, 0);
      if (t < 7) {
        if constexpr (C::kSchedValu > 0) {
          // interleave: one MFMA, then kSchedValu decode VALU ops, repeated
#pragma unroll
          for (int g = 0; g < C::FM * C::FN; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, C::kSchedValu, 0);   // VALU
          }
        }
#pragma unroll
        for (int i = 0; i < C::FM; ++i) a_cur[i] = a_nxt[i];
#pragma unroll
        for (int j = 0; j < C::FN; ++j) b_cur[j] = b_nxt[j];
      }
    }
  };

  // Three LDS stages: tile kt computes while tiles kt+1 and kt+2 stream in.
  constexpr int kStages = 3;
  constexpr int kPer = AsyncLoader<C, EPI>::kPerTile;
  const int nk_full = p.K / kBK;  // full K tiles: asynchronous LDS-DMA path
  AsyncLoader<C, EPI> ld;
  ld.init(p, m0, n0, n_hi, wave, lane);
  if (nk_full > 0) ld.issue(smem, 0);
  if (nk_full > 1) {
    ld.issue(smem + C::kStage, 1);
    wait_vmem<kPer>();  // tile 0 landed, tile 1 may still fly
  } else {
    wait_vmem<0>();
  }
  barrier_lds();
  for (int kt = 0; kt < nk_full; ++kt) {
    compute_tile(smem + (kt % kStages) * C::kStage, [&] {
      if (kt + 2 < nk_full) ld.issue(smem + ((kt + 2) % kStages) * C::kStage, kt + 2);
    });
    if (kt + 2 < nk_full) wait_vmem<kPer>();  // tile kt+1 landed
    else wait_vmem<0>();
    barrier_lds();
  }
  if (p.K % kBK != 0) {  // partial last K tile through registers, zero-filled beyond K
    uint8_t* st = smem + (nk_full % kStages) * C::kStage;
    TailLoader<C, EPI> tl;
    tl.load(p, m0, n0, n_hi, nk_full);
    tl.store(st);
    barrier_lds();
    compute_tile(st, [] {});
  }

  finish_tile<C, EPI>(p, acc, m0, n0, n_hi, fm0, fn0, wn, lane, smem);
}

// Shapes whose K is a whole number (>= 2) of 128-wide tiles: one wave per
// SIMD (for 256x256 tiles each owning 128x128 outputs: 16 accumulator
// fragments in the accumulation registers, so every decoded fragment feeds
// four MFMAs and a k-step decodes 8 fragments for 16 MFMAs).  One wave per
// SIMD has no second wave to cover its stalls, so the K loop is
// software-pipelined across tiles: the codes of k-steps 4-7 are read from
// LDS during k-step 1, the next tile's k-steps 0-3 and scales during k-step
// 4 (after the workgroup barrier that certifies that tile's copies), and
// k-step 7 decodes the next tile's first k-step.  The barrier of tile kt
// also releases its LDS stage: every wave reaches it after its last read of
// the stage, and copies into that stage (tile kt+3) go out only after it.
template <class C, int EPI>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(C::kPipeOcc, C::kPipeOcc)))
void gemm_kernel_pipe(const GemmArgs p, int n_lo, int n_hi) {
  static_assert(C::kWavesPerSimd == 1, "one wave per SIMD");
  static_assert((C::FM + C::FN) % C::FM == 0, "decode split");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tiles_m = (p.M + C::BM - 1) / C::BM;
  constexpr int kCols = tile_cols<C, EPI>();
  const int tiles_n = (n_hi - n_lo + kCols - 1) / kCols;
  int tm, tn;
  tile_of((int)blockIdx.x, (int)gridDim.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = n_lo + tn * kCols;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WGN, wn = wave % C::WGN;
  const int fm0 = wm * C::FM, fn0 = wn * C::FN;
  constexpr int NF = C::FM + C::FN;  // fragments: A first, then W

  floatx16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // This lane's code chunk (k-steps 0-3; +1024 bytes: 4-7) and scale dword
  // of fragment f in a stage.
  auto code_at = [&](const uint8_t* st, int f, int half) __attribute__((always_inline)) -> u32x4 {
    const int off = f < C::FM ? (fm0 + f) * 2048 : C::kACode + (fn0 + f - C::FM) * 2048;
    return *reinterpret_cast<const u32x4*>(st + off + half * 1024 + lane * 16);
  };
  // Scales: [row][16 B] (A rows, then W rows); this K tile's 8 bytes first.
  auto scale_at = [&](const uint8_t* st, int f) __attribute__((always_inline)) -> uint32_t {
    const int row = (f < C::FM ? (fm0 + f) * 32 : C::BM + (fn0 + f - C::FM) * 32) + (lane & 31);
    return *reinterpret_cast<const uint32_t*>(st + C::kACode + C::kBCode + row * 16 + (lane >> 5) * 4);
  };

  constexpr int kPer = AsyncLoader<C, EPI, true>::kPerTile;
  const int nk = p.K / kBK;  // >= 2, K % 128 == 0 (checked by the launcher)
  AsyncLoader<C, EPI, true> ld;
  ld.init(p, m0, n0, n_hi, wave, lane);
  // A tile's copies go out in two parts: slots [0, kPart1) during k-steps
  // 4-7 of the tile three before it (into the stage that tile has just
  // released), slots [kPart1, kPer) during k-steps 0-3 of the tile two
  // before it, spread one or two per region.  A wave can keep only a few
  // LDS-DMA copies in flight: beyond that, issuing the next one stalls it
  // (measured: issuing three whole tiles back to back took ~12K cycles, and
  // the wait for the first then took none), so no burst is longer than a
  // tile and a half.  Every wave keeps exactly the copies of one tile in
  // flight behind the one it waits for: past the last tile it re-copies the
  // last tile (in bounds) into a stage nobody reads again, so the waits are
  // the same every tile and the K loop has no branches.
  // The prologue copies tiles 0 and 1 only; the first tile sends all of
  // tile 2 in its k-steps 0-3.
  constexpr int kPart1 = (kPer + 1) / 2;
  ld.issue(smem, 0);
  ld.issue(smem + C::kStageWide, 1);
  wait_vmem<kPer>();  // tile 0 landed
  barrier_lds();

  u32x4 c_lo[NF];
  uint32_t sc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    c_lo[f] = code_at(smem, f, 0);
    sc[f] = scale_at(smem, f);
  }
  half2v s2[NF];
  half8 cur[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    s2[f] = scale_pair(sc[f], 0);
    cur[f] = decode8(c_lo[f][0], s2[f]);
  }

  // One K tile; MORE: a next tile follows (its first k-step is decoded here);
  // FIRST: tile 0.
  auto tile = [&](int kt, auto more_tag, auto first_tag) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    const uint8_t* st = smem + (kt % 3) * C::kStageWide;
    u32x4 c_hi[NF], n_lo[NF];
    uint32_t nsc[NF];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t == 1) {
#pragma unroll
        for (int f = 0; f < NF; ++f) c_hi[f] = code_at(st, f, 1);
      }
      if constexpr (MORE) {
        if (t == 4) {
          wait_vmem<kPer>();  // tile kt+1 landed, kt+2 may fly
          barrier_lds();
          // the barrier's lgkmcnt(0) again, visible to the compiler's own
          // wait insertion (it cannot see inside the asm): the codes read
          // before the barrier need no further wait
          __builtin_amdgcn_s_waitcnt(0xC07F);
          const uint8_t* nst = smem + ((kt + 1) % 3) * C::kStageWide;
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            n_lo[f] = code_at(nst, f, 0);
            nsc[f] = scale_at(nst, f);
          }
        }
      }
      // The k-step in FM regions, each scheduled as one unit: region r
      // issues the MFMAs of accumulator row r interleaved with the decode of
      // NF/FM fragments for the next k-step (W fragments first: every MFMA
      // of the next step's first region needs all of them) and its share of
      // the copies of later tiles (at most one or two: see above).
      const bool dec = t < 7 || MORE;
      constexpr int kPerRegion = NF / C::FM;
      half8 nxt[NF];
#pragma unroll
      for (int r = 0; r < C::FM; ++r) {
        if (dec) {
#pragma unroll
          for (int q = 0; q < kPerRegion; ++q) {
            const int e = r * kPerRegion + q;             // decode order
            const int f = e < C::FN ? C::FM + e : e - C::FN;  // W fragments, then A
            if (t < 7) {
              const int u = t + 1;
              if ((u & 1) == 0) s2[f] = scale_pair(sc[f], u >> 1);
              nxt[f] = decode8(u < 4 ? c_lo[f][u] : c_hi[f][u - 4], s2[f]);
            } else {
              s2[f] = scale_pair(nsc[f], 0);
              nxt[f] = decode8(n_lo[f][0], s2[f]);
            }
          }
        }
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
          acc[r][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cur[r], cur[C::FM + j], acc[r][j], 0, 0, 0);
        if (MORE || t < 4) {
          // k-steps 4-7: part 1 of tile kt+3 into this tile's stage; k-steps
          // 0-3: part 2 of tile kt+2 (whose part 1 went out one tile ago),
          // all of tile 2 in the first tile
          const int base = t < 4 && !FIRST ? kPart1 : 0;
          const int size = t < 4 ? (FIRST ? kPer : kPer - kPart1) : kPart1;
          const int per_step = (size + 3) / 4, per_region = (per_step + C::FM - 1) / C::FM;
          const int tgt = t < 4 ? kt + 2 : kt + 3;
#pragma unroll
          for (int q = 0; q < per_region; ++q) {
            const int o = r * per_region + q;  // copy o of this k-step
            const int i = (t & 3) * per_step + o;
            if (o < per_step && i < size)
              ld.issue_slot(smem + (tgt % 3) * C::kStageWide, min(tgt, nk - 1), base + i);
          }
        }
        if (dec) {
          if constexpr (C::kSchedValu > 0) {
#pragma unroll
            for (int g = 0; g < C::FN; ++g) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, C::kSchedValu, 0);  // VALU
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (dec) {
#pragma unroll
        for (int f = 0; f < NF; ++f) cur[f] = nxt[f];
      }
    }
    if constexpr (MORE) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        c_lo[f] = n_lo[f];
        sc[f] = nsc[f];
      }
    }
  };
  tile(0, std::true_type{}, std::true_type{});
  for (int kt = 1; kt + 1 < nk; ++kt) tile(kt, std::true_type{}, std::false_type{});
  tile(nk - 1, std::false_type{}, std::false_type{});
  wait_vmem<0>();  // the re-copies have landed before the epilogue reuses LDS

  finish_tile<C, EPI>(p, acc, m0, n0, n_hi, fm0, fn0, wn, lane, smem);
}

template <class C, int EPI, bool PIPE = false>
hipError_t launch_cfg(const GemmArgs& p, int n_lo, int n_hi, hipStream_t s) {
  const int tiles_m = (p.M + C::BM - 1) / C::BM;
  constexpr int kCols = tile_cols<C, EPI>();
  const int tiles_n = (n_hi - n_lo + kCols - 1) / kCols;
  const int64_t nblocks = (int64_t)tiles_m * tiles_n;
  // three K stages; the bf16 output tile is staged in the same memory afterwards
  const size_t tile = (size_t)C::BM * staged_row_bytes<kCols>();
  const size_t stages = 3 * (size_t)(PIPE ? C::kStageWide : C::kStage);
  const size_t lds = stages > tile ? stages : tile;
  // raising the dynamic-LDS limit is idempotent and cheap
  const void* fn;
  if constexpr (PIPE) fn = (const void*)gemm_kernel_pipe<C, EPI>;
  else fn = (const void*)gemm_kernel<C, EPI>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  if constexpr (PIPE)
    gemm_kernel_pipe<C, EPI><<<(unsigned)nblocks, C::kThreads, lds, s>>>(p, n_lo, n_hi);
  else
    gemm_kernel<C, EPI><<<(unsigned)nblocks, C::kThreads, lds, s>>>(p, n_lo, n_hi);
  return hipGetLastError();
}

// Large prefill shapes with a ragged last K tile: 8 waves, two per SIMD, so
// one wave's decode VALU work runs while the other's MFMAs occupy the
// matrix core.
using CfgL = TileCfg<256, 256, 4, 2, 7>;
using CfgM = TileCfg<128, 128, 2, 2, 0>;  // medium shapes / better wave fill
using CfgS = TileCfg<32, 128, 1, 4, 0>;   // M <= 32
using CfgH = TileCfg<256, 128, 4, 2, 7>;  // the columns past whole waves of CfgL tiles
using CfgP = TileCfg<256, 256, 2, 2, 4>;  // CfgL's tiles, one wave per SIMD (gemm_kernel_pipe)
using CfgQ = TileCfg<256, 128, 4, 1, 6>;  // CfgH's tiles, one wave per SIMD (gemm_kernel_pipe)
using CfgR = TileCfg<128, 128, 2, 2, 8>;  // CfgM's tiles (gemm_kernel_pipe, two workgroups per CU)

// 256x256 tiles: the pipelined one-wave-per-SIMD kernel when K is a whole
// number (>= 2) of K tiles, else the two-wave kernel with its tail path.
template <int EPI>
hipError_t launch_large(const GemmArgs& p, int n_lo, int n_hi, hipStream_t s) {
  if (p.K % kBK == 0 && p.K >= 2 * kBK) return launch_cfg<CfgP, EPI, true>(p, n_lo, n_hi, s);
  return launch_cfg<CfgL, EPI>(p, n_lo, n_hi, s);
}
// 256x128 tiles, likewise.
hipError_t launch_half(const GemmArgs& p, int n_lo, int n_hi, hipStream_t s) {
  if (p.K % kBK == 0 && p.K >= 2 * kBK) return launch_cfg<CfgQ, kEpiPlain, true>(p, n_lo, n_hi, s);
  return launch_cfg<CfgH, kEpiPlain>(p, n_lo, n_hi, s);
}
// 128x128 tiles, likewise.
template <int EPI>
hipError_t launch_medium(const GemmArgs& p, int n_lo, int n_hi, hipStream_t s) {
  if (p.K % kBK == 0 && p.K >= 2 * kBK) return launch_cfg<CfgR, EPI, true>(p, n_lo, n_hi, s);
  return launch_cfg<CfgM, EPI>(p, n_lo, n_hi, s);
}

double fill(int64_t tiles) {
  const int64_t waves = (tiles + 255) / 256;
  return (double)tiles / (double)(waves * 256);
}

hipError_t launch_range(const GemmArgs& p, int n_lo, int n_hi, bool gate, hipStream_t s) {
  const int n = n_hi - n_lo;
  if (skinny_eligible(p)) return launch_gemm_skinny(p, n_lo, n_hi, gate, s);
  if (gate) {
    if (p.M <= 32) return launch_cfg<CfgS, kEpiGate>(p, n_lo, n_hi, s);
    return launch_medium<kEpiGate>(p, n_lo, n_hi, s);
  }
  if (p.M <= 32) return launch_cfg<CfgS, kEpiPlain>(p, n_lo, n_hi, s);
  const int64_t tl = (int64_t)((p.M + 255) / 256) * ((n + 255) / 256);
  const int64_t tmd = (int64_t)((p.M + 127) / 128) * ((n + 127) / 128);
  const bool pipe = p.K % kBK == 0 && p.K >= 2 * kBK;
  const bool large = p.M >= 256 && n >= 256 && fill(tl) >= 0.8 * fill(tmd);
  if (p.M >= 256 && n >= 256 && (large || pipe) && fill(tl) < 0.9) {
    // A partly filled last wave of 256x256 tiles: keep whole waves of them
    // on the leading columns and cover the rest in a second launch with
    // 256x128 tiles, or with 128x128 tiles when those fill the last wave
    // and 256x128 ones would not (a wave of smaller work instead of a
    // half-empty wave; every output column still sees its whole K in the
    // same order, so the outputs are bit-identical).
    const int64_t tm = (p.M + 255) / 256, tm128 = (p.M + 127) / 128;
    for (int k = n / 256; k > 0; --k) {
      if ((tm * k) % 256 != 0) continue;
      const int rest = n - 256 * k;
      if (rest <= 0) continue;
      const bool half = fill(tm * ((rest + 127) / 128)) >= 0.9;
      const bool quarter = pipe && fill(tm128 * ((rest + 127) / 128)) >= 0.9;
      if (!half && !quarter) continue;
      const hipError_t e = launch_large<kEpiPlain>(p, n_lo, n_lo + 256 * k, s);
      if (e != hipSuccess) return e;
      if (half) return launch_half(p, n_lo + 256 * k, n_hi, s);
      return launch_medium<kEpiPlain>(p, n_lo + 256 * k, n_hi, s);
    }
  }
  if (large) return launch_large<kEpiPlain>(p, n_lo, n_hi, s);
  return launch_medium<kEpiPlain>(p, n_lo, n_hi, s);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& p, hipStream_t s) {
  // Split the columns into maximal runs that are all gate columns or all
  // gate-free, and launch each run with the matching instantiation.
  int cuts[2 * NVFP4_MAX_SEGMENTS + 2];
  int ncut = 0;
  cuts[ncut++] = 0;
  for (int g = 0; g < 2; ++g) {
    const int seg = g == 0 ? p.ep.b_seg : p.ep.a_seg;
    if (seg < 0) continue;
    cuts[ncut++] = p.ep.seg_off[seg];
    cuts[ncut++] = p.ep.seg_off[seg + 1];
  }
  cuts[ncut++] = p.N;
  for (int i = 1; i < ncut; ++i)  // insertion sort of <= 6 cut points
    for (int j = i; j > 0 && cuts[j] < cuts[j - 1]; --j) {
      const int t = cuts[j];
      cuts[j] = cuts[j - 1];
      cuts[j - 1] = t;
    }
  auto gated = [&](int col) {
    for (int g = 0; g < 2; ++g) {
      const int seg = g == 0 ? p.ep.b_seg : p.ep.a_seg;
      if (seg >= 0 && col >= p.ep.seg_off[seg] && col < p.ep.seg_off[seg + 1]) return true;
    }
    return false;
  };
  int lo = 0;
  while (lo < p.N) {
    const bool g = gated(lo);
    int hi = p.N;
    for (int i = 0; i < ncut; ++i)  // next cut where the gate state may change
      if (cuts[i] > lo && gated(cuts[i] < p.N ? cuts[i] : p.N - 1) != g) {
        hi = cuts[i];
        break;
      }
    const hipError_t e = launch_range(p, lo, hi, g, s);
    if (e != hipSuccess) return e;
    lo = hi;
  }
  return hipSuccess;
}

hipError_t launch_gemm_swiglu(const GemmArgs& p, hipStream_t s) {
  if (p.ep.partials != nullptr) {
    const hipError_t e = launch_zero(p.ep.partials, p.ep.n_partials, s);
    if (e != hipSuccess) return e;
  }
  const int inter = p.ep.inter;
  const int64_t tl = (int64_t)((p.M + 255) / 256) * ((inter + 127) / 128);
  const int64_t tmd = (int64_t)((p.M + 127) / 128) * ((inter + 63) / 64);
  if (p.M >= 256 && inter >= 128 && fill(tl) >= 0.8 * fill(tmd))
    return launch_large<kEpiSwiglu>(p, 0, inter, s);
  return launch_medium<kEpiSwiglu>(p, 0, inter, s);
}

}  // namespace nvfp4
