// W4A4 NVFP4 GEMM for decode (M <= 16 tokens against a whole weight) on a
// weight repacked offline into the order the kernel consumes it, and the
// same GEMM with the activations quantized inside the launch.
//
// Same mathematics as the tiled kernels (exact E2M1 x E4M3 -> fp16 decode,
// fp32 MFMA accumulation, per-segment global scales and the GDN gates in the
// epilogue; format: evolve.pub review of arXiv 2609.04098, "Scope & Claims";
// segments keep their own scales: chatpaper.ai English abstract).  Decode is
// bound by streaming the weight from HBM once, so the weight is laid out for
// that stream: every load instruction of a wave reads 1 KB of contiguous
// bytes that land in the lanes exactly as the MFMA wants them (no LDS
// staging, no shuffles).  The row-major layout puts the 16 rows an MFMA
// operand spans in 16 places, which costs the vector memory path far more
// than the bytes themselves.
//
// Packed layout (nvfp4_decode_weight_pack), for a weight [N, K]:
//   Q = ceil(K / 1024) chunks of 32 elements per lane; the weight is cut
//   into units (g, w): 16 rows g*16 .. g*16+15 (a "group") times the K
//   slice w*128Q .. (w+1)*128Q (w < 8, one per wave of a workgroup).
//   Unit (g, w) starts at byte (g*8 + w) * Q*1152:
//     codes  [qi < Q][lane < 64][16 B]: lane (r = lane%16, h = lane/16)
//            holds the 32 codes of row g*16+r at k = w*128Q + 128qi + 32h
//            + (0..31), two per byte, even element in the low nibble;
//     scales the two E4M3 block scales of each (lane, chunk): chunks in
//            quads [j][lane][8 B] (chunk 4j+c at bytes 2c, 2c+1), then a
//            pair [lane][4 B] when Q % 4 >= 2, then [lane][2 B] when Q is
//            odd.
//   Rows beyond N and elements beyond K are zero codes with zero scales,
//   which decode to 0.
// An MFMA sums over its 32 k values, so any permutation of k that the
// activations share is allowed: lane (r, h) of wave w feeds, at chunk qi and
// MFMA step t, k = w*128Q + 128qi + 32h + 8t + e (e < 8) for both operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

using namespace dev;
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kSlices = 8;  // K slices of a 16-row group (units of the packed layout)
// groups per round: one 16x16 partial each in LDS (fewer for wide K slices,
// whose activations take more registers), a whole number of D-unit steps
template <int Q, int D>
constexpr int round_of() { return (Q >= 6 ? 8 : 16) / D * D; }

__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One unit's operands of this lane: Q code chunks and their scale bytes
// (sc[i] holds chunks 2i and 2i+1, two bytes each).
template <int Q>
struct Unit {
  u32x4 c[Q];
  uint32_t sc[(Q + 1) / 2];
};

// Load unit (g, wave) from the packed weight; `valid` false loads nothing
// from memory (a buffer of zero records returns zeros).
// A lane with `mine` false reads zeros without touching memory (its offsets
// are pushed past the buffer's end).
template <int Q>
__device__ __attribute__((always_inline)) inline void load_unit(Unit<Q>& u, const uint8_t* packed, int64_t g,
                                                                int slice, int lane, bool valid, bool mine) {
  constexpr int kUnit = Q * 1152;
  const uint8_t* base = packed + (g * kSlices + slice) * (int64_t)kUnit;
  const __amdgpu_buffer_rsrc_t r = rsrc_of(base, valid ? (uint32_t)kUnit : 0u);
  const int off_lane = mine ? 0 : 0x40000000;
#pragma unroll
  for (int qi = 0; qi < Q; ++qi)
    u.c[qi] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off_lane + lane * 16, qi * 1024, 0));
  int off = Q * 1024;
#pragma unroll
  for (int j = 0; j < Q / 4; ++j) {
    const uint64_t v =
        __builtin_bit_cast(uint64_t, __builtin_amdgcn_raw_buffer_load_b64(r, off_lane + lane * 8, off, 0));
    u.sc[2 * j] = (uint32_t)v;
    u.sc[2 * j + 1] = (uint32_t)(v >> 32);
    off += 512;
  }
  if constexpr (Q % 4 >= 2) {
    u.sc[2 * (Q / 4)] = __builtin_amdgcn_raw_buffer_load_b32(r, off_lane + lane * 4, off, 0);
    off += 256;
  }
  if constexpr (Q % 2 == 1) u.sc[(Q - 1) / 2] = __builtin_amdgcn_raw_buffer_load_b16(r, off_lane + lane * 2, off, 0);
}

// Scale pair for MFMA step t of chunk qi (steps 0-1: the chunk's first block).
template <int Q>
__device__ inline half2v unit_scale(const uint32_t (&sc)[(Q + 1) / 2], int qi, int t) {
  return scale_pair(sc[qi >> 1], 2 * (qi & 1) + (t >> 1));
}

struct DecodeArgs {
  // activations: pre-quantized NVFP4 (a_codes != null) or dense x quantized here
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  int64_t lda_c, lda_s;
  const float* a_g;
  const void* x;
  int x_dtype;
  int64_t ld_x;
  float* x_g_out;  // the dynamic global scale of x, or null
  const uint8_t* packed;
  void* out;
  int64_t ld_out;
  int out_bf16;
  int M, N, K;
  EpilogueArgs ep;
};

// Row stride (bytes) of the activation codes / scales staged in LDS by the
// in-launch quantization (16-byte rows, plus 16 bytes that move rows off
// each other's banks).
__host__ __device__ constexpr int lds_code_stride(int K) { return ((K / 2 + 15) / 16) * 16 + 16; }
__host__ __device__ constexpr int lds_scale_stride(int K) { return K / 16 + 16; }

// Activations of the kernel: 0 = pre-quantized NVFP4, 1 = bf16 x quantized
// in the launch, 2 = float32 x quantized in the launch.
template <int XQ, int S>
struct XBlocks {
  static constexpr int kChunks = XQ == 2 ? 4 : 2;  // 16-byte chunks per 16-element block
  static constexpr int kRegs = 5 * S;  // blocks per thread kept in registers (2560 blocks per workgroup)
};

// 16 elements of x block b (row-major blocks of [M, K]) as floats.
template <int XQ>
__device__ inline const uint8_t* x_block_ptr(const DecodeArgs& p, int b, int bpr) {
  const int m = b / bpr, j = b - m * bpr;
  constexpr int esz = XQ == 2 ? 4 : 2;
  return reinterpret_cast<const uint8_t*>(p.x) + ((int64_t)m * p.ld_x + (int64_t)j * 16) * esz;
}
template <int XQ>
__device__ inline void x_block_load(const uint8_t* src, uint4 (&c)[XBlocks<XQ, 1>::kChunks]) {
#pragma unroll
  for (int i = 0; i < XBlocks<XQ, 1>::kChunks; ++i) c[i] = reinterpret_cast<const uint4*>(src)[i];
}
template <int XQ>
__device__ inline void x_block_values(const uint4 (&c)[XBlocks<XQ, 1>::kChunks], float v[16]) {
#pragma unroll
  for (int i = 0; i < XBlocks<XQ, 1>::kChunks; ++i) {
    const uint32_t w[4] = {c[i].x, c[i].y, c[i].z, c[i].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (XQ == 2) {
        v[4 * i + e] = __uint_as_float(w[e]);
      } else {
        v[8 * i + 2 * e] = __uint_as_float(w[e] << 16);
        v[8 * i + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
      }
    }
  }
}

// S K slices per wave: 8 / S waves per workgroup (S = 2: one wave per SIMD
// with twice the registers, which also drops the issue-priority skew between
// two waves sharing a SIMD).
template <int Q, int D, bool GATE, int XQ, int S>
__global__ __launch_bounds__(kSlices / S * 64) __attribute__((amdgpu_waves_per_eu(S == 1 ? 2 : 1, S == 1 ? 2 : 1)))
void decode_kernel(const DecodeArgs p, int groups) {
  constexpr int NW = kSlices / S, NT = NW * 64;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  // This workgroup's share: an equal run of half-groups (8 rows), so every
  // workgroup streams the same number of bytes; a run may begin with the
  // upper half of a group and end with the lower half of one.  Local index
  // j -> group g_first + j, n_mine groups.
  const int64_t halves = 2 * (int64_t)groups;
  const int h0 = (int)(((int64_t)blockIdx.x * halves) / gridDim.x);
  const int h1 = (int)(((int64_t)(blockIdx.x + 1) * halves) / gridDim.x);
  const int g_first = h0 >> 1, g_last = (h1 - 1) >> 1;
  const int n_mine = g_last - g_first + 1;
  auto group_of = [&](int j) { return g_first + j; };
  // rows of local group j this workgroup owns: lanes outside load nothing
  // and store nothing
  auto owns_row = [&](int j, int r) {
    const int g = g_first + j;
    return !((g == g_first && (h0 & 1) && r < 8) || (g == g_last && (h1 & 1) && r >= 8));
  };
  const bool live = r16 < p.M;

  // --- activations, loaded before the weight so that waiting for them
  // never waits for weight loads (loads complete in issue order)
  u32x4 a_c[S][Q];
  uint32_t a_s[S][Q];
  using XB = XBlocks<XQ == 0 ? 1 : XQ, S>;
  uint4 xr[XQ == 0 ? 1 : XB::kRegs][XB::kChunks];
  const int bpr = p.K >> 4;
  const int nblk = p.M * bpr;
  if constexpr (XQ == 0) {
    // pre-quantized: this wave's K slices of the M rows straight from memory
    const uint8_t* crow = p.a_codes + (int64_t)(live ? r16 : 0) * p.lda_c;
    const uint8_t* srow = p.a_scales + (int64_t)(live ? r16 : 0) * p.lda_s;
#pragma unroll
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
      for (int qi = 0; qi < Q; ++qi) {
        const int k0 = (wave * S + sl) * 128 * Q + 128 * qi + 32 * h;
        const bool in = live && k0 < p.K;
        a_c[sl][qi] = *reinterpret_cast<const u32x4*>(crow + (in ? (k0 >> 1) : 0));
        a_s[sl][qi] = *reinterpret_cast<const uint16_t*>(srow + (in ? (k0 >> 4) : 0));
        if (!in) {
          a_c[sl][qi] = u32x4{0u, 0u, 0u, 0u};
          a_s[sl][qi] = 0u;
        } else if (k0 + 32 > p.K) {  // 16 valid elements: the first block only
          a_c[sl][qi][2] = 0u;
          a_c[sl][qi][3] = 0u;
          a_s[sl][qi] &= 0xFFu;
        }
      }
  } else {
    // dense x: the first XB::kRegs blocks of this thread into registers
#pragma unroll
    for (int i = 0; i < XB::kRegs; ++i) {
      const int b = (int)threadIdx.x + i * NT;
      x_block_load<XQ>(x_block_ptr<XQ>(p, b < nblk ? b : 0, bpr), xr[i]);
    }
  }

  // --- the weight stream starts: units of the first D groups in flight
  Unit<Q> buf[D][S];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int sl = 0; sl < S; ++sl)
      load_unit<Q>(buf[d][sl], p.packed, group_of(d), wave * S + sl, lane, d < n_mine, owns_row(d, r16));

  float ga;
  if constexpr (XQ != 0) {
    // Dynamic NVFP4 quantization of x [M, K] inside the launch: every
    // workgroup takes the amax of all of x (a few tens of KB from L2), forms
    // g = fl32(amax / (6 * 448)) and quantizes all M x K/16 blocks with the
    // quantizer's own block routine into LDS (row-major codes and scales):
    // bit for bit what nvfp4_quantize writes.  Blocks past the register
    // cache (large M x K only) are loaded again where they are needed.
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < XB::kRegs; ++i) {
      if ((int)threadIdx.x + i * NT < nblk) {
        float v[16];
        x_block_values<XQ>(xr[i], v);
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
      }
    }
    for (int b = (int)threadIdx.x + XB::kRegs * NT; b < nblk; b += NT) {
      uint4 c[XB::kChunks];
      float v[16];
      x_block_load<XQ>(x_block_ptr<XQ>(p, b, bpr), c);
      x_block_values<XQ>(c, v);
#pragma unroll
      for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(v[e]));
    }
    m = wave_max(m);
    float* red = reinterpret_cast<float*>(smem);
    if (lane == 0) red[wave] = m;
    barrier_lds();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    float amax = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) amax = fmaxf(amax, red[i]);
    ga = (float)((double)amax / 2688.0);  // one correctly rounded division (53 >= 2*24+2)
    if (p.x_g_out != nullptr && blockIdx.x == 0 && threadIdx.x == 0) *p.x_g_out = ga;
    barrier_lds();  // everyone has read red[] before the codes overwrite it
    uint8_t* lc = smem;
    uint8_t* ls = smem + p.M * lds_code_stride(p.K);
    auto quant_store = [&](int b, const float (&v)[16]) __attribute__((always_inline)) {
      uint2 c;
      const uint32_t sc = quantize_block16(v, ga, &c);
      const int mm = b / bpr, j = b - mm * bpr;
      *reinterpret_cast<uint2*>(lc + mm * lds_code_stride(p.K) + j * 8) = c;
      ls[mm * lds_scale_stride(p.K) + j] = (uint8_t)sc;
    };
#pragma unroll
    for (int i = 0; i < XB::kRegs; ++i) {
      const int b = (int)threadIdx.x + i * NT;
      if (b < nblk) {
        float v[16];
        x_block_values<XQ>(xr[i], v);
        quant_store(b, v);
      }
    }
    for (int b = (int)threadIdx.x + XB::kRegs * NT; b < nblk; b += NT) {
      uint4 c[XB::kChunks];
      float v[16];
      x_block_load<XQ>(x_block_ptr<XQ>(p, b, bpr), c);
      x_block_values<XQ>(c, v);
      quant_store(b, v);
    }
    barrier_lds();
    __builtin_amdgcn_s_waitcnt(0xC07F);
#pragma unroll
    for (int sl = 0; sl < S; ++sl)
#pragma unroll
      for (int qi = 0; qi < Q; ++qi) {
        const int k0 = (wave * S + sl) * 128 * Q + 128 * qi + 32 * h;
        const bool in = live && k0 < p.K;
        const int row = live ? r16 : 0, kk = in ? k0 : 0;
        a_c[sl][qi] = *reinterpret_cast<const u32x4*>(lc + row * lds_code_stride(p.K) + (kk >> 1));
        a_s[sl][qi] = *reinterpret_cast<const uint16_t*>(ls + row * lds_scale_stride(p.K) + (kk >> 4));
        if (!in) {
          a_c[sl][qi] = u32x4{0u, 0u, 0u, 0u};
          a_s[sl][qi] = 0u;
        } else if (k0 + 32 > p.K) {  // 16 valid elements: the first block only
          a_c[sl][qi][2] = 0u;
          a_c[sl][qi][3] = 0u;
          a_s[sl][qi] &= 0xFFu;
        }
      }
  } else {
    ga = *p.a_g;
  }

  half8 areg[S][Q][4];
#pragma unroll
  for (int sl = 0; sl < S; ++sl)
#pragma unroll
    for (int qi = 0; qi < Q; ++qi)
#pragma unroll
      for (int t = 0; t < 4; ++t) areg[sl][qi][t] = decode8(a_c[sl][qi][t], scale_pair(a_s[sl][qi], t >> 1));

  // --- the group loop: D units in flight per wave, rounds of <= kRound
  // groups.  The loop body has no branch between a unit's loads and their
  // use (an invalid group loads nothing and writes its partial to a spare
  // LDS slot), so the waits stay exact: each step waits only for the unit
  // it computes, the next D - 1 units stay in flight.
  constexpr int kRound = round_of<Q, D>();
  static_assert(kRound % D == 0, "every round starts on buffer 0");
  floatx4* red = reinterpret_cast<floatx4*>(smem);  // [kRound + 1][8 waves][64 lanes]
  barrier_lds();  // every wave has read its activations from the LDS staging
  for (int r0 = 0; r0 < n_mine; r0 += kRound) {
    const int ng = min(kRound, n_mine - r0);
    for (int j = 0; j < ng; j += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int jj = j + d;
        floatx4 a4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < S; ++sl)
#pragma unroll
          for (int qi = 0; qi < Q; ++qi)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  areg[sl][qi][t], decode8(buf[d][sl].c[qi][t], unit_scale<Q>(buf[d][sl].sc, qi, t)), a4, 0, 0, 0);
        red[((jj < ng ? jj : kRound) * NW + wave) * 64 + lane] = a4;
        // the buffer's next unit goes out right after its last use (the
        // scheduler would otherwise gather the D computations ahead of all
        // D reloads, leaving nothing in flight at the top of the loop)
        __builtin_amdgcn_sched_barrier(0);
        const int jn = r0 + jj + D;  // the local group this buffer takes next
#pragma unroll
        for (int sl = 0; sl < S; ++sl)
          load_unit<Q>(buf[d][sl], p.packed, group_of(jn), wave * S + sl, lane, jn < n_mine, owns_row(jn, r16));
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    barrier_lds();  // every wave's partials of the round are in LDS
    __builtin_amdgcn_s_waitcnt(0xC07F);
    for (int j = wave; j < ng; j += NW) {
      floatx4 sum = red[(j * NW) * 64 + lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) sum += red[(j * NW + w) * 64 + lane];
      // D[i][j] of the 16x16 MFMA: column = lane % 16, rows 4 * (lane / 16) + r
      const int n = group_of(r0 + j) * 16 + r16;
      if (n < p.N && owns_row(r0 + j, r16)) {
        int seg = 0;
        for (int s = 1; s < p.ep.n_seg; ++s) seg += (n >= p.ep.seg_off[s]) ? 1 : 0;
        const float sc = ga * p.ep.seg_g[seg];
        int kind = 0;
        float ealog = 0.0f, dtb = 0.0f;
        if constexpr (GATE) {
          kind = (seg == p.ep.b_seg) ? 1 : (seg == p.ep.a_seg ? 2 : 0);
          if (kind == 2) {
            const int hh = n - p.ep.seg_off[seg];
            ealog = expf(p.ep.A_log[hh]);
            dtb = p.ep.dt_bias[hh];
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 4 * h + r;
          if (m < p.M) {
            float v = sum[r] * sc;
            if constexpr (GATE) v = gate_value(v, kind, ealog, dtb);
            if (p.out_bf16)
              reinterpret_cast<uint16_t*>(p.out)[(int64_t)m * p.ld_out + n] = (uint16_t)f32_to_bf16_bits(v);
            else
              reinterpret_cast<float*>(p.out)[(int64_t)m * p.ld_out + n] = v;
          }
        }
      }
    }
    barrier_lds();  // the next round's partials reuse this LDS
  }
  wait_vmem<0>();  // the look-ahead loads past the last group (zero records) have returned
}

// Packing: one thread per (unit, lane) writes its Q code chunks and scale bytes.
template <int Q>
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int64_t ldc,
                                                   const uint8_t* __restrict__ scales, int64_t lds, int N, int K,
                                                   uint8_t* __restrict__ out, int64_t units) {
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= units * 64) return;
  const int64_t unit = id >> 6;
  const int lane = (int)(id & 63), r = lane & 15, h = lane >> 4;
  const int64_t g = unit / kSlices;
  const int w = (int)(unit % kSlices);
  const int64_t n = g * 16 + r;
  uint8_t* base = out + unit * (int64_t)(Q * 1152);
  uint8_t sb[2 * Q];
#pragma unroll
  for (int qi = 0; qi < Q; ++qi) {
    const int k0 = w * 128 * Q + 128 * qi + 32 * h;
    uint32_t c[4] = {0u, 0u, 0u, 0u};
    uint8_t s0 = 0, s1 = 0;
    if (n < N && k0 < K) {
      const uint8_t* crow = codes + n * ldc + k0 / 2;
      const uint8_t* srow = scales + n * lds + k0 / 16;
      const int nb = K - k0 >= 32 ? 16 : 8;  // code bytes present (K % 16 == 0)
      for (int b = 0; b < nb; ++b) c[b >> 2] |= (uint32_t)crow[b] << (8 * (b & 3));
      s0 = srow[0];
      if (nb == 16) s1 = srow[1];
    }
    *reinterpret_cast<uint4*>(base + qi * 1024 + lane * 16) = make_uint4(c[0], c[1], c[2], c[3]);
    sb[2 * qi] = s0;
    sb[2 * qi + 1] = s1;
  }
  int off = Q * 1024, qi = 0;
  for (int j = 0; j < Q / 4; ++j, qi += 4, off += 512)
    for (int b = 0; b < 8; ++b) base[off + lane * 8 + b] = sb[2 * qi + b];
  if (Q % 4 >= 2) {
    for (int b = 0; b < 4; ++b) base[off + lane * 4 + b] = sb[2 * qi + b];
    qi += 2;
    off += 256;
  }
  if (Q % 2 == 1)
    for (int b = 0; b < 2; ++b) base[off + lane * 2 + b] = sb[2 * qi + b];
}

template <int Q, int D, int S>
hipError_t launch_q(const DecodeArgs& p, bool gate, hipStream_t s) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) cus = 256;
  const int groups = (p.N + 15) / 16;
  const int grid = groups < cus ? groups : cus;
  const int xq = p.x == nullptr ? 0 : (p.x_dtype == NVFP4_DTYPE_BF16 ? 1 : 2);
  constexpr int NW = kSlices / S;
  size_t lds = (size_t)(round_of<Q, D>() + 1) * NW * 64 * 16;
  if (xq != 0) {
    const size_t a = (size_t)p.M * (lds_code_stride(p.K) + lds_scale_stride(p.K));
    if (a > lds) lds = a;
  }
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e2 = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e2 != hipSuccess) return e2;
    kern<<<grid, NW * 64, lds, s>>>(p, groups);
    return hipGetLastError();
  };
  if (gate) {
    if (xq == 1) return go(decode_kernel<Q, D, true, 1, S>);
    if (xq == 2) return go(decode_kernel<Q, D, true, 2, S>);
    return go(decode_kernel<Q, D, true, 0, S>);
  }
  if (xq == 1) return go(decode_kernel<Q, D, false, 1, S>);
  if (xq == 2) return go(decode_kernel<Q, D, false, 2, S>);
  return go(decode_kernel<Q, D, false, 0, S>);
}

}  // namespace

int64_t decode_pack_chunks(int64_t K) { return (K + 1023) / 1024; }

size_t decode_weight_bytes(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * kSlices * (size_t)decode_pack_chunks(K) * 1152;
}

hipError_t launch_decode_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int N, int K,
                              uint8_t* out, hipStream_t s) {
  const int Q = (int)decode_pack_chunks(K);
  const int64_t units = (int64_t)((N + 15) / 16) * kSlices;
  const int64_t threads = units * 64;
  const unsigned grid = (unsigned)((threads + 255) / 256);
  switch (Q) {
    case 1: pack_kernel<1><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 2: pack_kernel<2><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 3: pack_kernel<3><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 4: pack_kernel<4><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 5: pack_kernel<5><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 6: pack_kernel<6><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 7: pack_kernel<7><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    case 8: pack_kernel<8><<<grid, 256, 0, s>>>(codes, ldc, scales, lds, N, K, out, units); break;
    default: return hipErrorInvalidValue;  // the caller checks K <= kDecodeMaxK
  }
  return hipGetLastError();
}

hipError_t launch_gemm_decode(const GemmArgs& g, const uint8_t* packed, const void* x, int x_dtype, int64_t ld_x,
                              float* x_g_out, bool gate, hipStream_t s) {
  DecodeArgs p{};
  p.a_codes = g.a_codes;
  p.a_scales = g.a_scales;
  p.lda_c = g.lda_c;
  p.lda_s = g.lda_s;
  p.a_g = g.ep.a_g;
  p.x = x;
  p.x_dtype = x_dtype;
  p.ld_x = ld_x;
  p.x_g_out = x_g_out;
  p.packed = packed;
  p.out = g.out;
  p.ld_out = g.ld_out;
  p.out_bf16 = g.out_bf16;
  p.M = g.M;
  p.N = g.N;
  p.K = g.K;
  p.ep = g.ep;
  switch (decode_pack_chunks(g.K)) {
    case 1: return launch_q<1, 4, 1>(p, gate, s);
    case 2: return launch_q<2, 4, 1>(p, gate, s);
    case 3: return launch_q<3, 2, 1>(p, gate, s);
    case 4: return launch_q<4, 2, 1>(p, gate, s);
    case 5: return launch_q<5, 3, 1>(p, gate, s);  // K = 5120: three units in flight (2: 0.7-1.3 us slower, 4: slower)
    case 6: return launch_q<6, 2, 1>(p, gate, s);
    case 7: return launch_q<7, 2, 1>(p, gate, s);
    case 8: return launch_q<8, 1, 1>(p, gate, s);
    default: return hipErrorInvalidValue;  // the caller checks K <= kDecodeMaxK
  }
}

}  // namespace nvfp4
