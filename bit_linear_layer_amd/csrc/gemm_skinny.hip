// W4A4 NVFP4 GEMM for small M (decode: a few tokens against a whole
// weight), bound by streaming the weight's codes and scales from HBM.
//
// Same mathematics as the tiled kernel (exact E2M1 x E4M3 -> fp16 decode,
// fp32 MFMA accumulation, per-segment global scales and the GDN gates in the
// epilogue), different shape of work:
//   - one workgroup per CU, 8 waves, owning a contiguous share of 16-column
//     groups of the weight; the waves split K into slices;
//   - each wave decodes its K slice of the M <= 16 activation rows once into
//     registers;
//   - each wave streams ITS slice of every group (16 rows x QPW*64 code bytes
//     + QPW*8 scale bytes) global -> its own LDS stages with LDS-DMA copies
//     (runs of contiguous bytes per row), three groups in flight, with no
//     barrier: a stage is copied to registers before its next copy is
//     issued.  MFMA operand layouts put 16 rows in consecutive lanes, so
//     plain loads into registers scatter every instruction over dozens of
//     cache lines (measured: the vector L1 stalls at ~5 B/cycle/CU);
//   - reads in MFMA order are conflict-free (16-byte pieces XOR-swizzled by
//     row); decode + v_mfma_f32_16x16x32_f16 accumulate one 16x16 partial
//     per group in registers; once per round of <= 16 groups the 8 partial
//     tiles are summed through LDS and the epilogue stores the M valid rows.
// K order: lane (row r, h = lane/16) of wave w feeds, at chunk qi and MFMA
// step t, k = w*128*QPW + h*32*QPW + 32*qi + 8t + e (e < 8), for A and W alike.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"

namespace nvfp4 {

namespace {

using namespace dev;
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kStages = 3;

// Per-lane valid elements of the 32-element chunk at k0: 32, 16 or 0.
__device__ inline int chunk_valid(int k0, int K) { return max(0, min(32, K - k0)); }
// zero what lies beyond K: 16 valid elements keep code dwords 0-1 and scale byte 0
__device__ inline void mask_chunk(u32x4& c, uint32_t& sc, int valid) {
  const uint32_t hi = valid >= 32 ? 0xFFFFFFFFu : 0u, lo = valid > 0 ? 0xFFFFFFFFu : 0u;
  c[0] &= lo; c[1] &= lo; c[2] &= hi; c[3] &= hi;
  sc &= valid >= 32 ? 0xFFFFu : (valid > 0 ? 0xFFu : 0u);
}

// Per-wave LDS stage for one group: codes [16 rows][4*QPW pieces of 16 B],
// piece q of row r at slot r*4QPW + (q ^ ((r >> kSh) & (kG-1))), then the
// scales [16 rows][2*QPW dwords] (padded to 256-byte DMA copies).  kG is the
// power of two (<= 16) dividing 4*QPW: XOR stays inside aligned kG-piece
// groups, and the 16 lanes reading one piece of 16 rows hit 16 distinct
// 16-byte bank groups.
template <int QPW>
struct SkLayout {
  static constexpr int kPieces = 4 * QPW;                               // 16 B pieces per row
  static constexpr int kG = (kPieces % 16 == 0) ? 16 : (kPieces % 8 == 0) ? 8 : 4;
  static constexpr int kSh = kG == 16 ? 0 : (kG == 8 ? 1 : 2);
  static constexpr int kCodeDma = QPW;                                  // 64-lane x 16 B copies
  static constexpr int kScaleDma = (QPW + 1) / 2;                       // 64-lane x 4 B copies
  static constexpr int kDma = kCodeDma + kScaleDma;
  static constexpr int kCodeBytes = 16 * kPieces * 16;
  static constexpr int kStage = kCodeBytes + kScaleDma * 256;
  __device__ static int slot(int r, int q) { return r * kPieces + (q ^ ((r >> kSh) & (kG - 1))); }
};

constexpr int kRound = 16;  // groups per round (one 16x16 partial each in registers)

template <int QPW, bool GATE, bool FULL>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void skinny_kernel(const GemmArgs p, int n_lo, int n_hi, int groups_per_block) {
  using L = SkLayout<QPW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, h = lane >> 4;
  const int kw = wave * QPW * 128;   // this wave's K slice start
  const int kh = kw + h * QPW * 32;  // this lane's contiguous QPW*32 elements
  const int ldc = (int)p.ldw_c, lds_ = (int)p.ldw_s;
  int valid[QPW];
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) valid[qi] = FULL ? 32 : chunk_valid(kh + 32 * qi, p.K);

  // This lane's part of every copy (offsets relative to the group's first row).
  const i32x4 rc = buffer_rsrc(p.w_codes, (uint32_t)((int64_t)p.N * p.ldw_c));
  const i32x4 rs = buffer_rsrc(p.w_scales, (uint32_t)((int64_t)p.N * p.ldw_s));
  int cvoff[L::kCodeDma], svoff[L::kScaleDma];
#pragma unroll
  for (int i = 0; i < L::kCodeDma; ++i) {
    const int S = 64 * i + lane, r = S / L::kPieces, qs = S % L::kPieces;
    const int q = qs ^ ((r >> L::kSh) & (L::kG - 1));
    const int byte = (kw >> 1) + 16 * q;
    cvoff[i] = r * ldc + (byte < ldc ? byte : 0);  // beyond the row: any valid bytes (masked)
  }
#pragma unroll
  for (int i = 0; i < L::kScaleDma; ++i) {
    const int S = 64 * i + lane, r = S / (2 * QPW), d = S % (2 * QPW);
    const int byte = (kw >> 4) + 4 * d;
    svoff[i] = r < 16 && byte < lds_ ? r * lds_ + byte : 0;  // padding lanes: any valid bytes
  }
  uint8_t* mine = smem + wave * kStages * L::kStage;  // this wave's three stages

  const int groups = (n_hi - n_lo + 15) / 16;
  const int g_begin = blockIdx.x * groups_per_block;
  const int g_end = min(g_begin + groups_per_block, groups);
  // copy group g (clamped into this workgroup's range) into stage st
  auto issue = [&](int g, int st) {
    g = min(g, g_end - 1);
    const int row0 = n_lo + g * 16;
    uint8_t* dst = mine + st * L::kStage;
#pragma unroll
    for (int i = 0; i < L::kCodeDma; ++i)
      llvm_amdgcn_raw_buffer_load_lds(rc, (lds_u32_ptr)(dst + i * 1024), 16, cvoff[i], row0 * ldc, 0, 0);
#pragma unroll
    for (int i = 0; i < L::kScaleDma; ++i)
      llvm_amdgcn_raw_buffer_load_lds(rs, (lds_u32_ptr)(dst + L::kCodeBytes + i * 256), 4, svoff[i],
                                      row0 * lds_, 0, 0);
  };

  __builtin_amdgcn_sched_barrier(0);  // copy offsets are ready before any load
  // The weight stream starts first; then this wave's K slice of the
  // activation rows, decoded once into registers (the decode waits for the
  // three copies as well: vmcnt counts in issue order).
  // (the grid gives every workgroup at least one group: g_begin < g_end)
  issue(g_begin, 0);
  issue(g_begin + 1, 1);
  issue(g_begin + 2, 2);
  __builtin_amdgcn_sched_barrier(0);  // keep the copies ahead of the activation loads
  u32x4 a_c[QPW];
  uint32_t a_s[QPW];
  const bool live = r16 < p.M;
  {
    const uint8_t* crow = p.a_codes + (int64_t)(live ? r16 : 0) * p.lda_c;
    const uint8_t* srow = p.a_scales + (int64_t)(live ? r16 : 0) * p.lda_s;
#pragma unroll
    for (int qi = 0; qi < QPW; ++qi) {
      const int k0 = kh + 32 * qi;
      const bool in = valid[qi] > 0;
      a_c[qi] = *reinterpret_cast<const u32x4*>(crow + (in ? (k0 >> 1) : 0));
      a_s[qi] = *reinterpret_cast<const uint16_t*>(srow + (in ? (k0 >> 4) : 0));
    }
  }
  half8 areg[QPW][4];
#pragma unroll
  for (int qi = 0; qi < QPW; ++qi) {
    mask_chunk(a_c[qi], a_s[qi], live ? valid[qi] : 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) areg[qi][t] = decode8(a_c[qi][t], scale_pair(a_s[qi], t >> 1));
  }

  const float ga = *p.ep.a_g;
  for (int r0 = g_begin; r0 < g_end; r0 += kRound) {
    const int ng = min(kRound, g_end - r0);
    if (r0 != g_begin) {
      issue(r0, 0);
      issue(r0 + 1, 1);
      issue(r0 + 2, 2);
    }
    floatx4 acc[kRound];
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      if (j < ng) {
        // group j landed: j+1 and j+2 still fly while they exist (the three
        // copies before the loop are unconditional, clamped into the range)
        if (j + 2 < ng) wait_vmem<2 * L::kDma>();
        else if (j + 1 < ng) wait_vmem<L::kDma>();
        else wait_vmem<0>();
        const uint8_t* st = mine + (j % kStages) * L::kStage;
        u32x4 c[QPW];
        uint32_t sc[QPW];
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
          c[qi] = *reinterpret_cast<const u32x4*>(st + 16 * L::slot(r16, h * QPW + qi));
          sc[qi] = *reinterpret_cast<const uint16_t*>(st + L::kCodeBytes + r16 * 8 * QPW + 2 * (h * QPW + qi));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the stage is in registers
        if (j + 3 < ng) issue(r0 + j + 3, j % kStages);  // three groups ahead, none past the round
        floatx4 a4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int qi = 0; qi < QPW; ++qi) {
          if constexpr (!FULL) mask_chunk(c[qi], sc[qi], valid[qi]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const half8 w = decode8(c[qi][t], scale_pair(sc[qi], t >> 1));
            a4 = __builtin_amdgcn_mfma_f32_16x16x32_f16(areg[qi][t], w, a4, 0, 0, 0);
          }
        }
        acc[j] = a4;
      }
    }
    __syncthreads();  // every wave has drained its copies (the last wait was vmcnt(0))
    floatx4* red = reinterpret_cast<floatx4*>(smem);  // [kRound][8 waves][64 lanes]
#pragma unroll
    for (int j = 0; j < kRound; ++j)
      if (j < ng) red[(j * kWaves + wave) * 64 + lane] = acc[j];
    __syncthreads();
    // wave w reduces groups w, w + 8 of the round over the 8 K slices
    for (int j = wave; j < ng; j += kWaves) {
      floatx4 sum = red[(j * kWaves) * 64 + lane];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) sum += red[(j * kWaves + w) * 64 + lane];
      // D[i][j]: column = lane % 16, rows 4 * (lane / 16) + r
      const int n = n_lo + (r0 + j) * 16 + r16;
      if (n < n_hi) {
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
    __syncthreads();  // the next round's copies reuse this LDS
  }
}

template <int QPW>
hipError_t launch_qpw(const GemmArgs& p, int n_lo, int n_hi, bool gate, int cus, hipStream_t s) {
  using L = SkLayout<QPW>;
  const int groups = (n_hi - n_lo + 15) / 16;
  // contiguous, equal shares of the column groups, one workgroup per CU
  const int gpb = (groups + cus - 1) / cus;
  const int grid = (groups + gpb - 1) / gpb;
  size_t lds = (size_t)kWaves * kStages * L::kStage;
  const size_t red = (size_t)kRound * kWaves * 64 * 16;
  if (lds < red) lds = red;
  const bool full = p.K == kWaves * QPW * 128;
  auto go = [&](auto kern) -> hipError_t {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    kern<<<grid, kThreads, lds, s>>>(p, n_lo, n_hi, gpb);
    return hipGetLastError();
  };
  if (gate && full) return go(skinny_kernel<QPW, true, true>);
  if (gate) return go(skinny_kernel<QPW, true, false>);
  if (full) return go(skinny_kernel<QPW, false, true>);
  return go(skinny_kernel<QPW, false, false>);
}

}  // namespace

// M <= 16; K slices up to 5 quads per wave (K <= 5120) keep the decoded
// activations in registers and the three LDS stages of 8 waves within
// 160 KB; scale copies are 4-byte aligned; byte offsets fit the 32-bit
// buffer range.
bool skinny_eligible(const GemmArgs& p) {
  return p.M <= 16 && p.K <= kWaves * 5 * 128 && p.ldw_s % 4 == 0 &&
         reinterpret_cast<uintptr_t>(p.w_scales) % 4 == 0 &&
         (int64_t)p.N * p.ldw_c < ((int64_t)1 << 31) && (int64_t)p.N * p.ldw_s < ((int64_t)1 << 31);
}

hipError_t launch_gemm_skinny(const GemmArgs& p, int n_lo, int n_hi, bool gate, hipStream_t s) {
  // compute units of the current device, asked on every call (the library
  // keeps no state between calls; the runtime answers from its own cache)
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) cus = 256;
  const int quads = (p.K + 127) / 128;
  const int qpw = (quads + kWaves - 1) / kWaves;
  switch (qpw) {
    case 1: return launch_qpw<1>(p, n_lo, n_hi, gate, cus, s);
    case 2: return launch_qpw<2>(p, n_lo, n_hi, gate, cus, s);
    case 3: return launch_qpw<3>(p, n_lo, n_hi, gate, cus, s);
    case 4: return launch_qpw<4>(p, n_lo, n_hi, gate, cus, s);
    case 5: return launch_qpw<5>(p, n_lo, n_hi, gate, cus, s);
    default: return hipErrorInvalidValue;  // the caller checks skinny_eligible() first
  }
}

}  // namespace nvfp4
