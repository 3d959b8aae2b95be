// FP8 (E4M3) KV cache with a calibrated per-tensor scale (evolve.pub review
// of arXiv 2609.04098, "Key claims under review", fifth claim; chatpaper.ai
// English abstract): calibration s = fl32(amax / 448); write: the E4M3 byte
// nearest to the exact real x / s (ties to even code, saturating at 448,
// IEEE sign), scattered to cache rows by an optional slot index; read:
// fl32(e4m3 * s), optionally rounded to bf16.  s = 1 is the uncalibrated
// cache, so calibrated and uncalibrated caches run the same code.
//
// The write without a division per element.  With R = 1/s and the bracket
// R_lo = R (1 - 2^-18), R_hi = R (1 + 2^-18), the float32 products x R_lo and
// x R_hi lie on either side of the exact quotient x / s (the margin exceeds
// the roundings of R and of the products); clamped to +-448, both go through
// gfx950's E4M3 conversion, which rounds to nearest with ties to even (and
// keeps the sign of zero) but does not saturate -- hence the clamp, which is
// the saturating rule's own answer (when every product of a wavefront's
// chunks lies within +-448 already, the clamps are skipped: they would change
// nothing).  Where both bytes agree that byte is
// exact (the map is monotone).  Where they differ (codes m and m + 1, the
// bracket being far narrower than a grid step) the quotient sits next to the
// midpoint mu between the two values; mu has <= 5 significant bits, so
// fma(mu, s, -|x|) rounds the exact difference once and its sign decides
// (zero on a tie, which goes to the even code).  Scales outside [2^-90,
// 2^126] -- where that difference could leave float32's normal range --
// divide in float64 instead (e4m3_rne, exact by the bit counts).  A power-of-
// two scale (the unit scale among them) needs no bracket: x / s is then an
// exact float32 product and one conversion is the answer.  The read
// decodes with the hardware conversion (exact for every byte) and rounds to
// bf16 with the hardware conversion (nearest even).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

using namespace dev;

// 8 consecutive elements as floats from a 16-byte (bf16) or 32-byte (f32) run.
template <int DT>
__device__ inline void load8(const uint8_t* p, float v[8]) {
  if constexpr (DT == NVFP4_DTYPE_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 16);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Walk over the 8-element chunks of a [rows, cpr] matrix from chunk `start`
// in steps of `stride` chunks, keeping (row, chunk-in-row) without a division
// per step.
struct ChunkWalk {
  int64_t r, c, cpr, rows, dr, dc;
  __device__ ChunkWalk(int64_t rows_, int64_t cpr_, int64_t start, int64_t stride) : cpr(cpr_), rows(rows_) {
    r = start / cpr;
    c = start - r * cpr;
    dr = stride / cpr;
    dc = stride - dr * cpr;
  }
  __device__ bool valid() const { return r < rows; }
  __device__ void next() {
    r += dr;
    c += dc;
    if (c >= cpr) {
      c -= cpr;
      ++r;
    }
  }
};

// Each thread takes two chunks per iteration, one grid-width apart (so every
// load instruction of a wavefront still reads contiguous bytes), and the
// cache and output bytes go out as streaming stores.  A write of contiguous
// rows without slots runs a kernel that walks one linear chunk index
// instead of (row, chunk) pairs and 64-bit row products, and issues both
// loads before the first wait.  Measured on 32768 x 1024 bf16 with 16
// rotating buffers (none left in the last-level cache), against one chunk
// per iteration with plain stores: calibrated write 25.7 -> 21.4 us (the
// linear walk and the skipped clamps -2.9 us of it), unit-scale write
// 21.7 -> 20.3 us, bf16 read unchanged at 20.5-20.9 us; four chunks per
// iteration, or fewer workgroups, were slower.
constexpr int kChunksPerIter = 2;

// Magnitude of the E4M3 byte P of `src`, decoded by the hardware conversion (exact).
template <int P>
__device__ inline float e4m3_byte_mag(uint32_t src) {
  return fabsf(__builtin_amdgcn_cvt_f32_fp8((int)src, P));
}

// Bracket repair of byte P: lo and hi differ there (magnitudes m, m + 1).
template <int P>
__device__ inline void repair_byte(uint32_t& word, uint32_t lo, uint32_t hi, float x, float s) {
  constexpr int sh = 8 * P;
  if (((lo ^ hi) >> sh) & 0xFFu) {
    const float mid = 0.5f * (e4m3_byte_mag<P>(lo) + e4m3_byte_mag<P>(hi));  // exact, <= 5 bits
    const float d = fmaf(mid, s, -fabsf(x));
    const bool up = d < 0.0f || (d == 0.0f && ((lo >> sh) & 1u));
    if (up) word = (word & ~(0xFFu << sh)) | (hi & (0xFFu << sh));
  }
}

// Four E4M3 bytes (element 0 in the low byte) of x[0..3] * r with r = 1/s a
// power of two: the products are exact (or far below the first midpoint, or
// clamped), so one conversion is the exact answer.
__device__ inline uint32_t e4m3_quad_exact(const float* x, float r) {
  const float y0 = __builtin_amdgcn_fmed3f(x[0] * r, -448.0f, 448.0f);
  const float y1 = __builtin_amdgcn_fmed3f(x[1] * r, -448.0f, 448.0f);
  const float y2 = __builtin_amdgcn_fmed3f(x[2] * r, -448.0f, 448.0f);
  const float y3 = __builtin_amdgcn_fmed3f(x[3] * r, -448.0f, 448.0f);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)w, true);
}

// Four E4M3 bytes (element 0 in the low byte) of x[0..3] / s, exactly rounded.
__device__ inline uint32_t e4m3_quad(const float* x, float r_lo, float r_hi, float s) {
  const float l0 = __builtin_amdgcn_fmed3f(x[0] * r_lo, -448.0f, 448.0f);
  const float l1 = __builtin_amdgcn_fmed3f(x[1] * r_lo, -448.0f, 448.0f);
  const float l2 = __builtin_amdgcn_fmed3f(x[2] * r_lo, -448.0f, 448.0f);
  const float l3 = __builtin_amdgcn_fmed3f(x[3] * r_lo, -448.0f, 448.0f);
  const float h0 = __builtin_amdgcn_fmed3f(x[0] * r_hi, -448.0f, 448.0f);
  const float h1 = __builtin_amdgcn_fmed3f(x[1] * r_hi, -448.0f, 448.0f);
  const float h2 = __builtin_amdgcn_fmed3f(x[2] * r_hi, -448.0f, 448.0f);
  const float h3 = __builtin_amdgcn_fmed3f(x[3] * r_hi, -448.0f, 448.0f);
  uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(l0, l1, 0, false);
  lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(l2, l3, (int)lo, true);
  uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h0, h1, 0, false);
  hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h2, h3, (int)hi, true);
  uint32_t word = lo;
  if (lo != hi) {
    repair_byte<0>(word, lo, hi, x[0], s);
    repair_byte<1>(word, lo, hi, x[1], s);
    repair_byte<2>(word, lo, hi, x[2], s);
    repair_byte<3>(word, lo, hi, x[3], s);
  }
  return word;
}

// e4m3_quad without the clamps, for inputs whose bracket products are all
// within +-448 (then the clamps change nothing).
__device__ inline uint32_t e4m3_quad_in_range(const float* x, float r_lo, float r_hi, float s) {
  uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] * r_lo, x[1] * r_lo, 0, false);
  lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2] * r_lo, x[3] * r_lo, (int)lo, true);
  uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[0] * r_hi, x[1] * r_hi, 0, false);
  hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x[2] * r_hi, x[3] * r_hi, (int)hi, true);
  uint32_t word = lo;
  if (lo != hi) {
    repair_byte<0>(word, lo, hi, x[0], s);
    repair_byte<1>(word, lo, hi, x[1], s);
    repair_byte<2>(word, lo, hi, x[2], s);
    repair_byte<3>(word, lo, hi, x[3], s);
  }
  return word;
}

struct KvScale {
  float sf, R, r_lo, r_hi;
  double s;
  bool fast, pow2;
  __device__ explicit KvScale(float sf_) : sf(sf_) {
    fast = sf >= 0x1p-90f && sf <= 0x1p126f;  // uniform over the launch
    pow2 = fast && (__float_as_uint(sf) & 0x7FFFFFu) == 0u;  // 1/s exact (s = 1 among them)
    R = 1.0f / sf;
    r_lo = R * (1.0f - 0x1p-18f);
    r_hi = R * (1.0f + 0x1p-18f);
    s = (double)sf;
  }
  // The 8 E4M3 bytes of v[0..7] / s.
  __device__ uint2 encode8(const float v[8]) const {
    uint32_t w[2] = {0u, 0u};
    if (pow2) {
      w[0] = e4m3_quad_exact(v, R);
      w[1] = e4m3_quad_exact(v + 4, R);
    } else if (fast) {
      float mx = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(v[e]));
      if (__all(mx * r_hi <= 448.0f)) {  // the clamps would change nothing
        w[0] = e4m3_quad_in_range(v, r_lo, r_hi, sf);
        w[1] = e4m3_quad_in_range(v + 4, r_lo, r_hi, sf);
      } else {
        w[0] = e4m3_quad(v, r_lo, r_hi, sf);
        w[1] = e4m3_quad(v + 4, r_lo, r_hi, sf);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t m = e4m3_rne((double)fabsf(v[e]) / s);
        w[e >> 2] |= (m | ((__float_as_uint(v[e]) >> 31) << 7)) << (8 * (e & 3));
      }
    }
    return make_uint2(w[0], w[1]);
  }
};

// Contiguous x and cache rows, no slots: chunk i at byte i * chunk of x and
// i * 8 of the cache.
template <int DT>
__global__ __launch_bounds__(kElemThreads) void kv_quant_linear_kernel(const uint8_t* __restrict__ x, int64_t total,
                                                                       uint8_t* __restrict__ cache,
                                                                       const float* __restrict__ scale) {
  constexpr int kChunkBytes = DT == NVFP4_DTYPE_BF16 ? 16 : 32;
  const KvScale ks(*scale);
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += 2 * T) {
    const int64_t i1 = i + T;
    const bool ok1 = i1 < total;
    float v0[8], v1[8];
    load8<DT>(x + i * kChunkBytes, v0);
    load8<DT>(x + (ok1 ? i1 : i) * kChunkBytes, v1);
    const uint2 w0 = ks.encode8(v0);
    store_stream8(cache + i * 8, w0.x, w0.y);
    const uint2 w1 = ks.encode8(v1);
    if (ok1) store_stream8(cache + i1 * 8, w1.x, w1.y);
  }
}

template <int DT>
__global__ __launch_bounds__(kElemThreads) void kv_quant_kernel(
    const uint8_t* __restrict__ x, int64_t ld_bytes, int64_t rows, int64_t cpr,
    const int64_t* __restrict__ slots, int64_t cache_rows, uint8_t* __restrict__ cache,
    int64_t ld_cache, const float* __restrict__ scale) {
  constexpr int kChunkBytes = DT == NVFP4_DTYPE_BF16 ? 16 : 32;
  const KvScale ks(*scale);
  constexpr int U = kChunksPerIter;
  static_assert(U == 2, "the walkers below are listed one by one");
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  ChunkWalk it[U] = {ChunkWalk(rows, cpr, start, U * T), ChunkWalk(rows, cpr, start + T, U * T)};
  while (it[0].valid()) {
    float v[U][8];
    int64_t dst[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const bool ok = it[j].valid();
      dst[j] = ok ? (slots != nullptr ? slots[it[j].r] : it[j].r) : -1;
      if (ok) load8<DT>(x + it[j].r * ld_bytes + it[j].c * kChunkBytes, v[j]);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (dst[j] < 0 || dst[j] >= cache_rows) continue;  // documented: such rows are not written
      const uint2 wv = ks.encode8(v[j]);
      store_stream8(cache + dst[j] * ld_cache + it[j].c * 8, wv.x, wv.y);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) it[j].next();
  }
}

template <int OUT>
__global__ __launch_bounds__(kElemThreads) void kv_dequant_kernel(
    const uint8_t* __restrict__ cache, int64_t ld_cache, int64_t rows, int64_t cpr,
    const float* __restrict__ scale, uint8_t* __restrict__ out, int64_t ld_out_bytes) {
  const float s = *scale;
  constexpr int U = kChunksPerIter;
  static_assert(U == 2, "the walkers below are listed one by one");
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  ChunkWalk it[U] = {ChunkWalk(rows, cpr, start, U * T), ChunkWalk(rows, cpr, start + T, U * T)};
  while (it[0].valid()) {
    uint2 q[U];
#pragma unroll
    for (int j = 0; j < U; ++j)
      if (it[j].valid()) q[j] = *reinterpret_cast<const uint2*>(cache + it[j].r * ld_cache + it[j].c * 8);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (!it[j].valid()) continue;
      float f[8];
      const f32x2_t d0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j].x, false), d1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j].x, true);
      const f32x2_t d2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j].y, false), d3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[j].y, true);
      f[0] = d0.x * s; f[1] = d0.y * s; f[2] = d1.x * s; f[3] = d1.y * s;
      f[4] = d2.x * s; f[5] = d2.y * s; f[6] = d3.x * s; f[7] = d3.y * s;
      if constexpr (OUT == NVFP4_DTYPE_BF16) {
        store_stream16(out + it[j].r * ld_out_bytes + it[j].c * 16, pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                       pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
      } else {
        uint8_t* o = out + it[j].r * ld_out_bytes + it[j].c * 32;
        store_stream16(o, __float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
        store_stream16(o + 16, __float_as_uint(f[4]), __float_as_uint(f[5]), __float_as_uint(f[6]), __float_as_uint(f[7]));
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) it[j].next();
  }
}

// s = fl32(max(partials) / 448): one correctly rounded division (53 >= 2*24+2).
__global__ __launch_bounds__(kElemThreads) void kv_scale_kernel(const float* __restrict__ partials,
                                                                int n, float* __restrict__ scale) {
  __shared__ float red[kElemThreads / 64];
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, partials[i]);
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = red[0];
    for (int i = 1; i < kElemThreads / 64; ++i) v = fmaxf(v, red[i]);
    *scale = (float)((double)v / 448.0);
  }
}

// At most 2048 workgroups (8 per CU on 256 CUs, all resident at once),
// each thread walking several chunks: measured faster than 8192 or 32768
// workgroups with fewer chunks each (32768 x 1024 bf16: write 27.3 -> 25.9
// us calibrated, read 22.9 -> 20.6 us), and than 1024 or 1536.
int chunk_grid(int64_t chunks) {
  int64_t wg = (chunks + kElemThreads - 1) / kElemThreads;
  if (wg > 2048) wg = 2048;
  if (wg < 1) wg = 1;
  return (int)wg;
}

}  // namespace

hipError_t launch_kv_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const int64_t* slots, int64_t cache_rows, uint8_t* cache,
                              int64_t ld_cache, const float* scale, hipStream_t s) {
  const int64_t cpr = cols / 8;
  const int grid = chunk_grid(rows * cpr);
  if (slots == nullptr && ld_x == cols && ld_cache == cols) {
    if (dtype == NVFP4_DTYPE_BF16)
      kv_quant_linear_kernel<NVFP4_DTYPE_BF16><<<grid, kElemThreads, 0, s>>>((const uint8_t*)x, rows * cpr, cache, scale);
    else
      kv_quant_linear_kernel<NVFP4_DTYPE_F32><<<grid, kElemThreads, 0, s>>>((const uint8_t*)x, rows * cpr, cache, scale);
    return hipGetLastError();
  }
  if (dtype == NVFP4_DTYPE_BF16)
    kv_quant_kernel<NVFP4_DTYPE_BF16><<<grid, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * 2, rows, cpr, slots, cache_rows, cache, ld_cache, scale);
  else
    kv_quant_kernel<NVFP4_DTYPE_F32><<<grid, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * 4, rows, cpr, slots, cache_rows, cache, ld_cache, scale);
  return hipGetLastError();
}

hipError_t launch_kv_dequantize(const uint8_t* cache, int64_t rows, int64_t cols, int64_t ld_cache,
                                const float* scale, void* out, int out_dtype, int64_t ld_out,
                                hipStream_t s) {
  const int64_t cpr = cols / 8;
  const int grid = chunk_grid(rows * cpr);
  if (out_dtype == NVFP4_DTYPE_BF16)
    kv_dequant_kernel<NVFP4_DTYPE_BF16><<<grid, kElemThreads, 0, s>>>(cache, ld_cache, rows, cpr, scale,
                                                                      (uint8_t*)out, ld_out * 2);
  else
    kv_dequant_kernel<NVFP4_DTYPE_F32><<<grid, kElemThreads, 0, s>>>(cache, ld_cache, rows, cpr, scale,
                                                                     (uint8_t*)out, ld_out * 4);
  return hipGetLastError();
}

hipError_t launch_kv_scale(const float* partials, int n, float* scale, hipStream_t s) {
  kv_scale_kernel<<<1, kElemThreads, 0, s>>>(partials, n, scale);
  return hipGetLastError();
}

}  // namespace nvfp4
