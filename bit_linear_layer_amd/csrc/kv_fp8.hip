// FP8 (E4M3) KV cache with a calibrated per-tensor scale (evolve.pub review
// of arXiv 2609.04098, "Key claims under review", fifth claim; chatpaper.ai
// English abstract): calibration s = fl32(amax / 448); write: the E4M3 byte
// nearest to the exact real x / s (ties to even code, saturating at 448,
// IEEE sign), scattered to cache rows by an optional slot index; read:
// fl32(e4m3 * s), optionally rounded to bf16.  s = 1 is the uncalibrated
// cache, so calibrated and uncalibrated caches run the same code.
//
// Exactness of the write without a division per element: the float32
// estimate r = |x| * fl32(1/s) is within 2 ulps of the exact quotient, so
// truncating it to the E4M3 grid names the code `lo` just below the quotient
// and the midpoint above it (away from a grid point by far more than 2 ulps).
// The midpoint has <= 5 significant bits and is exact in float32, s has 24,
// so midpoint * s is an exact float64 number and comparing |x| with it (a
// tie goes to the even code) is the exact-real decision.  No lane branches,
// so calibrated and unit scales cost the same.  Subnormal scales, whose
// reciprocal overflows, divide in float64 instead (e4m3_rne, exact by the
// same bit counts).
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

// Grid-stride walk over [rows, cpr] 8-element chunks.
struct ChunkWalk {
  int64_t r, c, cpr, rows, dr, dc;
  __device__ ChunkWalk(int64_t rows_, int64_t cpr_) : cpr(cpr_), rows(rows_) {
    const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
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

// E4M3 (OCP FN) byte -> float, exact.  Normal: the 7 magnitude bits are the
// float32 exponent/mantissa fields shifted, exponent rebased 7 -> 127
// (+120 << 3); subnormal: m * 2^-9.
__device__ inline float e4m3_to_f32(uint32_t b) {
  const uint32_t mag = b & 0x7Fu;
  const float v = mag < 8u ? (float)mag * 0x1p-9f : __uint_as_float((mag + 960u) << 20);
  return __uint_as_float(__float_as_uint(v) | ((b & 0x80u) << 24));
}

// Magnitude code (0..0x7E) of the E4M3 value nearest to the exact real
// ax / s (ax >= 0), ties to the even code, saturating at 448.  Branch-free:
// r names the code `lo` just below the quotient and the midpoint above it;
// one exact float64 comparison decides.
__device__ inline uint32_t e4m3_quotient_code(float ax, float inv_s, double s) {
  const float r = ax * inv_s;
  const uint32_t b = __float_as_uint(r);
  const float t = r * 512.0f;  // subnormal grid k * 2^-9 (k = 8 is the smallest normal)
  const float k = floorf(t);
  const bool normal = r >= 0x1p-6f;
  const uint32_t lo = normal ? (b >> 20) - (120u << 3) : (uint32_t)k;  // mantissa truncated to 3 bits
  const float mid = normal ? __uint_as_float((b & 0xFFF00000u) | 0x80000u) : (k + 0.5f) * 0x1p-9f;
  const double m = (double)mid * s;  // exact: <= 5 bits times 24 bits
  const double a = (double)ax;
  const uint32_t up = (a > m || (a == m && (lo & 1u))) ? 1u : 0u;  // a tie goes to the even code
  return min(lo + up, 0x7Eu);
}

template <int DT>
__global__ __launch_bounds__(kElemThreads) void kv_quant_kernel(
    const uint8_t* __restrict__ x, int64_t ld_bytes, int64_t rows, int64_t cpr,
    const int64_t* __restrict__ slots, int64_t cache_rows, uint8_t* __restrict__ cache,
    int64_t ld_cache, const float* __restrict__ scale) {
  constexpr int kChunkBytes = DT == NVFP4_DTYPE_BF16 ? 16 : 32;
  const float sf = *scale;
  const float inv_s = 1.0f / sf;
  const double s = (double)sf;
  const bool fast = inv_s < 0x1p127f;  // 1/s overflows only for subnormal s: divide instead
  for (ChunkWalk it(rows, cpr); it.valid(); it.next()) {
    const int64_t dst = slots != nullptr ? slots[it.r] : it.r;
    if (dst < 0 || dst >= cache_rows) continue;  // documented: such rows are not written
    float v[8];
    load8<DT>(x + it.r * ld_bytes + it.c * kChunkBytes, v);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t m = fast ? e4m3_quotient_code(fabsf(v[e]), inv_s, s) : e4m3_rne((double)fabsf(v[e]) / s);
      const uint32_t b = m | ((__float_as_uint(v[e]) >> 31) << 7);
      w[e >> 2] |= b << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(cache + dst * ld_cache + it.c * 8) = make_uint2(w[0], w[1]);
  }
}

template <int OUT>
__global__ __launch_bounds__(kElemThreads) void kv_dequant_kernel(
    const uint8_t* __restrict__ cache, int64_t ld_cache, int64_t rows, int64_t cpr,
    const float* __restrict__ scale, uint8_t* __restrict__ out, int64_t ld_out_bytes) {
  const float s = *scale;
  for (ChunkWalk it(rows, cpr); it.valid(); it.next()) {
    const uint2 q = *reinterpret_cast<const uint2*>(cache + it.r * ld_cache + it.c * 8);
    const uint32_t w[2] = {q.x, q.y};
    float f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = e4m3_to_f32((w[e >> 2] >> (8 * (e & 3))) & 0xFFu) * s;
    if constexpr (OUT == NVFP4_DTYPE_BF16) {
      uint32_t h[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = f32_to_bf16_bits(f[2 * i]) | (f32_to_bf16_bits(f[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(out + it.r * ld_out_bytes + it.c * 16) = make_uint4(h[0], h[1], h[2], h[3]);
    } else {
      float4* o = reinterpret_cast<float4*>(out + it.r * ld_out_bytes + it.c * 32);
      o[0] = make_float4(f[0], f[1], f[2], f[3]);
      o[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
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

int chunk_grid(int64_t chunks) {
  int64_t wg = (chunks + kElemThreads - 1) / kElemThreads;
  if (wg > 8192) wg = 8192;
  if (wg < 1) wg = 1;
  return (int)wg;
}

}  // namespace

hipError_t launch_kv_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const int64_t* slots, int64_t cache_rows, uint8_t* cache,
                              int64_t ld_cache, const float* scale, hipStream_t s) {
  const int64_t cpr = cols / 8;
  const int grid = chunk_grid(rows * cpr);
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
