// MLP glue between the two NVFP4 GEMMs of a gated MLP: h = bf16(silu(gate) * up),
// with the amax partials of h produced on the way, so that the quantize pass
// of h needs no separate amax pass over it.  (The pages fix no MLP detail;
// the gated-MLP layout, gate = first half of the gate_up output, is this
// library's reading.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"

namespace nvfp4 {

namespace {

using namespace dev;

__global__ __launch_bounds__(kElemThreads) void silu_mul_kernel(
    const uint16_t* __restrict__ gu, int64_t ld_gu, uint16_t* __restrict__ h, int64_t ld_h,
    int64_t rows, int64_t inter, float* __restrict__ partials) {
  const int64_t cpr = inter / 8;  // 8-element chunks per row
  const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t r = start / cpr, c = start - r * cpr;
  const int64_t dr = stride / cpr, dc = stride - dr * cpr;
  float m = 0.0f;
  for (; r < rows; r += dr, c += dc) {
    if (c >= cpr) {
      c -= cpr;
      ++r;
      if (r >= rows) break;
    }
    const uint16_t* row = gu + r * ld_gu;
    const uint4 gq = *reinterpret_cast<const uint4*>(row + c * 8);
    const uint4 uq = *reinterpret_cast<const uint4*>(row + inter + c * 8);
    const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w};
    const uint32_t uw[4] = {uq.x, uq.y, uq.z, uq.w};
    uint32_t hw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float h0 = silu(__uint_as_float(gw[i] << 16)) * __uint_as_float(uw[i] << 16);
      const float h1 = silu(__uint_as_float(gw[i] & 0xFFFF0000u)) * __uint_as_float(uw[i] & 0xFFFF0000u);
      const uint32_t b0 = f32_to_bf16_bits(h0), b1 = f32_to_bf16_bits(h1);
      hw[i] = b0 | (b1 << 16);
      m = fmaxf(m, fmaxf(__uint_as_float((b0 & 0x7FFFu) << 16), __uint_as_float((b1 & 0x7FFFu) << 16)));
    }
    dev::store_stream16(h + r * ld_h + c * 8, hw[0], hw[1], hw[2], hw[3]);
  }
  if (partials != nullptr) {
    __shared__ float red[kElemThreads / 64];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float v = red[0];
      for (int i = 1; i < kElemThreads / 64; ++i) v = fmaxf(v, red[i]);
      partials[blockIdx.x] = v;
    }
  }
}

__global__ __launch_bounds__(kElemThreads) void zero_kernel(float* __restrict__ p, int n) {
  const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = 0.0f;
}

}  // namespace

hipError_t launch_zero(float* p, int n, hipStream_t s) {
  zero_kernel<<<(n + kElemThreads - 1) / kElemThreads, kElemThreads, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu,
                           uint16_t* h, int64_t ld_h, float* partials, int n_partials,
                           hipStream_t s) {
  silu_mul_kernel<<<n_partials, kElemThreads, 0, s>>>(gu, ld_gu, h, ld_h, rows, inter, partials);
  return hipGetLastError();
}

}  // namespace nvfp4
