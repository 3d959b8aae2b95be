// NVFP4 quantization kernels for gfx950: the amax pass and the quantize pass.
//
// Format (evolve.pub review of arXiv 2609.04098, "Scope & Claims";
// thevalue.engineering article, section on the fragility myth): E2M1 codes
// with one E4M3 scale per 16 consecutive elements, plus one float32 global
// scale per tensor.  The activations of every linear layer go through this
// on the fly (chatpaper.ai English abstract: W4A4 on all linear layers).
// The exact rounding of one block is quantize_block16 (quant_block.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_util.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// Max over the workgroup (kElemThreads threads); every thread gets it.
__device__ inline float block_max(float v) {
  __shared__ float red[kElemThreads / 64];
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kElemThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One 16-element block as raw words: 2 x 16 bytes (bf16) or 4 x 16 bytes (f32).
template <int DT>
struct RawBlock {
  static constexpr int kVec = DT == NVFP4_DTYPE_BF16 ? 2 : 4;
  uint4 q[kVec];
  __device__ void load(const uint8_t* p) {  // p 16-byte aligned
#pragma unroll
    for (int i = 0; i < kVec; ++i) q[i] = *reinterpret_cast<const uint4*>(p + 16 * i);
  }
  __device__ void to_float(float v[16]) const {
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
      const uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (DT == NVFP4_DTYPE_BF16) {
          v[8 * i + 2 * j] = bf16_lo(w[j]);
          v[8 * i + 2 * j + 1] = bf16_hi(w[j]);
        } else {
          v[4 * i + j] = __uint_as_float(w[j]);
        }
      }
    }
  }
};

// Walks the 16-element blocks of a [rows, bpr*16] matrix with a grid-stride
// loop, keeping (row, block-in-row) without a division per step.
struct BlockWalk {
  int64_t r, j, bpr, rows;
  int64_t dr, dj;
  __device__ BlockWalk(int64_t rows_, int64_t bpr_) : bpr(bpr_), rows(rows_) {
    const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    r = start / bpr;
    j = start - r * bpr;
    dr = stride / bpr;
    dj = stride - dr * bpr;
  }
  __device__ bool valid() const { return r < rows; }
  __device__ void next() {
    r += dr;
    j += dj;
    if (j >= bpr) {
      j -= bpr;
      ++r;
    }
  }
};

template <int DT>
__global__ __launch_bounds__(kElemThreads) void amax_kernel(const uint8_t* __restrict__ x,
                                                            int64_t ld_bytes, int64_t rows,
                                                            int64_t bpr,
                                                            float* __restrict__ partials) {
  constexpr int kBlockBytes = DT == NVFP4_DTYPE_BF16 ? 32 : 64;
  float m = 0.0f;
  // Contiguous rows: one linear block index, two blocks per iteration (both
  // loads in flight together), no 64-bit row products.
  if (ld_bytes == bpr * kBlockBytes) {
    const int64_t total = rows * bpr, T = (int64_t)gridDim.x * blockDim.x;
    for (int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; b < total; b += 2 * T) {
      const bool ok1 = b + T < total;
      RawBlock<DT> b0, b1;
      b0.load(x + b * kBlockBytes);
      b1.load(x + (ok1 ? b + T : b) * kBlockBytes);
      float v[16];
      b0.to_float(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      b1.to_float(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    m = block_max(m);
    if (threadIdx.x == 0) partials[blockIdx.x] = m;
    return;
  }
  for (BlockWalk it(rows, bpr); it.valid(); it.next()) {
    RawBlock<DT> b;
    b.load(x + it.r * ld_bytes + it.j * kBlockBytes);
    float v[16];
    b.to_float(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
  }
  m = block_max(m);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

template <int DT>
__global__ __launch_bounds__(kElemThreads) void quantize_kernel(
    const uint8_t* __restrict__ x, int64_t ld_bytes, int64_t rows, int64_t bpr,
    uint8_t* __restrict__ codes, int64_t ld_codes, uint8_t* __restrict__ scales,
    int64_t ld_scales, float* __restrict__ gptr, int mode, float* __restrict__ partials,
    int n_partials) {
  constexpr int kBlockBytes = DT == NVFP4_DTYPE_BF16 ? 32 : 64;
  float g;
  if (mode == 2) {
    // Small tensors, one workgroup: the amax pass runs here too (one launch
    // instead of two).  The partials are left as the amax kernel would
    // leave them (the max in slot 0, zeros after it).
    float m = 0.0f;
    for (BlockWalk it(rows, bpr); it.valid(); it.next()) {
      RawBlock<DT> b;
      b.load(x + it.r * ld_bytes + it.j * kBlockBytes);
      float v[16];
      b.to_float(v);
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    m = block_max(m);
    g = (float)((double)m / 2688.0);  // one correctly rounded division (53 >= 2*24+2)
    if (threadIdx.x == 0) *gptr = g;
    for (int i = threadIdx.x; i < n_partials; i += blockDim.x) partials[i] = i == 0 ? m : 0.0f;
  } else if (mode == 0) {
    float m = 0.0f;
    for (int i = threadIdx.x; i < n_partials; i += blockDim.x) m = fmaxf(m, partials[i]);
    m = block_max(m);
    g = (float)((double)m / 2688.0);  // one correctly rounded division (53 >= 2*24+2)
    if (blockIdx.x == 0 && threadIdx.x == 0) *gptr = g;
  } else {
    g = *gptr;
  }
  // Software-pipelined: the next block's load is issued before this block's
  // stores, so waiting for a load never waits for earlier stores (loads and
  // stores share one counter).  Past the end the load re-reads the current
  // block (a valid address) rather than branching around it.
  // Contiguous x, codes and scales: the same pipelined loop over one linear
  // block index (no 64-bit row products; h of the MLP step 68.7 -> 66.4 us,
  // X 36 -> 34.7 us with its amax pass, same-process A/B).
  if (ld_bytes == bpr * kBlockBytes && ld_codes == bpr * 8 && ld_scales == bpr) {
    const int64_t total = rows * bpr, T = (int64_t)gridDim.x * blockDim.x;
    int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= total) return;
    RawBlock<DT> cur;
    cur.load(x + b * kBlockBytes);
    while (true) {
      const int64_t bn = b + T;
      const bool more = bn < total;
      RawBlock<DT> nb;
      nb.load(x + (more ? bn : b) * kBlockBytes);
      float v[16];
      cur.to_float(v);
      uint2 c;
      const uint32_t s = dev::quantize_block16(v, g, &c);
      dev::store_stream8(codes + b * 8, c.x, c.y);
      dev::store_stream1(scales + b, (uint8_t)s);
      if (!more) break;
      cur = nb;
      b = bn;
    }
    return;
  }
  BlockWalk it(rows, bpr);
  if (!it.valid()) return;
  RawBlock<DT> cur;
  cur.load(x + it.r * ld_bytes + it.j * kBlockBytes);
  while (true) {
    BlockWalk nx = it;
    nx.next();
    const bool more = nx.valid();
    RawBlock<DT> nb;
    nb.load(x + (more ? nx.r : it.r) * ld_bytes + (more ? nx.j : it.j) * kBlockBytes);
    float v[16];
    cur.to_float(v);
    uint2 c;
    const uint32_t s = dev::quantize_block16(v, g, &c);
    dev::store_stream8(codes + it.r * ld_codes + it.j * 8, c.x, c.y);
    dev::store_stream1(scales + it.r * ld_scales + it.j, (uint8_t)s);
    if (!more) break;
    cur = nb;
    it = nx;
  }
}

}  // namespace

int partial_count(int64_t rows, int64_t cols, int chunk) {
  const int64_t work = rows * (cols / chunk);
  int64_t wg = (work + kElemThreads - 1) / kElemThreads;
  if (wg < 1) wg = 1;
  if (wg > kMaxPartials) wg = kMaxPartials;
  return (int)wg;
}

hipError_t launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                       float* partials, int n_partials, hipStream_t s) {
  const int esz = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  const int64_t bpr = cols / 16;
  if (dtype == NVFP4_DTYPE_BF16)
    amax_kernel<NVFP4_DTYPE_BF16><<<n_partials, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * esz, rows, bpr, partials);
  else
    amax_kernel<NVFP4_DTYPE_F32><<<n_partials, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * esz, rows, bpr, partials);
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           float* g, int mode, float* partials, int n_partials,
                           hipStream_t s) {
  const int esz = dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  const int64_t bpr = cols / 16;
  // enough workgroups to cover the chip several times, bounded so the
  // per-workgroup reduction of the partials stays cheap; mode 2 (amax in
  // the same kernel) runs as one workgroup
  int64_t wg = (rows * bpr + kElemThreads - 1) / kElemThreads;
  if (wg > 4096) wg = 4096;
  if (wg < 1 || mode == 2) wg = 1;
  if (dtype == NVFP4_DTYPE_BF16)
    quantize_kernel<NVFP4_DTYPE_BF16><<<(int)wg, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * esz, rows, bpr, codes, ld_codes, scales, ld_scales, g, mode,
        partials, n_partials);
  else
    quantize_kernel<NVFP4_DTYPE_F32><<<(int)wg, kElemThreads, 0, s>>>(
        (const uint8_t*)x, ld_x * esz, rows, bpr, codes, ld_codes, scales, ld_scales, g, mode,
        partials, n_partials);
  return hipGetLastError();
}

}  // namespace nvfp4
