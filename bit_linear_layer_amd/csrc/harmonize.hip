// Checkpoint-side scale harmonization of modules that one GEMM serves with a
// single global scale (evolve.pub review of arXiv 2609.04098, "Key claims
// under review", fourth claim; chatpaper.ai English abstract): the group
// shares G = max_s g_s and every block scale byte b of segment s becomes the
// E4M3 value nearest to the exact real e4m3(b) * g_s / G (ties to the even
// code; the ratio is <= 1, so nothing saturates).  E2M1 codes are unchanged.
//
// Exactness: e4m3(b) * g_s has <= 28 significant bits (exact in float64), G
// has 24; a non-tie quotient lies >= ~2^-30 (relative) from every E4M3
// midpoint and a tie divides exactly, so one float64 division rounded by
// e4m3_rne takes the exact-real decision.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

namespace {

using namespace dev;

__global__ __launch_bounds__(kElemThreads) void harmonize_kernel(
    const uint8_t* __restrict__ in, int64_t ld_in, uint8_t* out, int64_t ld_out, int64_t rows,
    int64_t bpr, SegmentTable seg, const float* __restrict__ seg_g, float* __restrict__ g_out) {
  float G = 0.0f;
  for (int s = 0; s < seg.n; ++s) G = fmaxf(G, seg_g[s]);
  if (blockIdx.x == 0 && threadIdx.x == 0) *g_out = G;
  const double G64 = (double)G;
  const int64_t start = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = start; i < rows * bpr; i += stride) {
    const int64_t r = i / bpr, j = i - r * bpr;
    int s = 0;
    while (s + 1 < seg.n && r >= seg.off[s + 1]) ++s;
    const uint32_t b = in[r * ld_in + j];  // read before the (possibly in-place) write
    const uint32_t nb = G64 > 0.0 ? e4m3_rne(e4m3_value(b) * (double)seg_g[s] / G64) : 0u;
    out[r * ld_out + j] = (uint8_t)nb;
  }
}

}  // namespace

hipError_t launch_harmonize(const uint8_t* in, int64_t ld_in, uint8_t* out, int64_t ld_out,
                            int64_t rows, int64_t bpr, const SegmentTable& seg, const float* seg_g,
                            float* g_out, hipStream_t s) {
  int64_t wg = (rows * bpr + kElemThreads - 1) / kElemThreads;
  if (wg > 4096) wg = 4096;
  if (wg < 1) wg = 1;
  harmonize_kernel<<<(int)wg, kElemThreads, 0, s>>>(in, ld_in, out, ld_out, rows, bpr, seg, seg_g, g_out);
  return hipGetLastError();
}

}  // namespace nvfp4
