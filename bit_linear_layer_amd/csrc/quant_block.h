// Exact NVFP4 quantization of one 16-element block, shared by the quantize
// pass and the GEMM epilogue that quantizes its own output.
//
// Format (evolve.pub review of arXiv 2609.04098, "Scope & Claims";
// thevalue.engineering article, section on the fragility myth): E2M1 codes
// with one E4M3 scale per 16 consecutive elements and one float32 global
// scale g per tensor.
//
// Exact rounding without division per element.  For a block with E4M3 scale
// s, the magnitude code of x is the number of E2M1 midpoints mu in {0.25,
// 0.75, 1.25, 1.75, 2.5, 3.5, 5} that |x| passes, where "passes" is > for
// the midpoints whose tie goes down (to an even code) and >= for those whose
// tie goes up.  |x| has <= 24 significant bits, mu * s * g <= 3 + 4 + 24 = 31
// bits, so both are exact float64 numbers and the float64 comparisons are the
// exact-real decisions.  The block scale is one correctly rounded float64
// division amax_b / (6 g): a non-tie quotient lies >= 2^-31 (relative) from
// every E4M3 midpoint, far above float64's 2^-53 rounding, so rounding the
// float64 quotient to E4M3 is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {
namespace dev {

// E4M3 (OCP FN) code nearest to r >= 0: ties to even code, r >= 448 -> 0x7E.
__device__ inline uint32_t e4m3_rne(double r) {
  if (r >= 448.0) return 0x7Eu;
  if (r < 0x1p-6) return (uint32_t)rint(r * 512.0);  // subnormal grid k * 2^-9 (8 = min normal)
  int e;
  const double f = frexp(r, &e);                     // r = f * 2^e, f in [0.5, 1)
  const uint32_t q = (uint32_t)rint(f * 16.0);       // 8..16, 16 carries into the exponent
  const uint32_t code = (uint32_t)((e + 6) << 3) + q - 8u;
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ inline double e4m3_value(uint32_t code) {
  const uint32_t e = code >> 3, m = code & 7u;
  return e == 0 ? (double)m * 0x1p-9 : ldexp(1.0 + (double)m * 0.125, (int)e - 7);
}

// Quantize v[0..15] with global scale g: 8 code bytes (low nibble = even
// element) in *codes, the E4M3 scale byte returned.
__device__ inline uint32_t quantize_block16(const float v[16], float g, uint2* codes) {
  const double g64 = (double)g;
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));

  uint32_t s = 0;
  if (g != 0.0f && amax_b != 0.0f) s = e4m3_rne((double)amax_b / (6.0 * g64));  // 6 g is exact

  // thresholds mu * s * g, exact in float64; s == 0 -> every magnitude code is 0
  double t0, t1, t2, t3, t4, t5, t6;
  if (s == 0) {
    t0 = t1 = t2 = t3 = t4 = t5 = t6 = __builtin_inf();
  } else {
    const double sg = e4m3_value(s) * g64;
    t0 = 0.25 * sg; t1 = 0.75 * sg; t2 = 1.25 * sg; t3 = 1.75 * sg;
    t4 = 2.5 * sg;  t5 = 3.5 * sg;  t6 = 5.0 * sg;
  }
  uint32_t word[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const double a = (double)fabsf(v[i]);
    uint32_t c = (a > t0) + (a >= t1) + (a > t2) + (a >= t3) + (a > t4) + (a >= t5) + (a > t6);
    c |= (__float_as_uint(v[i]) >> 31) << 3;
    word[i >> 3] |= c << (4 * (i & 7));
  }
  *codes = make_uint2(word[0], word[1]);
  return s;
}

}  // namespace dev
}  // namespace nvfp4
