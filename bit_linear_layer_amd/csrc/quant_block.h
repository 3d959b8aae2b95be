// Exact NVFP4 quantization of one 16-element block, shared by the quantize
// pass and the GEMM epilogue that quantizes its own output.  Blocks take a
// bracketed path on the hardware E2M1 pack with an exact per-element repair
// (quantize_block16), and the block scale a bracketed path on the hardware
// E4M3 conversion (block_scale_code); scales outside float32's comfortable
// range take the threshold count and the float64 division below.
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
// tie goes up.  mu * s * g <= 3 + 4 + 24 = 31 bits is an exact float64
// number; |x| is a float32, so "|x| > t" is "|x| >= the next float32 above
// t" and "|x| >= t" is "|x| >= the smallest float32 not below t" -- one exact
// float32 bound per threshold and block.  The float64 form of the block
// scale is one correctly rounded division amax_b / (6 g): a non-tie quotient
// lies >= 2^-31 (relative) from every E4M3 midpoint, far above float64's
// 2^-53 rounding, so rounding the float64 quotient to E4M3 is exact.
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

// Smallest float32 c with c >= t (strict: c > t), for a float64 t >= 0:
// for a float32 x, x >= t <=> x >= c (strict: x > t <=> x >= c).  Values
// beyond the float32 range give +inf (no float32 passes them).
__device__ inline float f32_ceil_bound(double t, bool strict) {
  float c = (float)t;  // nearest; may lie below t
  if ((double)c < t || (strict && (double)c == t)) c = __uint_as_float(__float_as_uint(c) + 1u);
  return c;
}

// Exact magnitude-count rounding of v[0..15] under block scale code s and
// global scale g.  The seven thresholds mu * s * g are exact float64
// numbers; each becomes a float32 bound once per block (f32_ceil_bound, with
// > or >= per midpoint's tie direction), so every element takes its exact
// decisions with float32 comparisons.
__device__ inline uint2 codes_by_thresholds(const float v[16], uint32_t s, float g) {
  float b0, b1, b2, b3, b4, b5, b6;
  if (s == 0) {  // every magnitude code is 0
    b0 = b1 = b2 = b3 = b4 = b5 = b6 = __builtin_inff();
  } else {
    const double sg = e4m3_value(s) * (double)g;
    b0 = f32_ceil_bound(0.25 * sg, true);  b1 = f32_ceil_bound(0.75 * sg, false);
    b2 = f32_ceil_bound(1.25 * sg, true);  b3 = f32_ceil_bound(1.75 * sg, false);
    b4 = f32_ceil_bound(2.5 * sg, true);   b5 = f32_ceil_bound(3.5 * sg, false);
    b6 = f32_ceil_bound(5.0 * sg, true);
  }
  uint32_t word[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float a = fabsf(v[i]);
    uint32_t c = (a >= b0) + (a >= b1) + (a >= b2) + (a >= b3) + (a >= b4) + (a >= b5) + (a >= b6);
    c |= (__float_as_uint(v[i]) >> 31) << 3;
    word[i >> 3] |= c << (4 * (i & 7));
  }
  return make_uint2(word[0], word[1]);
}

// E4M3 (OCP FN) magnitude code -> float32, exact (no NaN code reaches here).
__device__ inline float e4m3_value_f32(uint32_t code) {
  return code < 8u ? (float)code * 0x1p-9f : __uint_as_float((code + (120u << 3)) << 20);
}

// E4M3 code of the block scale: the nearest E4M3 value to the exact real
// amax_b / (6 g), ties to the even code, saturating at 448, 0 for a zero
// block or g = 0.  Bracketed like the elements: fl32(6 g) and its hardware
// reciprocal widened by 2^-18 each way put two float32 products on either
// side of the exact quotient; clamped to 448 (the saturating rule's own
// answer) both go through gfx950's E4M3 conversion (nearest, ties to even,
// subnormals included).  Equal codes are exact; otherwise the quotient is
// next to the midpoint mu of the two candidate values, and
// fma(6 mu, g, -amax_b) decides (6 mu has <= 7 bits; with 6 g in
// [2^-80, 2^100] a nonzero difference is a normal float32; zero is a tie,
// which goes to the even code).  Outside that range: one correctly rounded
// float64 division (exact by the bit counts above).
__device__ inline uint32_t block_scale_code(float amax_b, float g) {
  if (g == 0.0f || amax_b == 0.0f) return 0u;
  const float d6 = 6.0f * g;
  if (!(d6 >= 0x1p-80f && d6 <= 0x1p100f)) return e4m3_rne((double)amax_b / (6.0 * (double)g));  // 6 g is exact
  const float r = __builtin_amdgcn_rcpf(d6);
  const float q_lo = fminf(amax_b * (r * (1.0f - 0x1p-18f)), 448.0f);
  const float q_hi = fminf(amax_b * (r * (1.0f + 0x1p-18f)), 448.0f);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q_lo, q_hi, 0, false);
  const uint32_t lo = w & 0xFFu, hi = (w >> 8) & 0xFFu;
  if (lo == hi) return lo;
  const float mu6 = 3.0f * (e4m3_value_f32(lo) + e4m3_value_f32(hi));  // 6 * midpoint, exact
  const float d = fmaf(mu6, g, -amax_b);
  return (d < 0.0f || (d == 0.0f && (lo & 1u))) ? hi : lo;
}

// Byte P of lo / hi <- E2M1 codes of (a, b) times r_lo / r_hi (a in the low nibble).
template <int P>
__device__ inline void pack_pair(uint32_t& lo, uint32_t& hi, float a, float b, float r_lo, float r_hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, a * r_lo, b * r_lo, 1.0f, P);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, a * r_hi, b * r_hi, 1.0f, P);
}

// Quantize v[0..15] with global scale g: 8 code bytes (low nibble = even
// element) in *codes, the E4M3 scale byte returned.
//
// Bracketed fast path.  With S = fl32(s * g) in [2^-90, 2^126] and
// R = rcp(S) (within 2^-23 of 1/S), R_lo = R (1 - 2^-18) and
// R_hi = R (1 + 2^-18) put fl32(x R_lo) and fl32(x R_hi) on either side of
// the exact quotient x / (s g): the margin 2^-18 exceeds the sum of the four
// roundings (2^-24 each) and rcp's 2^-23.  gfx950's E2M1 pack instruction
// rounds to the nearest code with ties to even, saturates beyond 6 and keeps
// the sign of zero -- the same map as the exact definition -- and that map is
// monotone, so where both products give the same code, so does the exact
// quotient.  Products that underflow lie far below the first midpoint.
//
// Where the two codes differ (magnitudes m and m + 1: the bracket is far
// narrower than the gap between midpoints), the exact quotient sits next to
// the midpoint mu_m, and one fused multiply-add decides: mu_m * s is exact in
// float32 (<= 9 bits), fma(mu_m s, g, -|x|) rounds the exact difference once,
// so its sign is exact (zero only on a tie, which goes to the even code; with
// S >= 2^-90 a nonzero difference is a normal float32).  Bf16 data hits this
// often: with g = amax / 2688, many quotients fall within 2^-24 of a
// midpoint.  s == 0 gives R = 0: every product is a signed zero, the exact
// answer.  S outside the range above takes the threshold count.
__device__ inline uint32_t quantize_block16(const float v[16], float g, uint2* codes) {
  float amax_b = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));

  const uint32_t s = block_scale_code(amax_b, g);
  const float sv = e4m3_value_f32(s);
  const float S = sv * g;
  if (s != 0u && !(S >= 0x1p-90f && S <= 0x1p126f)) {
    *codes = codes_by_thresholds(v, s, g);
    return s;
  }
  const float R = s == 0u ? 0.0f : __builtin_amdgcn_rcpf(S);
  const float r_lo = R * (1.0f - 0x1p-18f), r_hi = R * (1.0f + 0x1p-18f);
  uint32_t lo0 = 0u, lo1 = 0u, hi0 = 0u, hi1 = 0u;
  pack_pair<0>(lo0, hi0, v[0], v[1], r_lo, r_hi);    pack_pair<0>(lo1, hi1, v[8], v[9], r_lo, r_hi);
  pack_pair<1>(lo0, hi0, v[2], v[3], r_lo, r_hi);    pack_pair<1>(lo1, hi1, v[10], v[11], r_lo, r_hi);
  pack_pair<2>(lo0, hi0, v[4], v[5], r_lo, r_hi);    pack_pair<2>(lo1, hi1, v[12], v[13], r_lo, r_hi);
  pack_pair<3>(lo0, hi0, v[6], v[7], r_lo, r_hi);    pack_pair<3>(lo1, hi1, v[14], v[15], r_lo, r_hi);

  const float mu_scale = 0.25f * sv;  // mu_m * s = (4 mu_m) * mu_scale, exact
  uint32_t word[2] = {lo0, lo1};
  const uint32_t hi[2] = {hi0, hi1};
  const uint32_t diff[2] = {lo0 ^ hi0, lo1 ^ hi1};
#pragma unroll
  for (int q = 0; q < 4; ++q) {  // groups of 4 elements: most waves skip most groups
    const int w = q >> 1;
    if ((diff[w] >> (16 * (q & 1))) & 0xFFFFu) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q + e, sh = 4 * (i & 7);
        if ((diff[w] >> sh) & 0xFu) {
          const uint32_t m = (word[w] >> sh) & 7u;
          const uint32_t mu4 = m < 4u ? 2u * m + 1u : (m == 6u ? 20u : 4u * m - 6u);  // 4 x {.25 .75 1.25 1.75 2.5 3.5 5}
          const float d = fmaf((float)mu4 * mu_scale, g, -fabsf(v[i]));
          const bool up = d < 0.0f || (d == 0.0f && (m & 1u));
          if (up) word[w] = (word[w] & ~(0xFu << sh)) | (hi[w] & (0xFu << sh));
        }
      }
    }
  }
  *codes = make_uint2(word[0], word[1]);
  return s;
}

}  // namespace dev
}  // namespace nvfp4
