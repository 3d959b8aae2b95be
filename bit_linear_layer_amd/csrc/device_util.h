// Device helpers shared by the NVFP4 GEMM kernels: exact decode of E2M1
// codes times an E4M3 block scale into fp16, bf16 rounding, gate functions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The LLVM intrinsic behind buffer_load ... lds (LDS DMA), declared by name.
typedef int32_t nvfp4_i32x4 __attribute__((ext_vector_type(4)));
extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(
    nvfp4_i32x4 rsrc, __attribute__((address_space(3))) uint32_t* lds, int size, int voffset,
    int soffset, int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace nvfp4 {
namespace dev {

typedef nvfp4_i32x4 i32x4;
typedef __attribute__((address_space(3))) uint32_t* lds_u32_ptr;


__device__ inline i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = (int32_t)(uint32_t)a;
  r[1] = (int32_t)((uint32_t)(a >> 32) & 0xFFFFu);  // stride 0: raw byte buffer
  r[2] = (int32_t)bytes;                             // num_records (bytes)
  r[3] = 0x00020000;                                 // gfx9 buffer format word
  return r;
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt split over bits 3:0 and 15:14,
// expcnt and lgkmcnt left at "no wait").
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}


// Workgroup barrier for kernels that count their own LDS-DMA copies with
// wait_vmem: it waits for this wave's LDS reads and writes only.  (A
// __syncthreads() also drains every vector-memory operation in flight, copies
// meant to land a few iterations later included.)  The "memory" clobber keeps
// the compiler from moving LDS accesses across it.
__device__ inline void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming stores, for results that the same launch never reads back: the
// nontemporal hint (global_store ... nt) keeps them from displacing inputs
// that are still being re-read through the caches.  Measured on one MI355X:
// NVFP4 quantization of the 8192 x 17408 MLP activation 77 -> 66 us, bf16
// GEMM outputs about 1 %, FP8 KV-cache write of 32768 x 1024 bf16 21.7 ->
// 20.0 us (16 rotating buffers, so no input is left in the last-level
// cache).  The hint is IR metadata that a rewrite of the store can lose, so
// the build tests look for the nt stores in the code objects.
__device__ inline void store_stream16(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4 v = {a, b, c, d};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ inline void store_stream8(void* p, uint32_t a, uint32_t b) {
  const u32x2 v = {a, b};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}
__device__ inline void store_stream1(uint8_t* p, uint8_t v) { __builtin_nontemporal_store(v, p); }

// E4M3 byte b -> the fp16 pair (s * 2^-8, s * 2^-8), exact: b shifted into
// an fp16's exponent/mantissa fields is s * 2^-8 (normal and subnormal
// alike).  decode8 converts the codes with a 2^8 scale, so the product is
// code * s with no separate correction.
__device__ inline half2v scale_pair(uint32_t sdw, int idx) {
  const uint32_t b = (sdw >> (8 * idx)) & 0xFFu;
  return __builtin_bit_cast(half2v, (b << 7) | (b << 23));
}

// 8 E2M1 codes (one dword) times their block scale -> 8 exact fp16 values:
// the conversion applies the exponent of its float32 scale operand, so the
// codes come out times 2^8 (at most 1536, exact), and one fp16 multiply by
// s * 2^-8 from scale_pair gives code * s (<= 5 significant bits, at least
// 2^-10: exact and normal).
__device__ inline half8 decode8(uint32_t codes, half2v s2) {
  half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 0);
  half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 1);
  half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 2);
  half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 256.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  half8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Map the linear workgroup id to an output tile.  Workgroups are dealt to
// the 8 XCDs round-robin; renumber them so each XCD works on a contiguous
// range of tiles (sharing its L2), then walk that range in column-major
// groups of kGroupM tile rows so neighbours share A and W panels.
__device__ inline void tile_of(int bid, int nblocks, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int kXcd = 8, kGroupM = 8;
  const int q = nblocks / kXcd, r = nblocks % kXcd;
  const int x = bid % kXcd, slot = bid / kXcd;
  const int l = x * q + min(x, r) + slot;
  const int group_size = kGroupM * tiles_n;
  const int group = l / group_size;
  const int first_m = group * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int in = l - group * group_size;
  tm = first_m + in % gm;
  tn = in / gm;
}

// float -> bf16 bits, round to nearest even, with gfx950's conversion
// instruction (v_cvt_pk_bf16_f32; checked on the device against the integer
// rounding (u + 0x7FFF + lsb) >> 16, ties and subnormals included).
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two floats -> packed bf16 (a in the low half) with gfx950's conversion
// instruction: round to nearest even, the same as f32_to_bf16_bits for every
// finite input (checked on the device, ties and subnormals included).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// silu(u) = u * sigmoid(u), with sigmoid evaluated without overflow.  The
// SiLU*mul kernel and the fused gate_up epilogue both call this one
// definition, so their bf16 results agree bit for bit.  e = exp(-|u|) comes
// from the hardware exp2 (v_exp_f32) and 1 / (1 + e) from the hardware
// reciprocal: a few float32 ulps, negligible against the bf16 rounding of
// the result.  Below 2^-126 the exp2 argument is lifted by 64 and the result
// scaled back by 2^-64, one rounding into the subnormal range.
__device__ inline float silu(float u) {
  const float t = -fabsf(u) * 1.44269504088896341f;  // log2(e)
  const bool tiny = t < -126.0f;
  const float e = __builtin_amdgcn_exp2f(tiny ? t + 64.0f : t) * (tiny ? 0x1p-64f : 1.0f);
  const float r = __builtin_amdgcn_rcpf(1.0f + e);
  return u * (u >= 0.0f ? r : e * r);
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// GDN gate epilogue on one scaled fp32 accumulator x (chatpaper.ai English
// abstract, mechanism (ii): sigmoid write strength, log-space
// softplus/exponential decay).  kind 1: sigmoid(x); kind 2:
// -exp_alog * softplus(x + dtb) with exp_alog = exp(A_log[h]); else x.
// Both share e = exp(-|t|): sigmoid(t) = (t >= 0 ? 1 : e) / (1 + e) and
// softplus(t) = max(t, 0) + log1p(e).  Each piece below is within a few
// float32 ulps (relative), all on full-rate or single transcendental
// instructions.

// exp(-a) for a >= 0, as es * 2^-64 when tiny (below 2^-126) and es
// otherwise.  a * log2(e) is split into its float32 rounding p and the
// remainder d (the fma gives the rounding error exactly, plus a times the
// constant's own tail), and 2^p from the hardware exp2 is corrected to first
// order: 2^(p + d) = 2^p (1 + d ln 2).  For |p| <= 190 (below that the
// result is zero) |d| < 2^-16, so the dropped second-order term is below
// 2^-33.  Tiny results are computed from the argument lifted by 64, so es
// stays a normal number; contraction is off so that the lifted argument is
// p + 64 exactly, not a fused a * log2(e) + 64.
struct ExpNeg {
  float es;
  bool tiny;
  __device__ float value() const { return tiny ? es * 0x1p-64f : es; }  // one rounding
};
__device__ inline ExpNeg exp_neg(float a) {
#pragma clang fp contract(off)
  const float kLog2e = 1.44269502162933349609375f;  // float32 nearest log2(e)
  const float kLog2eTail = 1.925963033500011e-08f;  // log2(e) - kLog2e
  const float p = -a * kLog2e;
  const float d = fmaf(-a, kLog2e, -p) - a * kLog2eTail;
  const bool tiny = p < -126.0f;
  const float e0 = __builtin_amdgcn_exp2f(tiny ? p + 64.0f : p);
  return {fmaf(e0, d * 0.693147180559945309f, e0), tiny};
}

// n / d for d in [1, 3]: hardware reciprocal, then one Newton correction of
// the quotient (error within ~1 ulp).
__device__ inline float div_small(float n, float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = n * r;
  return fmaf(fmaf(-d, q, n), r, q);
}

// log1p(e) for e in [0, 1]: 2 atanh(s) with s = e / (2 + e) in [0, 1/3],
// 2 s (1 + z/3 + z^2/5 + ... + z^7/15) with z = s^2 <= 1/9; the first
// omitted term is below 2^-28 of the sum.
__device__ inline float log1p_unit(float e) {
  const float s = div_small(e, 2.0f + e);
  const float z = s * s;
  float q = 1.0f / 15.0f;
  q = fmaf(q, z, 1.0f / 13.0f);
  q = fmaf(q, z, 1.0f / 11.0f);
  q = fmaf(q, z, 1.0f / 9.0f);
  q = fmaf(q, z, 1.0f / 7.0f);
  q = fmaf(q, z, 1.0f / 5.0f);
  q = fmaf(q, z, 1.0f / 3.0f);
  q = fmaf(q * z, 2.0f * s, 2.0f * s);
  return q;
}

// sigmoid: for a tiny e the quotient is e itself (one rounding in value()).
__device__ inline float sigmoid_from(float t, ExpNeg en) {
  const float e = en.value();
  return div_small(t >= 0.0f ? 1.0f : e, 1.0f + e);
}
// decay: with e below 2^-126, log1p(e) is e to float32 precision; for t < 0
// the result -exp_alog * e is formed from the lifted es and rounded into the
// subnormal range once (a subnormal e times exp_alog would scale its
// rounding error by exp_alog); for t > 0 it is -exp_alog * t.
__device__ inline float decay_from(float t, ExpNeg en, float exp_alog) {
  if (en.tiny) return t > 0.0f ? -exp_alog * t : (-exp_alog * en.es) * 0x1p-64f;
  return -exp_alog * (fmaxf(t, 0.0f) + log1p_unit(en.es));
}

__device__ inline float gate_value(float x, int kind, float exp_alog, float dtb) {
  const float t = kind == 2 ? x + dtb : x;
  const ExpNeg en = exp_neg(fabsf(t));
  return kind == 1 ? sigmoid_from(t, en) : (kind == 2 ? decay_from(t, en, exp_alog) : x);
}

}  // namespace dev
}  // namespace nvfp4
