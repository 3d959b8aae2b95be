// Internal declarations shared by the kernels' launchers and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4.h"

namespace nvfp4 {

// Amax partials: one float per workgroup of the amax pass (or of the fused
// SiLU*mul kernel), reduced again by every workgroup of the quantize pass.
constexpr int kMaxPartials = 1024;
constexpr int kElemThreads = 256;  // workgroup size of the elementwise kernels

// Number of amax partials (= workgroups) used for a [rows, cols] tensor
// walked in chunks of `chunk` elements per thread.
int partial_count(int64_t rows, int64_t cols, int chunk);

hipError_t launch_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                       float* partials, int n_partials, hipStream_t s);

// mode: 0 = dynamic (reduce partials, write *g), 1 = static (read *g),
// 2 = dynamic in one workgroup with the amax pass in the same kernel (small
// tensors: at most kFusedQuantBlocks 16-element blocks; writes the partials
// as the amax kernel would).
constexpr int64_t kFusedQuantBlocks = 4 * kElemThreads;
hipError_t launch_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           float* g, int mode, float* partials, int n_partials,
                           hipStream_t s);

// nvfp4_quantize in two halves (api.hip): every argument check except the
// workspace's, then the launches with the amax partials at `partials`
// (unused for NVFP4_SCALE_STATIC).  nvfp4_quantize_noalloc shares both.
int quantize_check(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, const uint8_t* codes,
                   int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, const float* global_scale,
                   int flags);
int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                    int64_t ld_codes, uint8_t* scales, int64_t ld_scales, float* global_scale, int flags,
                    float* partials, void* stream);
// NVFP4_ERR_HIP for a failed HIP call (its text kept for nvfp4_status_string).
int status_from_hip(hipError_t e);

hipError_t launch_silu_mul(const uint16_t* gu, int64_t rows, int64_t inter, int64_t ld_gu,
                           uint16_t* h, int64_t ld_h, float* partials, int n_partials,
                           hipStream_t s);

struct EpilogueArgs {
  int n_seg;
  int seg_off[NVFP4_MAX_SEGMENTS + 1];  // output-column offsets of the segments
  const float* seg_g;                   // device [n_seg] weight global scales
  const float* a_g;                     // device activation global scale
  int b_seg, a_seg;                     // gate segments, -1 = none
  const float* A_log;
  const float* dt_bias;
  // Gated-MLP epilogue (launch_gemm_swiglu): W rows [0, inter) are the gate,
  // [inter, 2 inter) the up projection; h = bf16(silu(gate) * up).
  int inter;
  uint16_t* h;                 // bf16 [M, inter] or null
  int64_t ld_h;
  uint8_t* hq_codes;           // NVFP4 h with the static global scale *hq_g, or null
  uint8_t* hq_scales;
  int64_t hq_ld_codes, hq_ld_scales;
  const float* hq_g;
  float* partials;             // amax partials of h (atomic max, zeroed first) or null
  int n_partials;
};

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  int64_t lda_c, lda_s;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  int64_t ldw_c, ldw_s;
  void* out;
  int64_t ld_out;
  int out_bf16;
  int M, N, K;
  EpilogueArgs ep;
};

hipError_t launch_gemm(const GemmArgs& args, hipStream_t s);

// Gated-MLP first half in one launch (zeroes ep.partials first when set).
hipError_t launch_gemm_swiglu(const GemmArgs& args, hipStream_t s);

hipError_t launch_zero(float* p, int n, hipStream_t s);

// FP8 (E4M3) KV cache with a per-tensor scale (kv_fp8.hip).
hipError_t launch_kv_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const int64_t* slots, int64_t cache_rows, uint8_t* cache,
                              int64_t ld_cache, const float* scale, hipStream_t s);
hipError_t launch_kv_dequantize(const uint8_t* cache, int64_t rows, int64_t cols, int64_t ld_cache,
                                const float* scale, void* out, int out_dtype, int64_t ld_out,
                                hipStream_t s);
hipError_t launch_kv_scale(const float* partials, int n, float* scale, hipStream_t s);

// Checkpoint-side scale harmonization (harmonize.hip).
struct SegmentTable {
  int n;
  int64_t off[NVFP4_MAX_SEGMENTS + 1];
};
hipError_t launch_harmonize(const uint8_t* in, int64_t ld_in, uint8_t* out, int64_t ld_out,
                            int64_t rows, int64_t bpr, const SegmentTable& seg, const float* seg_g,
                            float* g_out, hipStream_t s);

// Small-M (decode) path over the columns [n_lo, n_hi) when skinny_eligible().
bool skinny_eligible(const GemmArgs& p);
hipError_t launch_gemm_skinny(const GemmArgs& p, int n_lo, int n_hi, bool gate, hipStream_t s);

// Decode GEMM on a weight in the decode layout (gemm_decode.hip): M <= 16,
// K <= kDecodeMaxK.  Activations pre-quantized (g.a_codes, ...) or, with x
// non-null, dense x quantized inside the launch (its dynamic global scale
// written to x_g_out when non-null).
constexpr int64_t kDecodeMaxK = 8192;
constexpr int64_t kDecodeMaxM = 16;
size_t decode_weight_bytes(int64_t N, int64_t K);
hipError_t launch_decode_pack(const uint8_t* codes, int64_t ldc, const uint8_t* scales, int64_t lds, int N, int K,
                              uint8_t* out, hipStream_t s);
hipError_t launch_gemm_decode(const GemmArgs& g, const uint8_t* packed, const void* x, int x_dtype, int64_t ld_x,
                              float* x_g_out, bool gate, hipStream_t s);

// Gated delta-rule recurrence (gdn.hip).
struct GdnArgs {
  const void* q; int64_t ld_q;
  const void* k; int64_t ld_k;
  const void* v; int64_t ld_v;
  const void* beta; int64_t ld_beta;
  const void* g; int64_t ld_g;
  int in_dtype;
  int64_t T;
  int hk, hv, n_chunks, normalize;
  const float* s0;
  float* s_final;
  void* o; int64_t ld_o; int o_dtype;
};
size_t gdn_workspace_floats(int64_t T, int hv);
hipError_t launch_gdn(const GdnArgs& p, float* ws, hipStream_t s);

}  // namespace nvfp4
