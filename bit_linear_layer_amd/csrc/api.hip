// C ABI of the NVFP4 W4A4 library: argument validation (before any HIP
// call) and dispatch to the kernels' launchers.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "internal.h"
#include "nvfp4.h"

using namespace nvfp4;

namespace {

constexpr int64_t kIndexLimit = (int64_t)1 << 31;  // kernels index rows/cols with int

thread_local char g_hip_msg[256] = "";

int hip_status(hipError_t e) {
  if (e == hipSuccess) return NVFP4_OK;
  snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return NVFP4_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int check_tensor(const nvfp4_tensor* t) {
  if (t == nullptr || t->codes == nullptr || t->scales == nullptr) return NVFP4_ERR_NULL;
  if (t->rows <= 0 || t->cols <= 0 || t->cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (t->rows >= kIndexLimit || t->cols >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (t->ld_codes < t->cols / 2 || t->ld_codes % 16 != 0) return NVFP4_ERR_STRIDE;
  if (t->ld_scales < t->cols / 16 || t->ld_scales % 8 != 0) return NVFP4_ERR_STRIDE;
  // the GEMM kernels address an operand's code and scale bytes with 32-bit
  // offsets (and bound their buffer loads by the operand's byte size)
  if (t->rows * t->ld_codes >= kIndexLimit || t->rows * t->ld_scales >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 8)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int check_out(const void* out, int out_dtype, int64_t ld_out, int64_t n) {
  if (out == nullptr) return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (ld_out < n) return NVFP4_ERR_STRIDE;
  if (!aligned(out, out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

// Segment table and gate of a fused GEMM into the epilogue arguments.
int fill_segments(int n_segments, const int64_t* seg_offsets, const float* seg_global_scales,
                  const nvfp4_gdn_gate* gate, int64_t n, EpilogueArgs& ep) {
  if (n_segments < 1 || n_segments > NVFP4_MAX_SEGMENTS) return NVFP4_ERR_SEGMENTS;
  if (seg_offsets == nullptr || seg_global_scales == nullptr) return NVFP4_ERR_NULL;
  if (seg_offsets[0] != 0 || seg_offsets[n_segments] != n) return NVFP4_ERR_SEGMENTS;
  for (int s = 0; s < n_segments; ++s)
    if (seg_offsets[s + 1] <= seg_offsets[s]) return NVFP4_ERR_SEGMENTS;
  ep.n_seg = n_segments;
  for (int s = 0; s <= n_segments; ++s) ep.seg_off[s] = (int)seg_offsets[s];
  ep.seg_g = seg_global_scales;
  ep.b_seg = -1;
  ep.a_seg = -1;
  if (gate != nullptr) {
    const int bs = gate->b_segment, as = gate->a_segment;
    if (bs < -1 || bs >= n_segments || as < -1 || as >= n_segments) return NVFP4_ERR_GATE;
    if (bs >= 0 && bs == as) return NVFP4_ERR_GATE;
    if (as >= 0 && (gate->A_log == nullptr || gate->dt_bias == nullptr)) return NVFP4_ERR_GATE;
    ep.b_seg = bs;
    ep.a_seg = as;
    ep.A_log = gate->A_log;
    ep.dt_bias = gate->dt_bias;
  }
  return NVFP4_OK;
}

int check_decode_weight(const nvfp4_decode_weight* w) {
  if (w == nullptr || w->data == nullptr) return NVFP4_ERR_NULL;
  if (w->rows <= 0 || w->cols <= 0 || w->cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (w->rows >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (w->cols > kDecodeMaxK) return NVFP4_ERR_SHAPE;
  if (!aligned(w->data, 16)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

}  // namespace

namespace nvfp4 {

int quantize_check(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, const uint8_t* codes,
                   int64_t ld_codes, const uint8_t* scales, int64_t ld_scales, const float* global_scale,
                   int flags) {
  if (x == nullptr || codes == nullptr || scales == nullptr || global_scale == nullptr)
    return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (flags != NVFP4_SCALE_DYNAMIC && flags != NVFP4_SCALE_STATIC && flags != NVFP4_AMAX_PRECOMPUTED)
    return NVFP4_ERR_FLAGS;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit) return NVFP4_ERR_RANGE;
  const int esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ld_x < cols || (ld_x * esz) % 16 != 0) return NVFP4_ERR_STRIDE;
  if (ld_codes < cols / 2 || ld_codes % 8 != 0) return NVFP4_ERR_STRIDE;
  if (ld_scales < cols / 16) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(codes, 8) || !aligned(global_scale, 4)) return NVFP4_ERR_ALIGN;
  return NVFP4_OK;
}

int quantize_launch(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* codes,
                    int64_t ld_codes, uint8_t* scales, int64_t ld_scales, float* global_scale, int flags,
                    float* partials, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int np = partial_count(rows, cols, 16);
  if (flags == NVFP4_SCALE_DYNAMIC && rows * (cols / 16) <= kFusedQuantBlocks)
    return hip_status(launch_quantize(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales,
                                      ld_scales, global_scale, 2, partials, np, s));
  if (flags == NVFP4_SCALE_DYNAMIC) {
    const int st = hip_status(launch_amax(x, x_dtype, rows, cols, ld_x, partials, np, s));
    if (st != NVFP4_OK) return st;
  }
  return hip_status(launch_quantize(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales,
                                    ld_scales, global_scale, flags == NVFP4_SCALE_STATIC ? 1 : 0,
                                    partials, np, s));
}

int status_from_hip(hipError_t e) { return hip_status(e); }

}  // namespace nvfp4

extern "C" {

size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols < 16) return sizeof(float);
  return sizeof(float) * (size_t)partial_count(rows, cols, 16);
}

int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                   float* global_scale, int flags, void* workspace, size_t workspace_bytes,
                   void* stream) {
  const int st = quantize_check(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales, ld_scales,
                                global_scale, flags);
  if (st != NVFP4_OK) return st;
  if (flags != NVFP4_SCALE_STATIC) {
    if (workspace == nullptr) return NVFP4_ERR_WORKSPACE;
    if (workspace_bytes < nvfp4_quantize_workspace_bytes(rows, cols)) return NVFP4_ERR_WORKSPACE;
    if (!aligned(workspace, 4)) return NVFP4_ERR_ALIGN;
  }
  return quantize_launch(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales, ld_scales, global_scale,
                         flags, (float*)workspace, stream);
}

int nvfp4_gemm_fused_segments(const nvfp4_tensor* a, const nvfp4_tensor* w, int n_segments,
                              const int64_t* seg_offsets, const float* seg_global_scales,
                              const nvfp4_gdn_gate* gate, void* out, int out_dtype, int64_t ld_out,
                              void* stream) {
  int st = check_tensor(a);
  if (st != NVFP4_OK) return st;
  st = check_tensor(w);
  if (st != NVFP4_OK) return st;
  if (a->global_scale == nullptr) return NVFP4_ERR_NULL;
  if (a->cols != w->cols) return NVFP4_ERR_SHAPE;
  st = check_out(out, out_dtype, ld_out, w->rows);
  if (st != NVFP4_OK) return st;
  if (n_segments < 1 || n_segments > NVFP4_MAX_SEGMENTS) return NVFP4_ERR_SEGMENTS;
  if (seg_offsets == nullptr || seg_global_scales == nullptr) return NVFP4_ERR_NULL;
  if (seg_offsets[0] != 0 || seg_offsets[n_segments] != w->rows) return NVFP4_ERR_SEGMENTS;
  for (int s = 0; s < n_segments; ++s)
    if (seg_offsets[s + 1] <= seg_offsets[s]) return NVFP4_ERR_SEGMENTS;

  GemmArgs p{};
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.lda_c = a->ld_codes;
  p.lda_s = a->ld_scales;
  p.w_codes = w->codes;
  p.w_scales = w->scales;
  p.ldw_c = w->ld_codes;
  p.ldw_s = w->ld_scales;
  p.out = out;
  p.ld_out = ld_out;
  p.out_bf16 = out_dtype == NVFP4_DTYPE_BF16;
  p.M = (int)a->rows;
  p.N = (int)w->rows;
  p.K = (int)a->cols;
  p.ep.n_seg = n_segments;
  for (int s = 0; s <= n_segments; ++s) p.ep.seg_off[s] = (int)seg_offsets[s];
  p.ep.seg_g = seg_global_scales;
  p.ep.a_g = a->global_scale;
  p.ep.b_seg = -1;
  p.ep.a_seg = -1;
  if (gate != nullptr) {
    const int bs = gate->b_segment, as = gate->a_segment;
    if (bs < -1 || bs >= n_segments || as < -1 || as >= n_segments) return NVFP4_ERR_GATE;
    if (bs >= 0 && bs == as) return NVFP4_ERR_GATE;
    if (as >= 0 && (gate->A_log == nullptr || gate->dt_bias == nullptr)) return NVFP4_ERR_GATE;
    p.ep.b_seg = bs;
    p.ep.a_seg = as;
    p.ep.A_log = gate->A_log;
    p.ep.dt_bias = gate->dt_bias;
  }
  return hip_status(launch_gemm(p, (hipStream_t)stream));
}

int nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* w, void* out, int out_dtype,
               int64_t ld_out, void* stream) {
  int st = check_tensor(w);
  if (st != NVFP4_OK) return st;
  if (w->global_scale == nullptr) return NVFP4_ERR_NULL;
  const int64_t offs[2] = {0, w->rows};
  return nvfp4_gemm_fused_segments(a, w, 1, offs, w->global_scale, nullptr, out, out_dtype,
                                   ld_out, stream);
}

int nvfp4_gemm_swiglu(const nvfp4_tensor* a, const nvfp4_tensor* w_gate_up,
                      const float* seg_global_scales, void* h, int64_t ld_h,
                      void* amax_workspace, size_t workspace_bytes, const nvfp4_tensor* h_q,
                      void* stream) {
  int st = check_tensor(a);
  if (st != NVFP4_OK) return st;
  st = check_tensor(w_gate_up);
  if (st != NVFP4_OK) return st;
  if (a->global_scale == nullptr || seg_global_scales == nullptr) return NVFP4_ERR_NULL;
  if (h == nullptr && h_q == nullptr) return NVFP4_ERR_NULL;
  if (a->cols != w_gate_up->cols || w_gate_up->rows % 2 != 0) return NVFP4_ERR_SHAPE;
  const int64_t inter = w_gate_up->rows / 2;
  if (inter % 16 != 0) return NVFP4_ERR_SHAPE;
  if (h != nullptr) {
    if (ld_h < inter || ld_h % 8 != 0) return NVFP4_ERR_STRIDE;
    if (!aligned(h, 16)) return NVFP4_ERR_ALIGN;
  }
  if (h_q != nullptr) {
    st = check_tensor(h_q);
    if (st != NVFP4_OK) return st;
    if (h_q->global_scale == nullptr) return NVFP4_ERR_NULL;
    if (h_q->rows != a->rows || h_q->cols != inter) return NVFP4_ERR_SHAPE;
  }
  const int np = partial_count(a->rows, inter, 16);
  if (amax_workspace != nullptr) {
    if (workspace_bytes < sizeof(float) * (size_t)np) return NVFP4_ERR_WORKSPACE;
    if (!aligned(amax_workspace, 4)) return NVFP4_ERR_ALIGN;
  }

  GemmArgs p{};
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.lda_c = a->ld_codes;
  p.lda_s = a->ld_scales;
  p.w_codes = w_gate_up->codes;
  p.w_scales = w_gate_up->scales;
  p.ldw_c = w_gate_up->ld_codes;
  p.ldw_s = w_gate_up->ld_scales;
  p.M = (int)a->rows;
  p.N = (int)w_gate_up->rows;
  p.K = (int)a->cols;
  p.ep.n_seg = 2;
  p.ep.seg_off[0] = 0;
  p.ep.seg_off[1] = (int)inter;
  p.ep.seg_off[2] = (int)(2 * inter);
  p.ep.seg_g = seg_global_scales;
  p.ep.a_g = a->global_scale;
  p.ep.b_seg = -1;
  p.ep.a_seg = -1;
  p.ep.inter = (int)inter;
  p.ep.h = (uint16_t*)h;
  p.ep.ld_h = ld_h;
  if (h_q != nullptr) {
    p.ep.hq_codes = const_cast<uint8_t*>(h_q->codes);  // an output here
    p.ep.hq_scales = const_cast<uint8_t*>(h_q->scales);
    p.ep.hq_ld_codes = h_q->ld_codes;
    p.ep.hq_ld_scales = h_q->ld_scales;
    p.ep.hq_g = h_q->global_scale;
  }
  p.ep.partials = (float*)amax_workspace;
  p.ep.n_partials = np;
  return hip_status(launch_gemm_swiglu(p, (hipStream_t)stream));
}

int nvfp4_silu_mul(const void* gu, int64_t rows, int64_t inter, int64_t ld_gu, void* h,
                   int64_t ld_h, void* amax_workspace, size_t workspace_bytes, void* stream) {
  if (gu == nullptr || h == nullptr) return NVFP4_ERR_NULL;
  if (rows <= 0 || inter <= 0 || inter % 8 != 0) return NVFP4_ERR_SHAPE;
  if (rows >= kIndexLimit || inter >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (ld_gu < 2 * inter || ld_gu % 8 != 0 || ld_h < inter || ld_h % 8 != 0) return NVFP4_ERR_STRIDE;
  if (!aligned(gu, 16) || !aligned(h, 16)) return NVFP4_ERR_ALIGN;
  // Same partial count as a quantize of h (which needs inter % 16 == 0).
  const int np = partial_count(rows, inter, 16);
  if (amax_workspace != nullptr) {
    if (inter % 16 != 0) return NVFP4_ERR_SHAPE;
    if (workspace_bytes < sizeof(float) * (size_t)np) return NVFP4_ERR_WORKSPACE;
    if (!aligned(amax_workspace, 4)) return NVFP4_ERR_ALIGN;
  }
  return hip_status(launch_silu_mul((const uint16_t*)gu, rows, inter, ld_gu, (uint16_t*)h, ld_h,
                                    (float*)amax_workspace, np, (hipStream_t)stream));
}

int nvfp4_kv_fp8_calibrate(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           float* scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (x == nullptr || scale == nullptr || workspace == nullptr) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit) return NVFP4_ERR_RANGE;
  const int esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ld_x < cols || (ld_x * esz) % 16 != 0) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(scale, 4) || !aligned(workspace, 4)) return NVFP4_ERR_ALIGN;
  const int np = partial_count(rows, cols, 16);
  if (workspace_bytes < sizeof(float) * (size_t)np) return NVFP4_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int st = hip_status(launch_amax(x, x_dtype, rows, cols, ld_x, (float*)workspace, np, s));
  if (st != NVFP4_OK) return st;
  return hip_status(launch_kv_scale((const float*)workspace, np, scale, s));
}

int nvfp4_kv_fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                          const int64_t* slots, int64_t cache_rows, uint8_t* cache, int64_t ld_cache,
                          const float* scale, void* stream) {
  if (x == nullptr || cache == nullptr || scale == nullptr) return NVFP4_ERR_NULL;
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || cache_rows <= 0) return NVFP4_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit || cache_rows >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (slots == nullptr && cache_rows < rows) return NVFP4_ERR_SHAPE;
  const int esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ld_x < cols || (ld_x * esz) % 16 != 0) return NVFP4_ERR_STRIDE;
  if (ld_cache < cols || ld_cache % 8 != 0) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(cache, 8) || !aligned(scale, 4) || !aligned(slots, 8))
    return NVFP4_ERR_ALIGN;
  return hip_status(launch_kv_quantize(x, x_dtype, rows, cols, ld_x, slots, cache_rows, cache, ld_cache,
                                       scale, (hipStream_t)stream));
}

int nvfp4_kv_fp8_dequantize(const uint8_t* cache, int64_t rows, int64_t cols, int64_t ld_cache,
                            const float* scale, void* out, int out_dtype, int64_t ld_out,
                            void* stream) {
  if (cache == nullptr || scale == nullptr || out == nullptr) return NVFP4_ERR_NULL;
  if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (rows >= kIndexLimit || cols >= kIndexLimit) return NVFP4_ERR_RANGE;
  const int esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ld_cache < cols || ld_cache % 8 != 0) return NVFP4_ERR_STRIDE;
  if (ld_out < cols || (ld_out * esz) % 16 != 0) return NVFP4_ERR_STRIDE;
  if (!aligned(cache, 8) || !aligned(scale, 4) || !aligned(out, 16)) return NVFP4_ERR_ALIGN;
  return hip_status(launch_kv_dequantize(cache, rows, cols, ld_cache, scale, out, out_dtype, ld_out,
                                         (hipStream_t)stream));
}

int nvfp4_harmonize_scales(const nvfp4_tensor* w, int n_segments, const int64_t* seg_offsets,
                           const float* seg_global_scales, uint8_t* out_scales,
                           int64_t ld_out_scales, float* out_global_scale, void* stream) {
  if (w == nullptr || w->scales == nullptr) return NVFP4_ERR_NULL;
  if (seg_offsets == nullptr || seg_global_scales == nullptr || out_scales == nullptr ||
      out_global_scale == nullptr)
    return NVFP4_ERR_NULL;
  if (w->rows <= 0 || w->cols <= 0 || w->cols % 16 != 0) return NVFP4_ERR_SHAPE;
  if (w->rows >= kIndexLimit || w->cols >= kIndexLimit) return NVFP4_ERR_RANGE;
  if (w->ld_scales < w->cols / 16 || ld_out_scales < w->cols / 16) return NVFP4_ERR_STRIDE;
  if (!aligned(out_global_scale, 4)) return NVFP4_ERR_ALIGN;
  if (n_segments < 1 || n_segments > NVFP4_MAX_SEGMENTS) return NVFP4_ERR_SEGMENTS;
  if (seg_offsets[0] != 0 || seg_offsets[n_segments] != w->rows) return NVFP4_ERR_SEGMENTS;
  SegmentTable seg{};
  seg.n = n_segments;
  for (int s = 0; s <= n_segments; ++s) {
    if (s > 0 && seg_offsets[s] <= seg_offsets[s - 1]) return NVFP4_ERR_SEGMENTS;
    seg.off[s] = seg_offsets[s];
  }
  return hip_status(launch_harmonize(w->scales, w->ld_scales, out_scales, ld_out_scales, w->rows,
                                     w->cols / 16, seg, seg_global_scales, out_global_scale,
                                     (hipStream_t)stream));
}

size_t nvfp4_gdn_workspace_bytes(int64_t tokens, int v_heads) {
  if (tokens <= 0 || v_heads <= 0) return 0;
  return sizeof(float) * gdn_workspace_floats(tokens, v_heads);
}

int nvfp4_gdn_recurrence(const nvfp4_gdn_inputs* in, int in_dtype, int64_t tokens, int k_heads,
                         int v_heads, int normalize_qk, const float* s0, float* s_final, void* o,
                         int o_dtype, int64_t ld_o, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (in == nullptr || in->q == nullptr || in->k == nullptr || in->v == nullptr ||
      in->beta == nullptr || in->g == nullptr || o == nullptr || workspace == nullptr)
    return NVFP4_ERR_NULL;
  if (in_dtype != NVFP4_DTYPE_BF16 && in_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (o_dtype != NVFP4_DTYPE_BF16 && o_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (tokens <= 0 || k_heads <= 0 || v_heads <= 0 || v_heads % k_heads != 0 || v_heads > 4096)
    return NVFP4_ERR_SHAPE;
  if (tokens >= kIndexLimit) return NVFP4_ERR_RANGE;
  const int64_t kw = (int64_t)k_heads * 128, vw = (int64_t)v_heads * 128;
  if (in->ld_q < kw || in->ld_k < kw || in->ld_v < vw || in->ld_beta < v_heads || in->ld_g < v_heads ||
      ld_o < vw)
    return NVFP4_ERR_STRIDE;
  const uintptr_t ea = in_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if ((in->ld_q * (int64_t)ea) % 16 != 0 || (in->ld_k * (int64_t)ea) % 16 != 0 ||
      (in->ld_v * (int64_t)ea) % 16 != 0)
    return NVFP4_ERR_STRIDE;  // q, k, v rows are read with 16-byte loads
  if (!aligned(in->q, 16) || !aligned(in->k, 16) || !aligned(in->v, 16) || !aligned(in->beta, ea) ||
      !aligned(in->g, ea) || !aligned(o, o_dtype == NVFP4_DTYPE_BF16 ? 2 : 4) || !aligned(workspace, 16) ||
      !aligned(s0, 4) || !aligned(s_final, 4))
    return NVFP4_ERR_ALIGN;
  if (workspace_bytes < nvfp4_gdn_workspace_bytes(tokens, v_heads)) return NVFP4_ERR_WORKSPACE;
  GdnArgs p{};
  p.q = in->q; p.ld_q = in->ld_q;
  p.k = in->k; p.ld_k = in->ld_k;
  p.v = in->v; p.ld_v = in->ld_v;
  p.beta = in->beta; p.ld_beta = in->ld_beta;
  p.g = in->g; p.ld_g = in->ld_g;
  p.in_dtype = in_dtype;
  p.T = tokens;
  p.hk = k_heads;
  p.hv = v_heads;
  p.n_chunks = (int)((tokens + 63) / 64);
  p.normalize = normalize_qk != 0;
  p.s0 = s0;
  p.s_final = s_final;
  p.o = o;
  p.ld_o = ld_o;
  p.o_dtype = o_dtype;
  return hip_status(launch_gdn(p, (float*)workspace, (hipStream_t)stream));
}

size_t nvfp4_decode_weight_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || cols > kDecodeMaxK || rows >= kIndexLimit) return 0;
  return decode_weight_bytes(rows, cols);
}

int nvfp4_decode_weight_pack(const nvfp4_tensor* w, void* packed, size_t packed_bytes, void* stream) {
  const int st = check_tensor(w);
  if (st != NVFP4_OK) return st;
  if (packed == nullptr) return NVFP4_ERR_NULL;
  if (w->cols > kDecodeMaxK) return NVFP4_ERR_SHAPE;
  if (!aligned(packed, 16)) return NVFP4_ERR_ALIGN;
  if (packed_bytes < decode_weight_bytes(w->rows, w->cols)) return NVFP4_ERR_WORKSPACE;
  return hip_status(launch_decode_pack(w->codes, w->ld_codes, w->scales, w->ld_scales, (int)w->rows,
                                       (int)w->cols, (uint8_t*)packed, (hipStream_t)stream));
}

int nvfp4_gemm_decode(const nvfp4_tensor* a, const nvfp4_decode_weight* w, int n_segments,
                      const int64_t* seg_offsets, const float* seg_global_scales, const nvfp4_gdn_gate* gate,
                      void* out, int out_dtype, int64_t ld_out, void* stream) {
  int st = check_tensor(a);
  if (st != NVFP4_OK) return st;
  st = check_decode_weight(w);
  if (st != NVFP4_OK) return st;
  if (a->global_scale == nullptr) return NVFP4_ERR_NULL;
  if (a->cols != w->cols || a->rows > kDecodeMaxM) return NVFP4_ERR_SHAPE;
  st = check_out(out, out_dtype, ld_out, w->rows);
  if (st != NVFP4_OK) return st;
  GemmArgs p{};
  st = fill_segments(n_segments, seg_offsets, seg_global_scales, gate, w->rows, p.ep);
  if (st != NVFP4_OK) return st;
  p.a_codes = a->codes;
  p.a_scales = a->scales;
  p.lda_c = a->ld_codes;
  p.lda_s = a->ld_scales;
  p.ep.a_g = a->global_scale;
  p.out = out;
  p.ld_out = ld_out;
  p.out_bf16 = out_dtype == NVFP4_DTYPE_BF16;
  p.M = (int)a->rows;
  p.N = (int)w->rows;
  p.K = (int)w->cols;
  return hip_status(launch_gemm_decode(p, (const uint8_t*)w->data, nullptr, 0, 0, nullptr, p.ep.b_seg >= 0 ||
                                       p.ep.a_seg >= 0, (hipStream_t)stream));
}

int nvfp4_linear_decode(const void* x, int x_dtype, int64_t rows, int64_t ld_x, float* x_global_scale,
                        const nvfp4_decode_weight* w, int n_segments, const int64_t* seg_offsets,
                        const float* seg_global_scales, const nvfp4_gdn_gate* gate, void* out, int out_dtype,
                        int64_t ld_out, void* stream) {
  if (x == nullptr) return NVFP4_ERR_NULL;
  int st = check_decode_weight(w);
  if (st != NVFP4_OK) return st;
  if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_F32) return NVFP4_ERR_DTYPE;
  if (rows <= 0 || rows > kDecodeMaxM) return NVFP4_ERR_SHAPE;
  const int esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
  if (ld_x < w->cols || (ld_x * esz) % 16 != 0) return NVFP4_ERR_STRIDE;
  if (!aligned(x, 16) || !aligned(x_global_scale, 4)) return NVFP4_ERR_ALIGN;
  st = check_out(out, out_dtype, ld_out, w->rows);
  if (st != NVFP4_OK) return st;
  GemmArgs p{};
  st = fill_segments(n_segments, seg_offsets, seg_global_scales, gate, w->rows, p.ep);
  if (st != NVFP4_OK) return st;
  p.out = out;
  p.ld_out = ld_out;
  p.out_bf16 = out_dtype == NVFP4_DTYPE_BF16;
  p.M = (int)rows;
  p.N = (int)w->rows;
  p.K = (int)w->cols;
  return hip_status(launch_gemm_decode(p, (const uint8_t*)w->data, x, x_dtype, ld_x, x_global_scale,
                                       p.ep.b_seg >= 0 || p.ep.a_seg >= 0, (hipStream_t)stream));
}

const char* nvfp4_status_string(int status) {
  switch (status) {
    case NVFP4_OK: return "ok";
    case NVFP4_ERR_NULL: return "a required pointer is NULL";
    case NVFP4_ERR_SHAPE: return "bad shape (rows/cols must be > 0, cols % 16 == 0, K must match)";
    case NVFP4_ERR_DTYPE: return "unknown dtype code";
    case NVFP4_ERR_STRIDE: return "leading dimension too small or not a multiple of the required alignment";
    case NVFP4_ERR_ALIGN: return "base pointer misaligned";
    case NVFP4_ERR_SEGMENTS: return "bad segment table";
    case NVFP4_ERR_GATE: return "bad gate specification";
    case NVFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case NVFP4_ERR_FLAGS: return "unknown flags";
    case NVFP4_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP error";
    case NVFP4_ERR_RANGE: return "size beyond 2^31";
    default: return "unknown status";
  }
}

int nvfp4_version(void) { return 100; }

}  // extern "C"
