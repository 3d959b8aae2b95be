/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 W4A4 linear-layer library.
 *
 * The operations follow one paper, "Why Gated DeltaNet Survives 4-Bit
 * Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM"
 * (arXiv 2609.04098), as the web pages about it describe it:
 *
 *   - NVFP4 stores E2M1 element codes with one E4M3 scale per 16 elements
 *     (evolve.pub review, "Scope & Claims"; thevalue.engineering article,
 *     section on the fragility myth) and one float32 global scale per tensor;
 *   - weights and activations are both 4-bit on every linear layer, so the
 *     activations are quantized on the fly before each GEMM (chatpaper.ai
 *     English abstract; evolve.pub review, "Summary");
 *   - a fused GEMM over several modules keeps each module's global scale
 *     (the fused-GEMM global-scale mismatch of the chatpaper.ai abstract and
 *     the evolve.pub review, "Key claims under review", fourth claim);
 *   - the GDN gates: write strength through a sigmoid, decay through a
 *     log-space softplus/exponential (chatpaper.ai abstract, mechanism (ii)).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  Host
 *     arrays and structs are read only during the call.  The library
 *     allocates no memory and keeps no mutable state between calls apart
 *     from one address per device that nvfp4_quantize_noalloc looks up
 *     once (atomically), so calls from several host threads do not
 *     interfere (calls that write the same device memory still race, as any
 *     two kernels would).
 *   - Every call enqueues work on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns without synchronizing.
 *   - Matrices are row-major.  An NVFP4 matrix [rows, cols] is:
 *       codes  uint8 [rows, ld_codes]  two 4-bit codes per byte, element 2j
 *              in the low nibble of byte j; code = sign<<3 | E2M1 magnitude;
 *       scales uint8 [rows, ld_scales] one E4M3 (OCP "FN") byte per 16
 *              consecutive elements of a row;
 *       global float32, one per tensor (or per weight segment).
 *     An element decodes to (+-)e2m1 * e4m3 * global.
 *   - cols must be a multiple of 16.  Row strides: ld_codes >= cols/2 and a
 *     multiple of 16 bytes, ld_scales >= cols/16 and a multiple of 8 bytes;
 *     code and scale base pointers 16- and 8-byte aligned.  (Dense layouts
 *     satisfy this whenever cols % 128 == 0.)
 *   - Return value: NVFP4_OK (0) or a negative nvfp4_status.  Arguments are
 *     validated before any HIP call; an invalid call enqueues nothing.  A
 *     HIP launch error is returned as NVFP4_ERR_HIP and its text is kept for
 *     nvfp4_status_string.  Device faults surface at the caller's next
 *     synchronization, as in HIP.  Non-finite inputs are outside the
 *     contract (results unspecified).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_ERR_NULL = -1,      /* a required pointer is NULL */
  NVFP4_ERR_SHAPE = -2,     /* rows/cols <= 0, cols % 16 != 0, or mismatched K */
  NVFP4_ERR_DTYPE = -3,     /* unknown dtype code */
  NVFP4_ERR_STRIDE = -4,    /* a leading dimension too small or misaligned */
  NVFP4_ERR_ALIGN = -5,     /* a base pointer misaligned */
  NVFP4_ERR_SEGMENTS = -6,  /* bad segment table */
  NVFP4_ERR_GATE = -7,      /* bad gate specification */
  NVFP4_ERR_WORKSPACE = -8, /* workspace missing or too small */
  NVFP4_ERR_FLAGS = -9,     /* unknown flag bits */
  NVFP4_ERR_HIP = -10,      /* a HIP launch failed */
  NVFP4_ERR_RANGE = -11     /* a size beyond what the kernels index (2^31) */
} nvfp4_status;

/* Element types of dense (non-NVFP4) operands. */
enum { NVFP4_DTYPE_BF16 = 0, NVFP4_DTYPE_F32 = 1 };

/* nvfp4_quantize flags. */
enum {
  NVFP4_SCALE_DYNAMIC = 0,   /* compute g = fl32(amax / (6*448)) on the device and store it */
  NVFP4_SCALE_STATIC = 1,    /* read a caller-provided g from *global_scale (calibrated scale) */
  NVFP4_AMAX_PRECOMPUTED = 2 /* DYNAMIC, but the amax partials are already in the workspace
                                (written by nvfp4_silu_mul); skips the amax pass */
};

/* Most segments a fused GEMM accepts. */
#define NVFP4_MAX_SEGMENTS 16

/* Bytes of device workspace nvfp4_quantize needs for a [rows, cols]
 * input (per-workgroup amax partials).  Always > 0 and <= 4096. */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols);

/*
 * nvfp4_quantize -- NVFP4-quantize a dense matrix (on-the-fly activation
 * quantization; also used offline for weights, one call per module).
 *
 *   x        device, x_dtype elements [rows, ld_x], 16-byte aligned,
 *            ld_x * sizeof(elem) a multiple of 16 bytes.
 *   codes    device uint8 [rows, ld_codes]   (written)
 *   scales   device uint8 [rows, ld_scales]  (written)
 *   global_scale device float32[1]: written (DYNAMIC) or read (STATIC).
 *   workspace device, >= nvfp4_quantize_workspace_bytes(rows, cols) bytes,
 *            4-byte aligned; its contents need no initialization (DYNAMIC
 *            only; may be NULL for STATIC).
 *
 * Result, bit for bit: g = fl32(amax|x| / 2688) (DYNAMIC); per block of 16,
 * scale = E4M3 nearest to the exact amax_block / (6 g) (ties to even code,
 * > 448 saturates, g == 0 or an all-zero block gives 0); per element,
 * magnitude = E2M1 nearest to the exact |x| / (scale * g) (ties to even,
 * > 6 saturates, scale 0 gives 0), sign = IEEE sign bit of x.
 * Two kernel launches (amax pass, quantize pass) on `stream`; one for
 * DYNAMIC with at most 1024 blocks of 16 (the amax pass runs inside the
 * one-workgroup quantize kernel and leaves the workspace as the amax pass
 * would).
 */
int nvfp4_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                   float* global_scale, int flags, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * nvfp4_quantize_noalloc -- nvfp4_quantize for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same arguments and the same result
 * bit for bit, without the workspace.  The amax partials of the dynamic
 * global scale go to a static device array of NVFP4_NOALLOC_SCRATCH_BYTES
 * held by the library on each GPU it runs on until the process ends; that
 * covers every shape nvfp4_quantize accepts (a shape needing more would be
 * rejected with NVFP4_ERR_WORKSPACE).  No call allocates memory.
 *
 *   flags    NVFP4_SCALE_DYNAMIC or NVFP4_SCALE_STATIC;
 *            NVFP4_AMAX_PRECOMPUTED is rejected (NVFP4_ERR_FLAGS): there is
 *            no caller workspace to hold precomputed partials.
 * The first call on a device looks up the array's device address (one
 * hipGetSymbolAddress, kept per device).  All calls on one GPU share the
 * array: two dynamic calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race on it and may produce a
 * wrong global scale.  Calls in one stream are ordered and safe.
 */
#define NVFP4_NOALLOC_SCRATCH_BYTES 4096
int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                           float* global_scale, int flags, void* stream);

/* An NVFP4 operand of a GEMM (all pointers device).  rows * ld_codes and
 * rows * ld_scales must stay below 2^31 bytes (NVFP4_ERR_RANGE otherwise). */
typedef struct {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* global_scale; /* ignored for the weight of nvfp4_gemm_fused_segments */
  int64_t rows, cols;
  int64_t ld_codes, ld_scales;
} nvfp4_tensor;

/*
 * nvfp4_gemm -- W4A4 GEMM out[M, N] = g_a * g_w * sum_k dec(a)[m,k] * dec(w)[n,k]
 * (out = A W^T, as a linear layer), a = activations [M, K], w = weight [N, K].
 *
 *   out      device [M, ld_out] of out_dtype (bf16: round to nearest even).
 * Every decoded operand is exact in fp16; products are exact in fp32 and
 * are accumulated in fp32 (MFMA).  Agrees with the exact result within
 * 1e-5 * sum_k |a*w| per element (plus half a bf16 ulp for bf16 output).
 */
int nvfp4_gemm(const nvfp4_tensor* a, const nvfp4_tensor* w, void* out, int out_dtype,
               int64_t ld_out, void* stream);

/* GDN gate epilogue: columns of segment b_segment become sigmoid(x); columns
 * of segment a_segment become -exp(A_log[h]) * softplus(x + dt_bias[h]),
 * h = column - start of a_segment.  x is the scaled fp32 accumulator; both
 * gates are evaluated in float32 within a few ulps of the exact function of
 * that x (subnormal results within a few 2^-149).
 * Either segment index may be -1 (absent).  A_log and dt_bias are device
 * float32 [width of a_segment]; they may be NULL when a_segment == -1. */
typedef struct {
  int b_segment;
  int a_segment;
  const float* A_log;
  const float* dt_bias;
} nvfp4_gdn_gate;

/*
 * nvfp4_gemm_fused_segments -- one GEMM over a weight made of n_segments
 * row blocks (modules) concatenated along N, each with its own global scale:
 *   out[m, n] = g_a * seg_global_scales[s(n)] * sum_k dec(a)[m,k] * dec(w)[n,k]
 * where s(n) is the segment with seg_offsets[s] <= n < seg_offsets[s+1].
 * This equals the concatenation of one nvfp4_gemm per segment, and is the
 * repair of the global-scale mismatch: no segment is served with another
 * segment's scale.  Then the optional gate epilogue transforms the b/a
 * segment columns in place.
 *
 *   seg_offsets        HOST int64 [n_segments + 1], seg_offsets[0] == 0,
 *                      strictly increasing, seg_offsets[n] == w->rows.
 *   seg_global_scales  DEVICE float32 [n_segments].
 *   gate               HOST pointer, may be NULL (no gate epilogue).
 * 1 <= n_segments <= NVFP4_MAX_SEGMENTS.
 */
int nvfp4_gemm_fused_segments(const nvfp4_tensor* a, const nvfp4_tensor* w, int n_segments,
                              const int64_t* seg_offsets, const float* seg_global_scales,
                              const nvfp4_gdn_gate* gate, void* out, int out_dtype, int64_t ld_out,
                              void* stream);

/*
 * Decode (M <= 16 tokens): the weight streams from HBM once per call, so it
 * is bound by bandwidth, and the row-major layout above (16 rows of one
 * MFMA operand in 16 places) costs the memory path more than the bytes.
 * For this regime a weight is repacked once, offline like its
 * quantization (chatpaper.ai English abstract: weights quantized per
 * module, activations on every call), into the decode layout: for each 16
 * rows and each of 8 K slices, one contiguous unit in which every 1 KB is
 * one wavefront-wide load, already in MFMA operand order.  The layout is
 * internal to this library (its size from nvfp4_decode_weight_bytes); the
 * values are the row-major tensor's codes and scales, zero-padded to whole
 * 16-row groups and K slices.
 */
typedef struct {
  const void* data; /* device, nvfp4_decode_weight_bytes(rows, cols) bytes, 16-byte aligned */
  int64_t rows, cols;
} nvfp4_decode_weight;

/* Bytes of a [rows, cols] weight in the decode layout; 0 for a shape the
 * decode path does not take (cols % 16 != 0 or cols > 8192). */
size_t nvfp4_decode_weight_bytes(int64_t rows, int64_t cols);

/*
 * nvfp4_decode_weight_pack -- write w (row-major NVFP4, as nvfp4_quantize
 * leaves it) into the decode layout at `packed` (device, >=
 * nvfp4_decode_weight_bytes(w->rows, w->cols) bytes, 16-byte aligned;
 * NVFP4_ERR_WORKSPACE if shorter).  w->global_scale is not used: global
 * scales are passed to the GEMM.  cols <= 8192.
 */
int nvfp4_decode_weight_pack(const nvfp4_tensor* w, void* packed, size_t packed_bytes, void* stream);

/*
 * nvfp4_gemm_decode -- nvfp4_gemm_fused_segments for a weight in the decode
 * layout and a->rows <= 16: the same arguments, the same per-segment global
 * scales and gate epilogue, the same exact decode and fp32 MFMA
 * accumulation (outputs agree with nvfp4_gemm_fused_segments within the
 * same 1e-5 * sum|a*w| bound; the summation order differs).
 */
int nvfp4_gemm_decode(const nvfp4_tensor* a, const nvfp4_decode_weight* w, int n_segments,
                      const int64_t* seg_offsets, const float* seg_global_scales,
                      const nvfp4_gdn_gate* gate, void* out, int out_dtype, int64_t ld_out, void* stream);

/*
 * nvfp4_linear_decode -- the whole W4A4 linear layer at decode in one
 * launch: dense activations x [rows, w->cols] (bf16 or float32, rows <= 16,
 * row stride ld_x elements, rows 16-byte aligned) are NVFP4-quantized with
 * their dynamic global scale inside the launch -- codes, scales and g bit
 * for bit those of nvfp4_quantize(x, NVFP4_SCALE_DYNAMIC) -- and multiplied
 * with the packed weight as nvfp4_gemm_decode does; the output is bit for
 * bit that of nvfp4_quantize followed by nvfp4_gemm_decode.
 *   x_global_scale  device float32[1] receiving x's global scale, or NULL.
 * Other arguments as nvfp4_gemm_decode.
 */
int nvfp4_linear_decode(const void* x, int x_dtype, int64_t rows, int64_t ld_x, float* x_global_scale,
                        const nvfp4_decode_weight* w, int n_segments, const int64_t* seg_offsets,
                        const float* seg_global_scales, const nvfp4_gdn_gate* gate, void* out,
                        int out_dtype, int64_t ld_out, void* stream);

/*
 * nvfp4_silu_mul -- MLP glue between the gate_up and down projections:
 *   h[m, j] = bf16( silu(gu[m, j]) * gu[m, inter + j] ),  j < inter,
 * evaluated in fp32 from bf16 inputs, rounded to nearest even.
 *   gu   device bf16 [rows, ld_gu], ld_gu >= 2*inter;  h device bf16 [rows, ld_h].
 *   inter % 8 == 0; ld_gu, ld_h multiples of 8 elements; 16-byte aligned.
 *   amax_workspace: NULL, or a workspace of nvfp4_quantize_workspace_bytes(rows,
 *   inter) bytes that receives the amax partials of h, so that a following
 *   nvfp4_quantize of h with NVFP4_AMAX_PRECOMPUTED skips its amax pass.
 */
int nvfp4_silu_mul(const void* gu, int64_t rows, int64_t inter, int64_t ld_gu, void* h,
                   int64_t ld_h, void* amax_workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_gemm_swiglu -- the first half of a gated MLP in one launch: the
 * gate_up GEMM of nvfp4_gemm_fused_segments with two segments (gate, up),
 * followed in the same kernel by nvfp4_silu_mul's arithmetic.  The pages
 * fix no MLP detail; the gate|up row layout is this library's reading.
 * The static-scale output serves the per-module calibrated checkpoints the
 * pages describe (chatpaper.ai English abstract: per-module-calibrated NVFP4
 * checkpoints served by fused kernels).  The results are bit for bit those
 * of nvfp4_gemm_fused_segments (bf16 out) + nvfp4_silu_mul + nvfp4_quantize,
 * without the bf16 gate_up tensor (and, with h_q, without h) in memory.
 *
 *   a                  activations, [M, K].
 *   w_gate_up          weight, [2*inter, K]: rows [0, inter) are the gate
 *                      projection, rows [inter, 2*inter) the up projection.
 *   seg_global_scales  DEVICE float32 [2]: the gate's and the up
 *                      projection's global scales.
 *   h, ld_h            DEVICE bf16 [M, inter] output with ld_h (elements,
 *                      >= inter, multiple of 8), 16-byte aligned; or NULL.
 *   amax_workspace     NULL, or >= nvfp4_quantize_workspace_bytes(M, inter)
 *                      bytes of device memory (4-byte aligned) receiving the
 *                      amax partials of h, as nvfp4_silu_mul writes them: a
 *                      following nvfp4_quantize of h with
 *                      NVFP4_AMAX_PRECOMPUTED and this workspace computes
 *                      h's dynamic global scale without an amax pass.
 *   h_q                NULL, or an NVFP4 output [M, inter] whose
 *                      global_scale (device) holds a calibrated scale; its
 *                      codes and scales are written as nvfp4_quantize(h,
 *                      NVFP4_SCALE_STATIC) would write them.
 * At least one of h and h_q; inter % 16 == 0; w_gate_up->rows == 2*inter.
 * Errors as nvfp4_gemm_fused_segments, plus NVFP4_ERR_WORKSPACE for a short
 * workspace.
 */
int nvfp4_gemm_swiglu(const nvfp4_tensor* a, const nvfp4_tensor* w_gate_up,
                      const float* seg_global_scales, void* h, int64_t ld_h,
                      void* amax_workspace, size_t workspace_bytes, const nvfp4_tensor* h_q,
                      void* stream);

/*
 * FP8 (E4M3) KV cache with a calibrated per-tensor scale (evolve.pub review,
 * "Key claims under review", fifth claim: calibrated per-tensor FP8 KV-cache
 * scales; chatpaper.ai English abstract).  The scale s (DEVICE float32 [1])
 * is a decode multiplier: a cached byte q stands for e4m3(q) * s.  s = 1 is
 * the uncalibrated cache; calibrated and uncalibrated caches run the same
 * kernels.  Rows are cols elements, cols % 16 == 0.  Codes 0x7F/0xFF (NaN)
 * never come out of the write and are outside the contract of the read.
 *
 * nvfp4_kv_fp8_calibrate -- *scale = fl32(max|x| / 448) over x [rows, cols]
 *   (bf16 or float32, ld_x elements, rows 16-byte aligned).  workspace:
 *   nvfp4_quantize_workspace_bytes(rows, cols) bytes of device memory.
 */
int nvfp4_kv_fp8_calibrate(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           float* scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * nvfp4_kv_fp8_quantize -- write x [rows, cols] (bf16 or float32) into the
 * cache: cache[slot(i), j] = E4M3 byte nearest to the exact real x[i, j] / s,
 * ties to even code, |x / s| beyond 448 saturating to +-448, sign bit = IEEE
 * sign of x.  slot(i) = slots[i] (DEVICE int64 [rows]) or i when slots is
 * NULL; rows whose slot lies outside [0, cache_rows) are not written.
 * x must be finite: a NaN element gets an unspecified byte.
 * cache: DEVICE uint8 [cache_rows, ld_cache], ld_cache % 8 == 0, 8-byte
 * aligned; x rows 16-byte aligned.
 */
int nvfp4_kv_fp8_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                          const int64_t* slots, int64_t cache_rows, uint8_t* cache, int64_t ld_cache,
                          const float* scale, void* stream);

/*
 * nvfp4_kv_fp8_dequantize -- out[i, j] = fl32(e4m3(cache[i, j]) * s) (one
 * rounding of the exact product), stored as float32 or rounded to bf16
 * (nearest even).  out: DEVICE [rows, ld_out] elements, rows 16-byte aligned.
 */
int nvfp4_kv_fp8_dequantize(const uint8_t* cache, int64_t rows, int64_t cols, int64_t ld_cache,
                            const float* scale, void* out, int out_dtype, int64_t ld_out,
                            void* stream);

/*
 * nvfp4_harmonize_scales -- checkpoint-side repair of the global-scale
 * mismatch (evolve.pub review, "Key claims under review", fourth claim;
 * chatpaper.ai English abstract): per-module calibrated segments of a fused
 * weight are rewritten to share one global scale, so that a GEMM applying a
 * single global scale serves them.  G = max_s seg_global_scales[s]; every
 * block scale byte b of segment s becomes the E4M3 byte nearest to the exact
 * real e4m3(b) * g_s / G, ties to the even code.  E2M1 codes are unchanged:
 * the harmonized weight is {w->codes, out_scales, out_global_scale}.
 *
 *   w                  the segmented weight; only its scales are read
 *                      (w->global_scale is not used and may be NULL).
 *   seg_offsets        HOST int64 [n_segments + 1], as for
 *                      nvfp4_gemm_fused_segments; seg_global_scales DEVICE
 *                      float32 [n_segments], positive.
 *   out_scales         DEVICE uint8 [w->rows, ld_out_scales], ld_out_scales
 *                      >= w->cols / 16; may be w->scales (in place).
 *   out_global_scale   DEVICE float32 [1], receives G.
 */
int nvfp4_harmonize_scales(const nvfp4_tensor* w, int n_segments, const int64_t* seg_offsets,
                           const float* seg_global_scales, uint8_t* out_scales,
                           int64_t ld_out_scales, float* out_global_scale, void* stream);

/*
 * Gated delta-rule recurrence of a Gated DeltaNet layer (chatpaper.ai
 * English abstract, mechanisms (ii) and (iii); evolve.pub review, "Key
 * claims under review", third claim), consuming the gate epilogue's outputs
 * beta = sigmoid(b) and the log-space decay g.  The published update, per
 * value head h with a float32 state S in R^{128 x 128}:
 *     S_t = exp(g_t) S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t.
 * Heads are 128 wide.  Value head h reads q/k head h / (v_heads / k_heads).
 * With normalize_qk != 0, q and k are L2-normalized per head and q is scaled
 * by 128^-1/2 first (the short convolution of a GDN layer is not part of
 * this call).  Computed in float32, chunk-parallel (64 tokens per chunk).
 *
 * Each input is a row-major [tokens, width] matrix given by a device pointer
 * and a row stride in elements, all of one dtype (bf16 or float32), so the
 * columns of a fused in-projection output can be passed directly:
 *   q, k   [tokens, k_heads * 128];  v  [tokens, v_heads * 128];
 *   beta, g [tokens, v_heads].
 * q, k and v rows start on 16-byte boundaries (pointer and row stride).
 */
typedef struct {
  const void* q; int64_t ld_q;
  const void* k; int64_t ld_k;
  const void* v; int64_t ld_v;
  const void* beta; int64_t ld_beta;
  const void* g; int64_t ld_g;
} nvfp4_gdn_inputs;

/* Bytes of device workspace nvfp4_gdn_recurrence needs (per-chunk data,
 * about 115 KB per value head and 64 tokens). */
size_t nvfp4_gdn_workspace_bytes(int64_t tokens, int v_heads);

/*
 * nvfp4_gdn_recurrence -- o[t, h*128 + i] = (S_t q_t)[i] for every token t
 * and value head h.
 *   s0       DEVICE float32 [v_heads, 128, 128] initial states, or NULL (zeros).
 *   s_final  DEVICE float32 [v_heads, 128, 128] receives the last states, or NULL.
 *   o        DEVICE [tokens, ld_o] (bf16 or float32), ld_o >= v_heads * 128.
 *   workspace DEVICE, >= nvfp4_gdn_workspace_bytes(tokens, v_heads) bytes,
 *            16-byte aligned.
 * 1 <= k_heads, v_heads % k_heads == 0, v_heads <= 4096.
 */
int nvfp4_gdn_recurrence(const nvfp4_gdn_inputs* in, int in_dtype, int64_t tokens, int k_heads,
                         int v_heads, int normalize_qk, const float* s0, float* s_final, void* o,
                         int o_dtype, int64_t ld_o, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Human-readable text of a status (and of the last HIP error, for NVFP4_ERR_HIP). */
const char* nvfp4_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
