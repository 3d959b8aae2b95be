// Stand-ins for the kernel launchers, so that the C-ABI layer (api.hip) can
// be built as plain host C++ under AddressSanitizer / UBSan and driven on a
// machine without a GPU.  Each launcher records that it was called and
// returns the status the driver asks for (success by default); none touches
// the pointers it gets (they are device addresses in real use).  The pure
// host helpers mirror the shapes the kernels' own sources compute, which is
// all the argument validation needs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../bit_linear_layer_amd/csrc/internal.h"

namespace {
hipError_t g_next = hipSuccess;
int g_calls = 0;
hipError_t record() {
  ++g_calls;
  return g_next;
}
}  // namespace

extern "C" void nvfp4_stub_set_launch_status(int e) { g_next = (hipError_t)e; }
extern "C" int nvfp4_stub_calls(void) { return g_calls; }

namespace nvfp4 {

int partial_count(int64_t rows, int64_t cols, int chunk) {
  int64_t wg = (rows * (cols / chunk) + kElemThreads - 1) / kElemThreads;
  if (wg < 1) wg = 1;
  if (wg > kMaxPartials) wg = kMaxPartials;
  return (int)wg;
}
size_t gdn_workspace_floats(int64_t T, int hv) { return (size_t)((T + 63) / 64) * hv * (12420 + 16384); }
size_t decode_weight_bytes(int64_t N, int64_t K) { return (size_t)((N + 15) / 16) * 8 * ((K + 1023) / 1024) * 1152; }

hipError_t launch_amax(const void*, int, int64_t, int64_t, int64_t, float*, int, hipStream_t) { return record(); }
hipError_t launch_quantize(const void*, int, int64_t, int64_t, int64_t, uint8_t*, int64_t, uint8_t*, int64_t, float*,
                           int, float*, int, hipStream_t) { return record(); }
hipError_t launch_silu_mul(const uint16_t*, int64_t, int64_t, int64_t, uint16_t*, int64_t, float*, int, hipStream_t) {
  return record();
}
hipError_t launch_gemm(const GemmArgs& p, hipStream_t) {
  // read every field the real launcher reads on the host
  volatile int sink = p.M + p.N + p.K + p.ep.n_seg + p.ep.b_seg + p.ep.a_seg;
  for (int s = 0; s <= p.ep.n_seg; ++s) sink += p.ep.seg_off[s];
  (void)sink;
  return record();
}
hipError_t launch_gemm_swiglu(const GemmArgs& p, hipStream_t) {
  volatile int sink = p.ep.inter + p.ep.n_partials;
  (void)sink;
  return record();
}
hipError_t launch_zero(float*, int, hipStream_t) { return record(); }
hipError_t launch_kv_quantize(const void*, int, int64_t, int64_t, int64_t, const int64_t*, int64_t, uint8_t*, int64_t,
                              const float*, hipStream_t) { return record(); }
hipError_t launch_kv_dequantize(const uint8_t*, int64_t, int64_t, int64_t, const float*, void*, int, int64_t,
                                hipStream_t) { return record(); }
hipError_t launch_kv_scale(const float*, int, float*, hipStream_t) { return record(); }
hipError_t launch_harmonize(const uint8_t*, int64_t, uint8_t*, int64_t, int64_t, int64_t, const SegmentTable& seg,
                            const float*, float*, hipStream_t) {
  volatile int64_t sink = 0;
  for (int s = 0; s <= seg.n; ++s) sink += seg.off[s];
  (void)sink;
  return record();
}
hipError_t launch_gdn(const GdnArgs&, float*, hipStream_t) { return record(); }
hipError_t launch_decode_pack(const uint8_t*, int64_t, const uint8_t*, int64_t, int, int, uint8_t*, hipStream_t) {
  return record();
}
hipError_t launch_gemm_decode(const GemmArgs& p, const uint8_t*, const void*, int, int64_t, float*, bool,
                              hipStream_t) {
  volatile int sink = p.M + p.N + p.K;
  for (int s = 0; s <= p.ep.n_seg; ++s) sink += p.ep.seg_off[s];
  (void)sink;
  return record();
}

}  // namespace nvfp4
