// nvfp4_quantize_noalloc: nvfp4_quantize without a caller workspace, for
// callers that cannot allocate device memory.  The amax partials of the
// dynamic global scale live in a file-scope device array instead.
//
// Host code never passes `scratch` itself to a kernel: on the host that name
// is only a stand-in for the symbol.  The array's device address is looked
// up with hipGetSymbolAddress on the first call on each device (with that
// device current) and kept per device; every later use goes through that
// address.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "internal.h"
#include "nvfp4.h"

namespace nvfp4 {
namespace {

// Room for the largest partial count any shape produces (kMaxPartials).
constexpr size_t kScratchFloats = kMaxPartials;
static_assert(sizeof(float) * kScratchFloats == NVFP4_NOALLOC_SCRATCH_BYTES, "header states the size");
static __device__ __align__(256) float scratch[kScratchFloats];

// Device address of `scratch`, per device (written once per device; a race
// between two first calls stores the same address twice).
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_addr[kMaxDevices];

hipError_t scratch_address(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    float* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p != nullptr) {
      *out = p;
      return hipSuccess;
    }
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  if (cached) g_scratch_addr[dev].store(static_cast<float*>(p), std::memory_order_release);
  *out = static_cast<float*>(p);
  return hipSuccess;
}

}  // namespace
}  // namespace nvfp4

using namespace nvfp4;

extern "C" int nvfp4_quantize_noalloc(const void* x, int x_dtype, int64_t rows, int64_t cols, int64_t ld_x,
                                      uint8_t* codes, int64_t ld_codes, uint8_t* scales, int64_t ld_scales,
                                      float* global_scale, int flags, void* stream) {
  if (flags == NVFP4_AMAX_PRECOMPUTED) return NVFP4_ERR_FLAGS;  // no caller workspace to hold partials
  const int st = quantize_check(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales, ld_scales,
                                global_scale, flags);
  if (st != NVFP4_OK) return st;
  if (nvfp4_quantize_workspace_bytes(rows, cols) > sizeof(float) * kScratchFloats) return NVFP4_ERR_WORKSPACE;
  float* partials = nullptr;
  if (flags == NVFP4_SCALE_DYNAMIC) {
    const hipError_t e = scratch_address(&partials);
    if (e != hipSuccess) return status_from_hip(e);
  }
  return quantize_launch(x, x_dtype, rows, cols, ld_x, codes, ld_codes, scales, ld_scales, global_scale, flags,
                         partials, stream);
}
