/*
 * One NVFP4 W4A4 linear layer through the C ABI alone (plain C99, the HIP
 * runtime API and include/nvfp4.h; no Python, no torch): activation and
 * weight quantization with dynamic global scales, then the GEMM.
 *
 *   linear_layer DIR M N K
 * reads DIR/x.bin (bf16 [M, K]) and DIR/w.bin (bf16 [N, K]), raw
 * little-endian, and writes DIR/a_codes.bin, DIR/a_scales.bin, DIR/a_g.bin
 * (the activation's NVFP4 codes [M, K/2], scales [M, K/16] and global
 * scale) and DIR/out.bin (float32 [M, N]).  Exit status 0 on success; on a
 * failed call it prints the library's status text and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "nvfp4.h"

static int fail_hip(hipError_t e, const char* what) {
  fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return 1;
}

static int fail_nvfp4(int st, const char* what) {
  fprintf(stderr, "%s: %s (status %d)\n", what, nvfp4_status_string(st), st);
  return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (f == NULL) return NULL;
  void* buf = malloc(bytes);
  if (buf != NULL && fread(buf, 1, bytes, f) != bytes) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  return buf;
}

static int write_file(const char* dir, const char* name, const void* buf, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (f == NULL) return 1;
  const int bad = fwrite(buf, 1, bytes, f) != bytes;
  return fclose(f) != 0 || bad;
}

int main(int argc, char** argv) {
  if (argc != 5) {
    fprintf(stderr, "usage: %s DIR M N K\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int64_t M = atoll(argv[2]), N = atoll(argv[3]), K = atoll(argv[4]);
  if (M <= 0 || N <= 0 || K <= 0 || K % 128 != 0) {
    fprintf(stderr, "M, N, K must be positive and K a multiple of 128\n");
    return 2;
  }
  const size_t x_bytes = (size_t)(M * K * 2), w_bytes = (size_t)(N * K * 2);
  void* hx = read_file(dir, "x.bin", x_bytes);
  void* hw = read_file(dir, "w.bin", w_bytes);
  if (hx == NULL || hw == NULL) {
    fprintf(stderr, "cannot read x.bin / w.bin in %s\n", dir);
    return 1;
  }

  /* device buffers: dense rows, so ld_codes = K/2 and ld_scales = K/16 */
  const int64_t ldc = K / 2, lds = K / 16;
  const size_t ws_bytes = nvfp4_quantize_workspace_bytes(M > N ? M : N, K);
  void *dx, *dw, *dout, *dws;
  uint8_t *a_codes, *a_scales, *w_codes, *w_scales;
  float *a_g, *w_g;
  hipError_t e;
  if ((e = hipMalloc(&dx, x_bytes)) != hipSuccess) return fail_hip(e, "hipMalloc x");
  if ((e = hipMalloc(&dw, w_bytes)) != hipSuccess) return fail_hip(e, "hipMalloc w");
  if ((e = hipMalloc((void**)&a_codes, (size_t)(M * ldc))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc((void**)&a_scales, (size_t)(M * lds))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc((void**)&w_codes, (size_t)(N * ldc))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc((void**)&w_scales, (size_t)(N * lds))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc((void**)&a_g, sizeof(float))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc((void**)&w_g, sizeof(float))) != hipSuccess) return fail_hip(e, "hipMalloc");
  if ((e = hipMalloc(&dout, (size_t)(M * N) * sizeof(float))) != hipSuccess) return fail_hip(e, "hipMalloc out");
  if ((e = hipMalloc(&dws, ws_bytes)) != hipSuccess) return fail_hip(e, "hipMalloc workspace");
  if ((e = hipMemcpy(dx, hx, x_bytes, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip(e, "copy x");
  if ((e = hipMemcpy(dw, hw, w_bytes, hipMemcpyHostToDevice)) != hipSuccess) return fail_hip(e, "copy w");

  /* the weight offline, then the layer: quantize x, GEMM (default stream) */
  int st = nvfp4_quantize(dw, NVFP4_DTYPE_BF16, N, K, K, w_codes, ldc, w_scales, lds, w_g, NVFP4_SCALE_DYNAMIC,
                          dws, ws_bytes, NULL);
  if (st != NVFP4_OK) return fail_nvfp4(st, "nvfp4_quantize(w)");
  st = nvfp4_quantize(dx, NVFP4_DTYPE_BF16, M, K, K, a_codes, ldc, a_scales, lds, a_g, NVFP4_SCALE_DYNAMIC, dws,
                      ws_bytes, NULL);
  if (st != NVFP4_OK) return fail_nvfp4(st, "nvfp4_quantize(x)");
  const nvfp4_tensor a = {a_codes, a_scales, a_g, M, K, ldc, lds};
  const nvfp4_tensor w = {w_codes, w_scales, w_g, N, K, ldc, lds};
  st = nvfp4_gemm(&a, &w, dout, NVFP4_DTYPE_F32, N, NULL);
  if (st != NVFP4_OK) return fail_nvfp4(st, "nvfp4_gemm");
  if ((e = hipDeviceSynchronize()) != hipSuccess) return fail_hip(e, "synchronize");

  const size_t out_bytes = (size_t)(M * N) * sizeof(float);
  uint8_t* hc = malloc((size_t)(M * ldc));
  uint8_t* hs = malloc((size_t)(M * lds));
  float* ho = malloc(out_bytes);
  float hg = 0.0f;
  if (hc == NULL || hs == NULL || ho == NULL) return 1;
  if ((e = hipMemcpy(hc, a_codes, (size_t)(M * ldc), hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip(e, "copy");
  if ((e = hipMemcpy(hs, a_scales, (size_t)(M * lds), hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip(e, "copy");
  if ((e = hipMemcpy(&hg, a_g, sizeof(float), hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip(e, "copy");
  if ((e = hipMemcpy(ho, dout, out_bytes, hipMemcpyDeviceToHost)) != hipSuccess) return fail_hip(e, "copy out");
  if (write_file(dir, "a_codes.bin", hc, (size_t)(M * ldc)) || write_file(dir, "a_scales.bin", hs, (size_t)(M * lds)) ||
      write_file(dir, "a_g.bin", &hg, sizeof hg) || write_file(dir, "out.bin", ho, out_bytes)) {
    fprintf(stderr, "cannot write the outputs in %s\n", dir);
    return 1;
  }
  hipFree(dx); hipFree(dw); hipFree(a_codes); hipFree(a_scales); hipFree(w_codes); hipFree(w_scales);
  hipFree(a_g); hipFree(w_g); hipFree(dout); hipFree(dws);
  free(hx); free(hw); free(hc); free(hs); free(ho);
  printf("linear layer %lldx%lldx%lld through the C ABI: ok\n", (long long)M, (long long)N, (long long)K);
  return 0;
}
