/*
 * A plain C99 client of the attention library: it uses only include/attn_fwd.h
 * and the HIP runtime's C API, no C++ and no Python, to show the boundary is
 * a C ABI.
 *
 *   attn_c_client host
 *       Host-side checks that need no GPU: argument validation codes, the
 *       variant pick, status strings, and that attn_fwd itself returns the
 *       validation error before touching the GPU. Exit status 0 when all hold.
 *   attn_c_client run IN OUT
 *       Reads B, H, S, D (int32), scale (float32) and q, k, v (bf16 bits,
 *       [B,H,S,D] each) from IN, runs attn_fwd on the default stream and
 *       writes O (bf16 bits) and LSE (float32) to OUT.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "attn_fwd.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %d (%s), want %d (%s)\n", what, got, attn_status_str(got), want,
            attn_status_str(want));
    ++failures;
  }
}

static int host_checks(void) {
  /* Fake, aligned, non-overlapping device addresses: compared, never dereferenced. */
  const uintptr_t base = (uintptr_t)0x10000000u;
  const void* q = (const void*)(base);
  const void* k = (const void*)(base + 0x1000000u);
  const void* v = (const void*)(base + 0x2000000u);
  void* o = (void*)(base + 0x3000000u);
  float* lse = (float*)(base + 0x4000000u);
  const float sc = 0.08838834764831845f;

  expect(attn_fwd_check(q, k, v, o, lse, 2, 3, 256, 128, sc), ATTN_OK, "valid arguments");
  expect(attn_fwd_check(NULL, k, v, o, lse, 2, 3, 256, 128, sc), ATTN_ERR_NULL, "null q");
  expect(attn_fwd_check(q, k, v, o, lse, 2, 3, 256, 64, sc), ATTN_ERR_SHAPE, "D = 64");
  expect(attn_fwd_check(q, k, v, o, lse, 2, 3, 200, 128, sc), ATTN_ERR_SHAPE, "S = 200");
  expect(attn_fwd_check(q, k, v, o, lse, 0, 3, 256, 128, sc), ATTN_ERR_SHAPE, "B = 0");
  expect(attn_fwd_check((const char*)q + 8, k, v, o, lse, 2, 3, 256, 128, sc), ATTN_ERR_ALIGN,
         "misaligned q");
  expect(attn_fwd_check(q, k, v, o, lse, 2, 3, 256, 128, 0.0f), ATTN_ERR_SCALE, "scale 0");
  expect(attn_fwd_check(q, k, v, (void*)q, lse, 2, 3, 256, 128, sc), ATTN_ERR_OVERLAP, "o aliases q");
  /* attn_fwd and attn_fwd_variant validate before any GPU work */
  expect(attn_fwd(NULL, k, v, o, lse, 2, 3, 256, 128, sc, NULL), ATTN_ERR_NULL, "attn_fwd null q");
  expect(attn_fwd_variant(q, k, v, o, lse, 2, 3, 256, 128, sc, 99, NULL), ATTN_ERR_VARIANT,
         "unknown variant");
  expect(attn_fwd_pick(1, 1, 256), ATTN_VARIANT_TILE128, "pick s256");
  expect(attn_fwd_pick(1, 16, 16384), ATTN_VARIANT_PAIR256, "pick s16k");
  if (strcmp(attn_status_str(ATTN_OK), "ok") != 0) {
    fprintf(stderr, "FAIL status string of ATTN_OK\n");
    ++failures;
  }
  printf("host checks: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}

#define HIP_OK(call)                                                           \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));        \
      return 2;                                                                \
    }                                                                          \
  } while (0)

static int run(const char* in_path, const char* out_path) {
  FILE* f = fopen(in_path, "rb");
  if (!f) {
    perror(in_path);
    return 2;
  }
  int32_t dims[4];
  float scale;
  if (fread(dims, sizeof dims, 1, f) != 1 || fread(&scale, sizeof scale, 1, f) != 1) {
    fprintf(stderr, "short header\n");
    fclose(f);
    return 2;
  }
  const int B = dims[0], H = dims[1], S = dims[2], D = dims[3];
  if (B < 1 || H < 1 || S < 1 || D < 1 || (size_t)B * H * S > ((size_t)1 << 26)) {
    fprintf(stderr, "bad dimensions\n");
    fclose(f);
    return 2;
  }
  const size_t n = (size_t)B * H * S * D, rows = (size_t)B * H * S;
  uint16_t* host = (uint16_t*)malloc(3 * n * sizeof(uint16_t));
  uint16_t* host_o = (uint16_t*)malloc(n * sizeof(uint16_t));
  float* host_lse = (float*)malloc(rows * sizeof(float));
  if (!host || !host_o || !host_lse || fread(host, sizeof(uint16_t), 3 * n, f) != 3 * n) {
    fprintf(stderr, "short input\n");
    fclose(f);
    return 2;
  }
  fclose(f);

  void *dq, *dk, *dv, *dout;
  float* dlse;
  HIP_OK(hipMalloc(&dq, n * 2));
  HIP_OK(hipMalloc(&dk, n * 2));
  HIP_OK(hipMalloc(&dv, n * 2));
  HIP_OK(hipMalloc(&dout, n * 2));
  HIP_OK(hipMalloc((void**)&dlse, rows * 4));
  HIP_OK(hipMemcpy(dq, host, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dk, host + n, n * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dv, host + 2 * n, n * 2, hipMemcpyHostToDevice));

  const int status = attn_fwd(dq, dk, dv, dout, dlse, B, H, S, D, scale, NULL);
  if (status != ATTN_OK) {
    fprintf(stderr, "attn_fwd: %s\n", attn_status_str(status));
    return 3;
  }
  HIP_OK(hipDeviceSynchronize());
  HIP_OK(hipMemcpy(host_o, dout, n * 2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host_lse, dlse, rows * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipFree(dq));
  HIP_OK(hipFree(dk));
  HIP_OK(hipFree(dv));
  HIP_OK(hipFree(dout));
  HIP_OK(hipFree(dlse));

  FILE* g = fopen(out_path, "wb");
  if (!g || fwrite(host_o, 2, n, g) != n || fwrite(host_lse, 4, rows, g) != rows) {
    fprintf(stderr, "cannot write %s\n", out_path);
    return 2;
  }
  fclose(g);
  free(host);
  free(host_o);
  free(host_lse);
  printf("attn_fwd B=%d H=%d S=%d D=%d: ok\n", B, H, S, D);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 2 && strcmp(argv[1], "host") == 0) return host_checks();
  if (argc == 4 && strcmp(argv[1], "run") == 0) return run(argv[2], argv[3]);
  fprintf(stderr, "usage: %s host | %s run IN OUT\n", argv[0], argv[0]);
  return 2;
}
