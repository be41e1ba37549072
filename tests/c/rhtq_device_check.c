/* The C ABI driven from C99 with the HIP runtime API: device buffers, a stream of its own,
 * rhtq_forward (INT4, one fp32 scale per row) and rhtq_rotate on 8 rows of 4096 bf16 values.
 * The input is x[t][j] = ((7 j + 13 t) mod 31 - 15) / 8, exact in bf16; the signs come from
 * seed 7.  Writes the codes, scales and rotation to the file named by argv[1] (packed bytes,
 * then fp32 scales, then fp32 y, each row-major) for the test to check against the oracle. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rhtq.h"

enum { T = 8, N = 4096 };

#define HIP_OK(call)                                                         \
  do {                                                                       \
    if ((call) != hipSuccess) {                                              \
      fprintf(stderr, "HIP call failed: %s\n", #call);                       \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static uint16_t bf16_bits(float v) {   /* exact for the values used here */
  uint32_t u;
  memcpy(&u, &v, 4);
  return (uint16_t)(u >> 16);
}

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  static uint16_t hx[T * N];
  static int8_t hs[N];
  static uint8_t hp[T * N / 2];
  static float hsc[T];
  static float hy[T * N];
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < N; ++j) hx[t * N + j] = bf16_bits((float)((7 * j + 13 * t) % 31 - 15) / 8.0f);
  if (rhtq_signs_from_seed(7, N, hs) != RHTQ_OK) return 1;

  void *dx, *ds, *dp, *dsc, *dy;
  HIP_OK(hipMalloc(&dx, sizeof hx));
  HIP_OK(hipMalloc(&ds, sizeof hs));
  HIP_OK(hipMalloc(&dp, sizeof hp));
  HIP_OK(hipMalloc(&dsc, sizeof hsc));
  HIP_OK(hipMalloc(&dy, sizeof hy));
  HIP_OK(hipMemcpy(dx, hx, sizeof hx, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(ds, hs, sizeof hs, hipMemcpyHostToDevice));
  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  int rc = rhtq_forward(dx, RHTQ_IN_BF16, T, N, (const int8_t*)ds, RHTQ_FMT_INT4, 0, RHTQ_SCALE_F32,
                        (uint8_t*)dp, dsc, NULL, 0, (rhtq_stream_t)st);
  if (rc != RHTQ_OK) {
    fprintf(stderr, "rhtq_forward: %s\n", rhtq_status_str(rc));
    return 1;
  }
  rc = rhtq_rotate(dx, RHTQ_IN_BF16, T, N, (const int8_t*)ds, (float*)dy, (rhtq_stream_t)st);
  if (rc != RHTQ_OK) {
    fprintf(stderr, "rhtq_rotate: %s\n", rhtq_status_str(rc));
    return 1;
  }
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipMemcpy(hp, dp, sizeof hp, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hsc, dsc, sizeof hsc, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(hy, dy, sizeof hy, hipMemcpyDeviceToHost));
  HIP_OK(hipStreamDestroy(st));
  HIP_OK(hipFree(dx));
  HIP_OK(hipFree(ds));
  HIP_OK(hipFree(dp));
  HIP_OK(hipFree(dsc));
  HIP_OK(hipFree(dy));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  const int ok = fwrite(hp, 1, sizeof hp, f) == sizeof hp && fwrite(hsc, 1, sizeof hsc, f) == sizeof hsc &&
                 fwrite(hy, 1, sizeof hy, f) == sizeof hy;
  fclose(f);
  printf("device check: wrote %d rows\n", T);
  return ok ? 0 : 1;
}
