/* The C ABI used from C99 without a GPU: version, status strings, the support matrix, host sign
 * generation, and argument checks that fail before any device call.  Prints the sign vector
 * for the test to compare with the Python generator; exits 1 at the first failed check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "rhtq.h"
#include "rhtq_floor.h"

static int failed(const char* what) {
  fprintf(stderr, "check failed: %s\n", what);
  return 1;
}

int main(void) {
  static int8_t signs[64];
  const void* fake = (const void*)(uintptr_t)0x100000;   /* never dereferenced */
  const void* mis = (const void*)(uintptr_t)0x100004;    /* not 16-byte aligned */

  if (rhtq_abi_version() != RHTQ_ABI_VERSION) return failed("abi version");
  if (strcmp(rhtq_status_str(RHTQ_OK), "ok") != 0) return failed("status string");
  if (!rhtq_supported(4096, RHTQ_FMT_INT4, 0) || !rhtq_supported(12288, RHTQ_FMT_INT4, 128) ||
      !rhtq_supported(11008, RHTQ_FMT_MXFP4, 32) || rhtq_supported(100, RHTQ_FMT_INT4, 0) ||
      rhtq_supported(4096, RHTQ_FMT_NVFP4, 32))
    return failed("support matrix");
  if (rhtq_signs_from_seed(12345, 64, signs) != RHTQ_OK) return failed("signs");
  if (rhtq_signs_from_seed(1, -1, signs) != RHTQ_EINVAL) return failed("signs: negative n");

  /* argument checks: nothing reaches the device */
  if (rhtq_rotate(fake, 7, 4, 4096, NULL, (float*)fake, NULL) != RHTQ_EINVAL) return failed("input type");
  if (rhtq_rotate(mis, RHTQ_IN_F16, 4, 4096, NULL, (float*)fake, NULL) != RHTQ_EINVAL) return failed("alignment");
  if (rhtq_rotate(fake, RHTQ_IN_BF16, 4, 100, NULL, (float*)fake, NULL) != RHTQ_EUNSUPPORTED) return failed("width");
  if (rhtq_rotate(NULL, RHTQ_IN_BF16, 0, 4096, NULL, NULL, NULL) != RHTQ_OK) return failed("empty call");
  if (rhtq_forward(fake, RHTQ_IN_BF16, -1, 4096, NULL, RHTQ_FMT_INT4, 0, RHTQ_SCALE_F32, (uint8_t*)fake,
                   (void*)fake, NULL, 0, NULL) != RHTQ_EINVAL)
    return failed("negative tokens");
  if (rhtq_forward(fake, RHTQ_IN_BF16, 4, 4096, NULL, RHTQ_FMT_INT4, 96, RHTQ_SCALE_F32, (uint8_t*)fake,
                   (void*)fake, NULL, 0, NULL) != RHTQ_EUNSUPPORTED)
    return failed("group");
  if (rhtq_stream_floor(fake, 4, 2048, (void*)fake, (void*)fake, 4, NULL) != RHTQ_EUNSUPPORTED)
    return failed("floor width");

  printf("signs");
  for (int i = 0; i < 64; ++i) printf(" %d", signs[i]);
  printf("\n");
  return 0;
}
