/* The C ABI used from plain C99: include/seqcomp.h compiles as C, the
 * library links, and the host-side entry points behave as declared.  Only
 * calls that return before any HIP call are made (queries, validation
 * failures, calls with zero entries), so no GPU is needed.  Exit status 0
 * means every check held; a failed check prints its line and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "seqcomp.h"

static int failures = 0;
#define CHECK(cond)                                                 \
  do {                                                              \
    if (!(cond)) {                                                  \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                   \
    }                                                               \
  } while (0)

int main(void) {
  int code;
  /* 16-byte aligned stand-ins: validation rejects the call before any of
   * them is dereferenced or handed to the device. */
  static _Alignas(16) unsigned char buf[4096];
  const int64_t cu[3] = {0, 1000, 2000};        /* 250 + 250 CSA entries at m = 4 */
  const int64_t cu_bad[3] = {0, 100, 50};       /* decreasing */
  const int64_t cu_short[2] = {0, 3};           /* shorter than m: no entries */

  CHECK(seqcomp_version() == 10000);
  for (code = SEQCOMP_OK; code <= SEQCOMP_E_SCRATCH; ++code) {
    const char* s = seqcomp_status_string(code);
    CHECK(s != NULL && strlen(s) > 0 && strcmp(s, "unknown status") != 0);
  }
  CHECK(strcmp(seqcomp_status_string(99), "unknown status") == 0);

  CHECK(seqcomp_num_entries(cu, 2, 4) == 250 + 250);
  CHECK(seqcomp_num_entries(cu, 2, 128) == 7 + 7);
  CHECK(seqcomp_num_entries(cu_bad, 2, 4) == -1);
  CHECK(seqcomp_num_entries(NULL, 1, 4) == -1);
  CHECK(seqcomp_workspace_bytes(SEQCOMP_OP_FUSED, SEQCOMP_MODE_CSA, 4, 512, cu, 2, SEQCOMP_BF16) > 0);
  CHECK(seqcomp_workspace_bytes(7, SEQCOMP_MODE_CSA, 4, 512, cu, 2, SEQCOMP_BF16) == (size_t)-1);
  CHECK(seqcomp_workspace_bytes(SEQCOMP_OP_POOL_CSA, 0, 4, 512, cu_short, 1, SEQCOMP_BF16) == 0);

  /* validation failures, in the order the header documents them */
  CHECK(seqcomp_project(buf, 64, 64, 9, buf, 128, buf + 2048, 128, SEQCOMP_BF16, NULL) == SEQCOMP_E_DTYPE);
  CHECK(seqcomp_project(NULL, 64, 64, SEQCOMP_BF16, buf, 128, buf + 2048, 128, SEQCOMP_BF16, NULL) ==
        SEQCOMP_E_NULL);
  CHECK(seqcomp_project(buf + 4, 64, 64, SEQCOMP_BF16, buf, 128, buf + 2048, 128, SEQCOMP_BF16, NULL) ==
        SEQCOMP_E_ALIGN);
  CHECK(seqcomp_compress_fused(SEQCOMP_MODE_CSA, 5, buf, 64, SEQCOMP_BF16, buf, 32, (const float*)buf,
                               (const float*)buf, cu, cu, 2, buf, SEQCOMP_BF16, NULL, buf, sizeof buf, NULL) ==
        SEQCOMP_E_UNSUPPORTED);
  CHECK(seqcomp_compress_fused(SEQCOMP_MODE_CSA, 4, buf, 64, SEQCOMP_BF16, buf, 32, (const float*)buf,
                               (const float*)buf, cu_bad, cu_bad, 2, buf, SEQCOMP_BF16, NULL, buf, sizeof buf,
                               NULL) == SEQCOMP_E_SEQLENS);
  /* zero entries: OK, and nothing is launched (no buffers needed) */
  CHECK(seqcomp_compress_fused(SEQCOMP_MODE_CSA, 4, NULL, 64, SEQCOMP_BF16, NULL, 32, NULL, NULL, cu_short, NULL,
                               1, NULL, SEQCOMP_BF16, NULL, NULL, 0, NULL) == SEQCOMP_OK);
  CHECK(seqcomp_pool_hca(NULL, NULL, 32, SEQCOMP_BF16, NULL, 128, 32, cu_short, NULL, 1, NULL, SEQCOMP_BF16, NULL,
                         NULL, 0, NULL) == SEQCOMP_OK);

  if (failures) return 1;
  printf("abi_from_c: all checks passed\n");
  return 0;
}
