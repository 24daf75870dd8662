/* A plain C99 client of include/smcsd.h: compiled with gcc -std=c99 -pedantic and linked
 * against libsmcsd.so, it checks that the header is valid C and that the host-side
 * entry points behave as documented without any device (no call here reaches a kernel:
 * every one is rejected, or answered, on the host).  Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "smcsd.h"

static int fails = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__);     \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  void *p = (void *)0x1000; /* never dereferenced: each call below fails validation first */
  int32_t *ip = (int32_t *)p;
  float *fp = (float *)p;

  CHECK(smcsd_version() == SMCSD_VERSION);
  CHECK(strcmp(smcsd_status_string(SMCSD_OK), "ok") == 0);
  CHECK(strstr(smcsd_status_string(SMCSD_ST_NOSPACE), "pool") != NULL);

  CHECK(smcsd_workspace_bytes(SMCSD_OP_VERIFY_SMC, 32, 16, 4, 128256, 0) > 0);
  CHECK(smcsd_workspace_bytes(SMCSD_OP_VERIFY_SMC, 1, 1, 33, 10, 0) == 0);
  CHECK(smcsd_workspace_bytes(SMCSD_OP_KV, 32, 16, 0, 0, 145920) > 0);
  CHECK(smcsd_workspace_bytes(SMCSD_OP_KV_CHECK, 0, 0, 0, 0, 1000) >= 8000);

  /* verify: a dtype the library does not take; an unsupported mode; a zero workspace */
  CHECK(smcsd_verify(p, p, 7, 64, 1, ip, 1, 1, 1, 64, 1.0f, 1.0f, SMCSD_MODE_SMC, 0, 0, NULL,
                     NULL, fp, ip, NULL, NULL, NULL, NULL, ip, p, 1 << 20, NULL) == SMCSD_EDTYPE);
  CHECK(smcsd_verify(p, p, SMCSD_DTYPE_BF16, 64, 1, ip, 1, 1, 1, 64, 1.0f, 1.0f, 9, 0, 0, NULL,
                     NULL, fp, ip, NULL, NULL, NULL, NULL, ip, p, 1 << 20, NULL) == SMCSD_EINVAL);
  CHECK(smcsd_verify(p, p, SMCSD_DTYPE_BF16, 64, 1, ip, 1, 1, 1, 64, 1.0f, 1.0f, SMCSD_MODE_SMC,
                     0, 0, NULL, NULL, fp, ip, NULL, NULL, NULL, NULL, ip, p, 16,
                     NULL) == SMCSD_EWORKSPACE);
  /* resample: N above the limit */
  CHECK(smcsd_resample(fp, 1, 1025, 0.5f, 0, 0, ip, fp, ip, ip, NULL) == SMCSD_EINVAL);
  /* KV: a reservation beyond M_cap slots */
  CHECK(smcsd_kv_reassign(ip, ip, 2, 4, ip, 8, 4, 30, 8, ip, ip, ip, 64, ip, ip, ip, p, 1 << 20,
                          NULL) == SMCSD_EINVAL);
  /* the whole round: SpS is not an SMC-SD round */
  CHECK(smcsd_step(p, p, SMCSD_DTYPE_BF16, 64, ip, 2, 4, 1, 64, 1.0f, 1.0f, SMCSD_MODE_SPS, 0.5f,
                   0, 0, NULL, fp, ip, NULL, NULL, NULL, NULL, ip, fp, ip, ip, 8, 4, 4, 2, ip, ip,
                   ip, 64, ip, ip, ip, p, 1 << 20, p, 1 << 20, NULL) == SMCSD_EINVAL);
  /* the KV check: slots beyond M_cap; a workspace too small */
  CHECK(smcsd_kv_check(ip, 4, 8, 9, ip, ip, ip, 100, ip, ip, p, 1 << 20, NULL) == SMCSD_EINVAL);
  CHECK(smcsd_kv_check(ip, 4, 8, 3, ip, ip, ip, 100, ip, ip, p, 16, NULL) == SMCSD_EWORKSPACE);
  /* the read-rate aid: a size that is not a multiple of 16; a pointer not 16-byte aligned */
  CHECK(smcsd_stream_read(p, 24, (uint32_t *)p, NULL) == SMCSD_EINVAL);
  CHECK(smcsd_stream_read((char *)p + 8, 32, (uint32_t *)p, NULL) == SMCSD_EINVAL);
  /* empty batches are no-ops that succeed without touching anything */
  CHECK(smcsd_resample(fp, 0, 4, 0.5f, 0, 0, ip, fp, ip, ip, NULL) == SMCSD_OK);

  if (fails) return 1;
  printf("ok\n");
  return 0;
}
