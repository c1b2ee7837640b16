/* A plain C caller of the ISD library: includes only include/isd.h, links libisd.so, and
 * exercises the host-side paths that need no GPU (version, status strings, validation
 * failures, workspace queries).  Exit status 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "isd.h"

static int fails = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
      ++fails;                                                   \
    }                                                            \
  } while (0)

int main(void) {
  CHECK(isd_abi_version() == ISD_ABI_VERSION);
  CHECK(strcmp(isd_status_string(ISD_OK), "ok") == 0);
  CHECK(isd_verify_workspace_bytes(64, 4, 151936) > 0);
  CHECK(isd_lm_head_verify_workspace_bytes(64, 4, 151936) > isd_verify_workspace_bytes(64, 4, 151936));
  CHECK(isd_attention_workspace_bytes(64, 4, 32, 8, 128, 4096) > 0);
  CHECK(isd_gated_lora_workspace_bytes(448, 4096, 4096, 128) > 0);
  CHECK(isd_proj_packed_bytes(4096, 4096, 128) == (size_t)(4096 + 128) * 4096 * 2 + (size_t)4096 * 128 * 2);

  /* validation failures return before anything is launched */
  void* fake = (void*)0x1000;
  CHECK(isd_lm_head(NULL, fake, fake, 448, 4096, 151936, NULL) == ISD_ERR_INVALID_ARG);
  CHECK(strlen(isd_last_error()) > 0);
  CHECK(isd_lm_head(fake, fake, fake, 448, 4096, 151937, NULL) == ISD_ERR_UNSUPPORTED);
  CHECK(isd_commit(fake, fake, fake, fake, fake, NULL, NULL, 4, 9, NULL) == ISD_ERR_UNSUPPORTED);
  CHECK(isd_gated_lora_proj(fake, fake, fake, fake, fake, fake, 0, 4096, 4096, 128, fake, 1 << 30,
                            NULL) == ISD_ERR_INVALID_ARG);
  CHECK(isd_pack_kv_pages(ISD_BF16, fake, (void*)0x2000, (void*)0x3000, (void*)0x4000, 10, 8, 96, NULL) ==
        ISD_ERR_UNSUPPORTED);
  CHECK(isd_unpack_kv_pages(ISD_BF16, NULL, fake, (void*)0x3000, (void*)0x4000, 10, 8, 128, NULL) ==
        ISD_ERR_INVALID_ARG);
  CHECK(isd_kv_read_sweep(fake, fake, (const int32_t*)fake, (const int32_t*)fake, 64, 8, 96, 257, 20000, 4096,
                          (uint32_t*)fake, NULL) == ISD_ERR_UNSUPPORTED);
  CHECK(isd_kv_read_sweep(fake, fake, (const int32_t*)fake, (const int32_t*)fake, 64, 8, 128, 257, 20000, 4096,
                          NULL, NULL) == ISD_ERR_INVALID_ARG);
  CHECK(isd_verify_carry_bytes(64, 4, 151936) > 0 && isd_verify_carry_bytes(64, 1, 151936) == 0);
  CHECK(isd_verify_carry(ISD_BF16, fake, fake, (const int32_t*)fake, (const float*)fake, 4, 4, 151936, 1.f,
                         (int32_t*)fake, (uint8_t*)fake, (int32_t*)fake, (int32_t*)fake, (int32_t*)fake, NULL, NULL,
                         NULL, fake, fake, fake, (size_t)1 << 30, NULL) == ISD_ERR_INVALID_ARG);
  CHECK(isd_pack_proj_weights_kn(NULL, fake, fake, fake, 4096, 4096, 128, NULL) == ISD_ERR_INVALID_ARG);
  CHECK(isd_pack_proj_weights_kn(fake, fake, fake, fake, 4096, 4100, 128, NULL) == ISD_ERR_UNSUPPORTED);
  if (fails == 0) printf("c abi ok\n");
  return fails == 0 ? 0 : 1;
}
