/* Host-only use of the C ABI from plain C11: version, workspace sizes and argument checks
 * (every call below fails validation, so no device is touched).  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>

#include "olmoe_moe.h"

#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                        \
    }                                                                  \
  } while (0)

int main(void) {
  CHECK(olmoe_abi_version() == OLMOE_ABI_VERSION);
  CHECK(olmoe_moe_workspace_bytes(-1) == 0);
  CHECK(olmoe_moe_workspace_bytes(256) > (size_t)8 * 256 * (1024 + 2048) * 2);
  CHECK(olmoe_moe_workspace_bytes(4096) > olmoe_moe_workspace_bytes(256));
  CHECK(olmoe_moe_ec_workspace_bytes(OLMOE_EC_MAX_TOKENS + 1) == 0);
  CHECK(olmoe_moe_saved_bytes(64) == olmoe_moe_backward_workspace_bytes(64));
  size_t perm = 0, inv = 0, offs = 0;
  CHECK(olmoe_moe_workspace_layout(100, &perm, &inv, &offs) == OLMOE_OK);
  CHECK(perm != inv && inv != offs && perm < olmoe_moe_workspace_bytes(100));
  /* bad arguments: NULL weights, negative T, short workspace */
  void* fake = (void*)(uintptr_t)(1u << 20);
  CHECK(olmoe_moe_forward(fake, NULL, fake, fake, fake, 4, fake, NULL, NULL, NULL, NULL, NULL, fake,
                          1u << 30, NULL) == OLMOE_EINVAL);
  CHECK(olmoe_last_error()[0] != '\0');
  CHECK(olmoe_moe_forward(fake, (const float*)fake, fake, fake, fake, -1, fake, NULL, NULL, NULL, NULL,
                          NULL, fake, 1u << 30, NULL) == OLMOE_EINVAL);
  CHECK(olmoe_moe_forward((void*)(uintptr_t)(1u << 20), (const float*)(uintptr_t)(2u << 20),
                          (void*)((uintptr_t)1 << 32), (void*)((uintptr_t)2 << 32), (void*)((uintptr_t)3 << 32), 16,
                          (void*)(uintptr_t)(4u << 20), NULL, NULL, NULL, NULL, NULL,
                          (void*)((uintptr_t)8 << 36), 1000, NULL) == OLMOE_EWORKSPACE);
  CHECK(olmoe_timing_enable(1 << 5) == OLMOE_EINVAL);
  CHECK(olmoe_timing_every(0) == OLMOE_EINVAL);
  CHECK(olmoe_timing_every(4) == OLMOE_OK);
  CHECK(olmoe_timing_enable(0) == OLMOE_OK);
  printf("C ABI host checks passed (ABI %d)\n", olmoe_abi_version());
  return 0;
}
