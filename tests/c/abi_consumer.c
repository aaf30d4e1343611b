/* A plain C consumer of libosdn.so: compiled with a C compiler against
 * include/osdn.h alone, it checks the host-side behaviour of the C ABI
 * (capability and workspace queries, argument validation) without launching
 * any GPU work, so it runs on a machine without a GPU. Exit status 0 = all
 * checks passed; otherwise the number of failed checks. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "osdn.h"

static int failures = 0;

#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "check failed (line %d): %s\n", __LINE__, #cond); \
      ++failures;                                                \
    }                                                            \
  } while (0)

#define P(x) ((void*)(uintptr_t)(x))

int main(void) {
  /* status texts */
  CHECK(strcmp(osdn_strerror(OSDN_OK), "ok") == 0);
  CHECK(osdn_strerror(OSDN_ERR_ALIASING) != NULL);
  CHECK(strcmp(osdn_strerror(1234), "unknown status") == 0);

  /* capability queries */
  CHECK(osdn_forward_supported(128, 128, 64, OSDN_BF16) == 1);
  CHECK(osdn_forward_supported(48, 128, 64, OSDN_BF16) == 0);
  CHECK(gdn2_forward_supported(128, 128, 64, OSDN_BF16) == 1);
  CHECK(osdn_gated_forward_supported(128, 128, 64, OSDN_BF16) == 1);

  /* workspace sizes: positive for the 1.3B-layer shape, 0 for bad sizes */
  CHECK(osdn_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, OSDN_BF16) > 0);
  CHECK(osdn_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, OSDN_BF16) % 256 == 0);
  CHECK(osdn_forward_workspace_bytes(-1, 16, 4096, 128, 128, 64, OSDN_BF16) == 0);
  CHECK(gdn2_forward_workspace_bytes(4, 16, 4096, 128, 128, 64, OSDN_BF16) > 0);
  CHECK(osdn_precond_workspace_bytes(4, 16, 4096, 128, OSDN_BF16) > 0);

  /* validation happens on the host, before any launch (the fake device
   * addresses below are never dereferenced) */
  const int B = 1, H = 1, T = 64, Dk = 32, Dv = 32, C = 16;
  const size_t wsb = 1u << 20;
  CHECK(osdn_forward(B, H, T, Dk, Dv, C, OSDN_BF16, NULL, P(0x20000), P(0x30000),
                     P(0x40000), NULL, 0.1f, NULL, NULL, 1.f, P(0x50000), NULL,
                     NULL, NULL, NULL, P(0x100000), wsb, NULL) == OSDN_ERR_NULL_ARG);
  CHECK(osdn_forward(B, H, -1, Dk, Dv, C, OSDN_BF16, P(0x10000), P(0x20000),
                     P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                     P(0x50000), NULL, NULL, NULL, NULL, P(0x100000), wsb,
                     NULL) == OSDN_ERR_BAD_DIMS);
  CHECK(osdn_forward(B, H, T, 48, Dv, C, OSDN_BF16, P(0x10000), P(0x20000),
                     P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                     P(0x50000), NULL, NULL, NULL, NULL, P(0x100000), wsb,
                     NULL) == OSDN_ERR_UNSUPPORTED);
  CHECK(osdn_forward(B, H, T, Dk, Dv, C, OSDN_BF16, P(0x10000), P(0x20000),
                     P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                     P(0x50000), NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == OSDN_ERR_WORKSPACE);
  CHECK(osdn_forward(B, H, T, Dk, Dv, C, OSDN_BF16, P(0x10000), P(0x20000),
                     P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                     P(0x30000 + 64), NULL, NULL, NULL, NULL, P(0x100000), wsb,
                     NULL) == OSDN_ERR_ALIASING);
  /* nothing to do: no pointer needed */
  CHECK(osdn_forward(0, H, T, Dk, Dv, C, OSDN_BF16, NULL, NULL, NULL, NULL, NULL,
                     0.1f, NULL, NULL, 1.f, NULL, NULL, NULL, NULL, NULL, NULL, 0,
                     NULL) == OSDN_OK);
  CHECK(osdn_decode(B, H, T, Dk, Dv, OSDN_BF16, P(0x10000), P(0x20000),
                    P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, P(0x300000),
                    1.f, P(0x50000), NULL) == OSDN_ERR_NULL_ARG);
  CHECK(gdn2_decode(B, H, T, Dk, Dv, OSDN_BF16, P(0x10000), P(0x20000),
                    P(0x30000), P(0x60000), P(0x70000), P(0x80000), P(0x70000),
                    1.f, P(0x50000), NULL) == OSDN_ERR_ALIASING);

  if (failures == 0) printf("abi_consumer: all checks passed\n");
  return failures;
}
