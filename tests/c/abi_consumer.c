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

  /* every supported size: the advertised workspace is the layout the header
   * states (chunk 64: phase-1 scratch + phase-2 scratch; otherwise the
   * preconditioned keys rounded up to 256 bytes + the larger of the two);
   * unsupported sizes advertise 0 */
  {
    static const int dims[3] = {32, 64, 128}, chunks[3] = {16, 32, 64};
    static const int shapes[3][3] = {{1, 1, 1}, {2, 3, 448}, {3, 1, 1000}};
    for (int dt = 0; dt < 2; ++dt)
      for (int a = 0; a < 3; ++a)
        for (int b = 0; b < 3; ++b)
          for (int c = 0; c < 3; ++c)
            for (int s = 0; s < 3; ++s) {
              const int Dk = dims[a], Dv = dims[b], Ch = chunks[c];
              const int Bq = shapes[s][0], Hq = shapes[s][1], Tq = shapes[s][2];
              const size_t got =
                  osdn_forward_workspace_bytes(Bq, Hq, Tq, Dk, Dv, Ch, dt);
              if (!osdn_forward_supported(Dk, Dv, Ch, dt)) {
                CHECK(got == 0);
                continue;
              }
              const size_t p1 = osdn_precond_workspace_bytes(Bq, Hq, Tq, Dk, dt);
              const size_t p2 =
                  osdn_chunk_workspace_bytes(Bq, Hq, Tq, Dk, Dv, Ch, dt);
              size_t kt = (size_t)Bq * Hq * Tq * Dk * (dt ? 2 : 4);
              kt = (kt + 255) / 256 * 256;
              const size_t need =
                  Ch == 64 ? p1 + p2 : kt + (p1 > p2 ? p1 : p2);
              CHECK(got == need);
            }
  }
  /* fp32, Dk = Dv = 64, chunk 64: the two regions side by side */
  CHECK(osdn_forward_workspace_bytes(2, 3, 448, 64, 64, 64, OSDN_F32) ==
        osdn_precond_workspace_bytes(2, 3, 448, 64, OSDN_F32) +
            osdn_chunk_workspace_bytes(2, 3, 448, 64, 64, 64, OSDN_F32));

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

  /* backward entry points: workspace layouts and host-side validation */
  {
    const int Bq = 2, Hq = 3, Tq = 130, K = 128, V = 64;
    const size_t nck = (Tq + 63) / 64, rs = V / 32, st = Tq < 64 ? Tq : 64;
    CHECK(osdn_backward_workspace_bytes(Bq, Hq, Tq, K, V) ==
          (size_t)Bq * Hq *
              ((size_t)Tq * (K + V) + (nck + 1) * V * K + (size_t)Tq * rs * (3 * K + 4)) *
              4);
    CHECK(gdn2_backward_workspace_bytes(Bq, Hq, Tq, K, V) ==
          (size_t)Bq * Hq *
              ((nck + 1 + st) * V * K + (size_t)Tq * rs * (4 * K + 4)) * 4);
    CHECK(osdn_gated_backward_workspace_bytes(Bq, Hq, Tq, K, V) ==
          gdn2_backward_workspace_bytes(Bq, Hq, Tq, K, V) + (size_t)Bq * Hq * Tq * K * 4);
    CHECK(osdn_backward_workspace_bytes(Bq, Hq, Tq, 48, V) == 0);
  }
  {
    const size_t need = osdn_backward_workspace_bytes(1, 1, 4, 32, 32);
    /* dq over q */
    CHECK(osdn_backward(1, 1, 4, 32, 32, OSDN_BF16, P(0x10000), P(0x20000),
                        P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                        P(0x60000), NULL, NULL, P(0x10000 + 8), P(0x200000),
                        P(0x300000), P(0x400000), P(0x500000), P(0x600000),
                        P(0x700000), P(0x900000), P(0x4000000), need,
                        NULL) == OSDN_ERR_ALIASING);
    /* missing dout */
    CHECK(osdn_backward(1, 1, 4, 32, 32, OSDN_BF16, P(0x10000), P(0x20000),
                        P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                        NULL, NULL, NULL, P(0x100000), P(0x200000),
                        P(0x300000), P(0x400000), P(0x500000), P(0x600000),
                        P(0x700000), P(0x900000), P(0x4000000), need,
                        NULL) == OSDN_ERR_NULL_ARG);
    /* workspace too small */
    CHECK(osdn_backward(1, 1, 4, 32, 32, OSDN_BF16, P(0x10000), P(0x20000),
                        P(0x30000), P(0x40000), NULL, 0.1f, NULL, NULL, 1.f,
                        P(0x60000), NULL, NULL, P(0x100000), P(0x200000),
                        P(0x300000), P(0x400000), P(0x500000), P(0x600000),
                        P(0x700000), P(0x900000), P(0x4000000), need - 4,
                        NULL) == OSDN_ERR_WORKSPACE);
    /* GDN-2: the decay's gradient over the decay */
    const size_t ng = gdn2_backward_workspace_bytes(1, 1, 4, 32, 32);
    CHECK(gdn2_backward(1, 1, 4, 32, 32, OSDN_BF16, P(0x10000), P(0x20000),
                        P(0x30000), P(0x80000), P(0x90000), P(0x98000), NULL,
                        1.f, P(0x60000), NULL, P(0x100000), P(0x200000),
                        P(0x300000), P(0x80000), P(0x400000), P(0x500000),
                        P(0x900000), P(0x4000000), ng, NULL) == OSDN_ERR_ALIASING);
    /* gated OSDN: unsupported head dim */
    CHECK(osdn_gated_backward(1, 1, 4, 16, 32, OSDN_BF16, P(0x10000),
                              P(0x20000), P(0x30000), P(0x40000), NULL, 0.1f,
                              P(0x80000), NULL, NULL, 1.f, P(0x60000), NULL,
                              NULL, P(0x100000), P(0x200000), P(0x300000),
                              P(0x400000), P(0x500000), P(0x600000),
                              P(0xa00000), P(0x700000), P(0x900000),
                              P(0x4000000), 1u << 20, NULL) == OSDN_ERR_UNSUPPORTED);
  }

  /* the allocation-free forward rejects sizes beyond its static scratch on
   * the host, before touching any device */
  CHECK(osdn_forward_noalloc(64, 16, 8192, 128, 128, 64, OSDN_BF16, P(0x10000),
                             P(0x20000), P(0x30000), P(0x40000), NULL, 0.1f,
                             NULL, NULL, 1.f, P(0x50000), NULL, NULL, NULL,
                             NULL, NULL) == OSDN_ERR_WORKSPACE);
  CHECK(osdn_forward_noalloc(0, 16, 64, 128, 128, 64, OSDN_BF16, NULL, NULL,
                             NULL, NULL, NULL, 0.1f, NULL, NULL, 1.f, NULL,
                             NULL, NULL, NULL, NULL, NULL) == OSDN_OK);

  /* kernel timing: enabling and reading with nothing recorded */
  osdn_kernel_timing(1);
  CHECK(osdn_kernel_times(0, NULL, NULL, NULL) == 0);
  osdn_kernel_timing(0);

  if (failures == 0) printf("abi_consumer: all checks passed\n");
  return failures;
}
