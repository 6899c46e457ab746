/*
 * Test driver: the host side of libssd's C ABI (argument checks, workspace
 * layouts, path choice, status strings) under AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Only calls that return before any HIP call
 * are made: size queries, and entry-point calls every one of which fails
 * validation (fake, non-dereferenced pointers).  Built and run by
 * tests/test_sanitizers.py; exits 0 when every result is as expected.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "ssd.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static void* P(uintptr_t a) { return (void*)a; }

int main(void) {
  /* size queries over a grid of shapes, including sizes near the limits */
  const int64_t bs[] = {0, 1, 2, 7, 65535, 65536, INT64_MAX / 2};
  const int64_t ls[] = {0, 1, 16, 17, 255, 256, 2049, 65536, (int64_t)1 << 40};
  const int64_t hs[] = {1, 4, 6, 64, 128, 65535, 65536};
  const int64_t ns[] = {16, 24, 64, 128, 256};
  const int qs[] = {32, 64, 128, 256};
  const int gs[] = {1, 2, 3, 8};
  size_t checksum = 0;
  for (int ib = 0; ib < 7; ++ib)
    for (int il = 0; il < 9; ++il)
      for (int ih = 0; ih < 7; ++ih)
        for (int in = 0; in < 5; ++in)
          for (int iq = 0; iq < 4; ++iq)
            for (int ig = 0; ig < 4; ++ig)
              for (int dt = 0; dt < 3; ++dt) {
                const int64_t b = bs[ib], L = ls[il], H = hs[ih], N = ns[in];
                const int Q = qs[iq], G = gs[ig];
                checksum += ssd_scan_fwd_workspace_size(b, L, H, 64, N, G, Q, dt);
                checksum += ssd_scan_fwd_varlen_workspace_size(b, L, H, 64, N, G, Q, dt);
                checksum += ssd_scan_bwd_workspace_size(b, L, H, 64, N, G, Q, dt);
                checksum += ssd_split_conv1d_scan_fwd_workspace_size(b, L, H, 64, N, G, Q, dt,
                                                                     4, 1);
                for (int path = -1; path <= 7; ++path) {
                  checksum += ssd_scan_fwd_path_workspace_size(b, L, H, 64, N, G, Q, dt, 0,
                                                               path);
                  checksum += (size_t)ssd_scan_fwd_taken_path(b, L, H, 64, N, G, Q, dt, 1,
                                                              path);
                }
              }
  printf("size queries: checksum %zu\n", checksum);

  /* rejected calls: nothing is launched */
  CHECK(ssd_scan_fwd(NULL, P(0x2000), (float*)P(0x3000), P(0x4000), P(0x5000), NULL, NULL, NULL,
                     0.f, INFINITY, 64, 1, NULL, P(0x9000), NULL, 1, 100, 4, 64, 16, SSD_F32,
                     NULL, 0, NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                     P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 3, NULL,
                     P(0x60000000), NULL, 1, 100, 4, 64, 16, SSD_F32, NULL, 0,
                     NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                     P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 1, NULL,
                     P(0x60000000), NULL, 1, 100, 4, 64, 16, SSD_F32, NULL, 0,
                     NULL) == SSD_ERR_WORKSPACE);
  CHECK(ssd_scan_fwd(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                     P(0x50000000), NULL, NULL, NULL, NAN, INFINITY, 64, 1, NULL,
                     P(0x60000000), NULL, 1, 100, 4, 64, 16, SSD_F32, NULL, 0,
                     NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                     P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 1, NULL,
                     P(0x10000100), NULL, 1, 100, 4, 64, 16, SSD_F32, NULL, 0,
                     NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                     P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 1, NULL,
                     P(0x60000000), NULL, 1, (int64_t)1 << 40, 65535, 64, 128, SSD_F32, NULL, 0,
                     NULL) != SSD_OK);
  CHECK(ssd_scan_fwd_path(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                          P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 1, NULL,
                          P(0x60000000), NULL, NULL, 1, 100, 4, 64, 16, SSD_F32, 9, NULL, 0,
                          NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd_varlen(P(0x10000000), P(0x20000000), (float*)P(0x30000000), P(0x40000000),
                            P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64, 1, NULL,
                            P(0x60000000), NULL, NULL, 1, 100, 4, 64, 16, SSD_F32, NULL, 0,
                            NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd_noalloc(P(0x10000000), P(0x20000000), (float*)P(0x30000000),
                             P(0x40000000), P(0x50000000), NULL, NULL, NULL, 0.f, INFINITY, 64,
                             3, NULL, P(0x60000000), NULL, 1, 100, 4, 64, 16, SSD_F32,
                             NULL) == SSD_ERR_INVALID_ARG);
  CHECK(ssd_scan_fwd_wait_status(NULL, 0, 1, 100, 4, 64, 16, 3, 64, 0, 0, 0, NULL) ==
        SSD_ERR_INVALID_ARG);
  for (int s = -8; s <= 1; ++s) CHECK(ssd_status_string(s) != NULL);
  CHECK(ssd_abi_version() == SSD_ABI_VERSION);
  puts("abi sanitizer driver: ok");
  return 0;
}
