/*
 * The C ABI of libfa2 as a C program sees it: include/fa2.h compiled as C99 by
 * the host C compiler, the library linked by name. Every call below either
 * fails argument validation or is an empty problem, both of which return
 * before any HIP call, so the program needs no GPU and launches nothing; the
 * pointers it passes are never dereferenced. Prints one line per failed
 * expectation and exits with the number of failures.
 */
#include <stdio.h>
#include <string.h>

#include "fa2.h"

static int failures = 0;

#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                  \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static size_t up256(size_t x) { return (x + 255) / 256 * 256; }

int main(void) {
  static char dummy[256] __attribute__((aligned(256)));
  void* P = dummy;         /* 16-byte aligned, never dereferenced */
  void* M = dummy + 4;     /* misaligned */
  float* F = (float*)P;
  const int* cu = (const int*)P;
  const unsigned char* mask = (const unsigned char*)P;
  const size_t WS = 1 << 20;

  /* status strings and version */
  EXPECT(fa2_status_string(FA2_OK) != NULL && strlen(fa2_status_string(FA2_OK)) > 0);
  EXPECT(strcmp(fa2_status_string(FA2_OK), fa2_status_string(FA2_ERR_HIP)) != 0);
  EXPECT(fa2_status_string((fa2_status_t)99) != NULL);
  EXPECT(fa2_version() >= 100);

  /* the allocation-free backward refuses more rows than its scratch array holds, before any HIP call */
  EXPECT(fa2_bwd_noalloc(P, P, P, P, F, P, P,
                         P, P, 4, 32, 16385, 128, 0.088f, 1, -1, -1, NULL, NULL) == FA2_ERR_UNSUPPORTED);

  /* effective window: a side reaching every key is unbounded, causal clamps the right side */
  {
    int l = 7, r = 7;
    EXPECT(fa2_effective_window(100, 0, 2147483647, 2147483647, &l, &r) == FA2_OK && l == -1 && r == -1);
    EXPECT(fa2_effective_window(100, 1, 40, 9, &l, &r) == FA2_OK && l == 40 && r == 0);
    EXPECT(fa2_effective_window(100, 0, -2, 0, &l, &r) == FA2_ERR_INVALID_ARG);
    EXPECT(fa2_effective_window(100, 0, 0, 0, NULL, &r) == FA2_ERR_INVALID_ARG);
  }

  /* workspace sizes: two per-row float arrays, then the float32 dQ accumulator */
  EXPECT(fa2_bwd_workspace_size(4, 32, 8192, 128) ==
         2 * up256((size_t)4 * 32 * 8192 * 4) + up256((size_t)4 * 32 * 8192 * 128 * 4));
  EXPECT(fa2_bwd_workspace_size(1, 1, 17, 64) == 2 * up256(17 * 4) + up256(17 * 64 * 4));
  EXPECT(fa2_bwd_workspace_size(0, 1, 17, 64) == 0);
  EXPECT(fa2_bwd_workspace_size(1, 1, 17, 96) == 0);

  /* forward: validation before any launch */
  EXPECT(fa2_fwd(NULL, P, P, P, F, 1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd(M, P, P, P, F, 1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd(P, P, P, P, F, 1, 2, 16, 96, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_UNSUPPORTED);
  EXPECT(fa2_fwd(P, P, P, P, F, 1, 2, 16, 64, 0.0f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd(P, P, P, P, F, 1, 2, 16, 64, 0.125f, 0, -2, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd(P, P, P, P, F, -1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd(P, P, P, P, F, 0, 2, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_OK);
  EXPECT(fa2_fwd_f32(F, F, F, F, F, 1, 2, 16, 96, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_UNSUPPORTED);
  EXPECT(fa2_fwd_f32(F, F, F, F, F, 1, 0, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_OK);

  /* backward and its passes */
  EXPECT(fa2_bwd(P, P, P, P, NULL, P, P, P, P, P, WS, 1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, 1, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd(P, P, P, P, F, P, P, P, P, P, 8, 1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, 1, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd(P, P, P, P, F, P, P, P, P, NULL, 0, 0, 2, 16, 64, 0.125f, 1, -1, -1, NULL, 1, NULL) == FA2_OK);
  EXPECT(fa2_bwd_prep(P, P, NULL, P, WS, 1, 2, 16, 64, 0.125f, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd_prep(P, P, F, P, 256, 1, 2, 16, 64, 0.125f, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd_dkdv(P, P, P, F, P, NULL, P, P, WS, 1, 2, 16, 64, 0.125f, 1, -1, -1, NULL, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd_dq(P, P, P, F, P, P, P, WS, 1, 2, 16, 128, -1.0f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);

  /* packed batches */
  EXPECT(fa2_fwd_varlen(P, P, P, P, F, NULL, 3, 100, 2, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_varlen(P, P, P, P, F, cu, 0, 100, 2, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_varlen(P, P, P, P, F, cu, 3, 0, 2, 64, 0.125f, 1, -1, -1, NULL, NULL) == FA2_OK);
  EXPECT(fa2_bwd_varlen(P, P, P, P, F, P, P, P, P, cu, P, 16, 3, 100, 2, 64, 0.125f, 1, -1, -1, NULL, NULL) ==
         FA2_ERR_INVALID_ARG);

  /* block-sparse batches */
  EXPECT(fa2_fwd_blocksparse(P, P, P, P, F, 1, 2, 300, 64, 0.125f, 1, -1, -1, NULL, NULL, 0, 9, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_blocksparse(P, P, P, P, F, 1, 2, 300, 64, 0.125f, 1, -1, -1, NULL, mask, -1, 9, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_blocksparse(P, P, P, P, F, 1, 2, 70000, 64, 0.125f, 1, -1, -1, NULL, mask, 0, 0, NULL) ==
         FA2_ERR_UNSUPPORTED);
  EXPECT(fa2_bwd_blocksparse(P, P, P, P, F, P, P, P, P, P, 0, 0, 2, 300, 64, 0.125f, 1, -1, -1, NULL, mask, 0, 9,
                             NULL) == FA2_OK);

  /* dropout */
  EXPECT(fa2_fwd_dropout(P, P, P, P, F, 1, 2, 300, 128, 0.125f, 1, -1, -1, NULL, 1.0f, 1, 0, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_dropout(P, P, P, P, F, 1, 2, 300, 128, 0.125f, 1, -1, -1, NULL, -0.1f, 1, 0, NULL) ==
         FA2_ERR_INVALID_ARG);
  EXPECT(fa2_bwd_dropout(P, P, P, P, F, P, P, P, P, P, 100, 1, 2, 300, 128, 0.125f, 1, -1, -1, NULL, 0.1f, 1, 0,
                         NULL) == FA2_ERR_INVALID_ARG);
  EXPECT(fa2_fwd_dropout(P, P, P, P, F, 0, 2, 300, 128, 0.125f, 1, -1, -1, NULL, 0.1f, 1, 0, NULL) == FA2_OK);
  /* the offset is the generator's 32-bit counter word */
  EXPECT(fa2_fwd_dropout(P, P, P, P, F, 0, 2, 300, 128, 0.125f, 1, -1, -1, NULL, 0.1f, 1, 1ull << 32, NULL) ==
         FA2_ERR_INVALID_ARG);

  printf("%d failure(s)\n", failures);
  return failures;
}
