/* Sanitizer driver for the host side of the C ABI (test infrastructure).
 * Built host-only with -fsanitize=address,undefined by
 * tests/test_sanitizers.py, it queries the workspace sizes and makes calls
 * whose arguments the host validation must reject, so that no call reaches
 * a kernel launch: it runs without a GPU.  Exit 0 when every status is the
 * expected one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "dspark_markov.h"

static int failures = 0;
static char fake[4096] __attribute__((aligned(256)));   /* never dereferenced: every call is rejected */
#define F ((void*)fake)
#define FI ((int64_t*)fake)

static void expect(const char* what, dspark_status_t got, dspark_status_t want) {
  if (got != want) {
    fprintf(stderr, "%s: %s, expected %s (%s)\n", what, dspark_status_string(got), dspark_status_string(want),
            dspark_markov_last_error());
    ++failures;
  }
}

int main(void) {
  const int64_t B = 2, M = 3, V = 64, r = 16, d = 32;
  const dspark_dtype_t bf = DSPARK_BF16;
  const size_t ws = dspark_markov_workspace_bytes(B, M, V, r, 1);
  const size_t gws = dspark_markov_gated_workspace_bytes(B, M, V, r, d, 0);
  const size_t bws = dspark_markov_backward_workspace_bytes(B, M, V, r);
  if (ws == 0 || gws == 0 || bws == 0) {
    fprintf(stderr, "zero workspace size\n");
    ++failures;
  }
  /* sizes that cannot be represented: SIZE_MAX, never a wrapped small size */
  if (dspark_markov_workspace_bytes(INT64_MAX / 2, 2, 1 << 20, 512, 1) != SIZE_MAX ||
      dspark_markov_workspace_bytes(1 << 20, 2, INT64_MAX, 512, 1) != SIZE_MAX ||
      dspark_markov_gated_workspace_bytes(INT64_MAX / 8, 16, 1 << 20, 512, 1 << 12, 0) != SIZE_MAX ||
      dspark_markov_gated_workspace_bytes(1 << 20, 4, 1 << 20, 512, INT64_MAX / 4, 1) != SIZE_MAX ||
      dspark_markov_backward_workspace_bytes(INT64_MAX / 4, 4, 1 << 20, 512) != SIZE_MAX ||
      dspark_markov_backward_workspace_bytes(1 << 30, 1 << 20, 1 << 20, 512) != SIZE_MAX) {
    fprintf(stderr, "an unrepresentable workspace size did not saturate\n");
    ++failures;
  }
  /* the sampling workspace does not grow with the block length */
  if (dspark_markov_workspace_bytes(4, INT64_MAX / 2, 1 << 20, 512, 1) != dspark_markov_workspace_bytes(4, 2, 1 << 20, 512, 1)) {
    fprintf(stderr, "the sampling workspace depends on M\n");
    ++failures;
  }

  /* apply */
  expect("apply null base", dspark_markov_apply_block(NULL, bf, FI, F, F, bf, B, M, V, r, F, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply null ids", dspark_markov_apply_block(F, bf, NULL, F, F, bf, B, M, V, r, F, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply bad dtype", dspark_markov_apply_block(F, (dspark_dtype_t)9, FI, F, F, bf, B, M, V, r, F, F, 1 << 20,
                                                      NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply rank 0", dspark_markov_apply_block(F, bf, FI, F, F, bf, B, M, V, 0, F, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply negative M", dspark_markov_apply_block(F, bf, FI, F, F, bf, B, -1, V, r, F, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply overflowing sizes", dspark_markov_apply_block(F, bf, FI, F, F, bf, INT64_MAX / 2, 4, V, r, F, F,
                                                              1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("apply small workspace", dspark_markov_apply_block(F, bf, FI, F, F, bf, B, M, V, r, F, F, 8, NULL),
         DSPARK_ERR_WORKSPACE_TOO_SMALL);
  expect("apply empty", dspark_markov_apply_block(F, bf, FI, F, F, bf, 0, M, V, r, F, F, 1 << 20, NULL), DSPARK_OK);

  /* sample */
  int64_t* tok = FI;
  expect("sample NaN temperature", dspark_markov_sample_block(F, bf, FI, F, F, bf, B, M, V, r, NAN, 0, 0, 0, tok, NULL,
                                                              F, 1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("sample null tokens", dspark_markov_sample_block(F, bf, FI, F, F, bf, B, M, V, r, 0.0, 0, 0, 0, NULL, NULL,
                                                          F, 1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("sample null first", dspark_markov_sample_block(F, bf, NULL, F, F, bf, B, M, V, r, 0.0, 0, 0, 0, tok, NULL,
                                                         F, 1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("sample null workspace", dspark_markov_sample_block(F, bf, FI, F, F, bf, B, M, V, r, 0.0, 0, 0, 0, tok, NULL,
                                                             NULL, 1 << 20, NULL), DSPARK_ERR_WORKSPACE_TOO_SMALL);
  expect("sample empty", dspark_markov_sample_block(F, bf, FI, F, F, bf, B, 0, V, r, 0.0, 0, 0, 0, tok, NULL, F,
                                                    1 << 20, NULL), DSPARK_OK);

  /* gated */
  expect("gated apply no gate weight", dspark_markov_apply_block_gated(F, bf, FI, F, bf, d, F, F, NULL, F, bf, B, M,
                                                                       V, r, F, NULL, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);
  expect("gated apply bad hidden dtype", dspark_markov_apply_block_gated(F, bf, FI, F, (dspark_dtype_t)5, d, F, F, F,
                                                                         F, bf, B, M, V, r, F, NULL, F, 1 << 20,
                                                                         NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("gated apply small workspace", dspark_markov_apply_block_gated(F, bf, FI, F, bf, d, F, F, F, F, bf, B, M, V,
                                                                        r, F, NULL, F, 16, NULL),
         DSPARK_ERR_WORKSPACE_TOO_SMALL);
  expect("gated sample NaN", dspark_markov_sample_block_gated(F, bf, FI, F, bf, d, F, F, F, F, bf, B, M, V, r, NAN, 0,
                                                              0, 0, tok, NULL, NULL, F, 1 << 20, NULL),
         DSPARK_ERR_INVALID_ARGUMENT);

  /* backward */
  expect("backward null grad", dspark_markov_apply_block_backward(NULL, bf, FI, F, F, bf, B, M, V, r, F, F, F,
                                                                  1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("backward null outputs", dspark_markov_apply_block_backward(F, bf, FI, F, F, bf, B, M, V, r, NULL, F, F,
                                                                     1 << 20, NULL), DSPARK_ERR_INVALID_ARGUMENT);
  expect("backward small workspace", dspark_markov_apply_block_backward(F, bf, FI, F, F, bf, B, M, V, r, F,
                                                                        (char*)F + 2048, F, 8, NULL),
         DSPARK_ERR_WORKSPACE_TOO_SMALL);

  /* status strings, including an unknown code */
  for (int s = 0; s <= 5; ++s)
    if (!dspark_status_string((dspark_status_t)s)) ++failures;
  (void)dspark_markov_last_error();

  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("ABI driver: all statuses as expected\n");
  return 0;
}
