/* Sanitizer driver for the CPU oracle (test infrastructure).  Built with
 * -fsanitize=address,undefined by tests/test_sanitizers.py, it runs every
 * oracle entry point on small inputs in both dtypes and on the argument
 * errors the oracle must reject with a status, never a crash.  Exit 0 when
 * every status is the expected one. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dspark_oracle.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) {  /* xorshift64*, [0, 1) */
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) * (1.0 / 9007199254740992.0);
}

/* n values of N(0, sd) (Box-Muller) in dtype dt (0 fp32, 1 bf16). */
static void* fill(int dt, size_t n, double sd) {
  void* p = malloc(n * (dt ? 2 : 4));
  for (size_t i = 0; i < n; ++i) {
    const double g = sqrt(-2.0 * log(1.0 - uniform())) * cos(6.283185307179586 * uniform()) * sd;
    if (dt) ((uint16_t*)p)[i] = dspark_oracle_round_bf16((float)g);
    else ((float*)p)[i] = (float)g;
  }
  return p;
}

static int64_t* ids(size_t n, int64_t V) {
  int64_t* p = malloc(n * sizeof(int64_t));
  for (size_t i = 0; i < n; ++i) p[i] = (int64_t)(uniform() * (double)V);
  return p;
}

static void run_dtype(int dt) {
  const int64_t B = 2, M = 5, V = 1024, r = 16, d = 24, rows = B * M;
  const size_t es = dt ? 2 : 4;
  void* base = fill(dt, (size_t)(rows * V), 2.0);
  void* w1 = fill(dt, (size_t)(V * r), 0.02);
  void* w2 = fill(dt, (size_t)(V * r), 0.02);
  void* hid = fill(dt, (size_t)(rows * d), 1.0);
  void* gw = fill(dt, (size_t)(r * (d + r)), 0.2);
  void* gb = fill(dt, (size_t)r, 0.2);
  void* grad = fill(dt, (size_t)(rows * V), 1.0);
  int64_t* tok_ids = ids((size_t)rows, V);
  int64_t* first = ids((size_t)B, V);
  void* out = malloc((size_t)(rows * V) * es);
  void* lat = malloc((size_t)(rows * r) * es);
  void* dw1 = malloc((size_t)(V * r) * es);
  void* dw2 = malloc((size_t)(V * r) * es);
  int64_t tokens[10];
  float lo[8], mid[8], hi[8], lat_lo[16 * 10], lat_hi[16 * 10], score[2];
  const int64_t prow[8] = {0, 1, 2, 3, 4, 5, 6, 9}, pcol[8] = {0, 1, 2, 511, 512, 1000, 1022, 1023};
  int64_t tok = 0, runner = 0;

  expect("apply", dspark_oracle_apply_block(base, dt, tok_ids, w1, w2, dt, B, M, V, r, out, 2), ORACLE_OK);
  expect("apply in place", dspark_oracle_apply_block(out, dt, tok_ids, w1, w2, dt, B, M, V, r, out, 1), ORACLE_OK);
  expect("apply mixed", dspark_oracle_apply_block(base, dt, tok_ids, w1, w2, dt, B, M, V, r, out, 1), ORACLE_OK);
  expect("greedy", dspark_oracle_sample_block(base, dt, first, w1, w2, dt, B, M, V, r, 0.0, 1, 0, 0, tokens, out, 2),
         ORACLE_OK);
  expect("temperature", dspark_oracle_sample_block(base, dt, first, w1, w2, dt, B, M, V, r, 0.7, 1234, 3, 1, tokens,
                                                   NULL, 2), ORACLE_OK);
  expect("select", dspark_oracle_select_token(base, dt, V, 0.7, 5, 0, 0, &tok, score, &runner), ORACLE_OK);
  expect("bounds", dspark_oracle_logit_bounds(base, dt, tok_ids, w1, w2, dt, V, r, 8, prow, pcol, lo, mid, hi),
         ORACLE_OK);
  expect("gated latent", dspark_oracle_gated_latent(hid, dt, d, tok_ids, w1, gw, gb, dt, rows, V, r, lat, lat_lo,
                                                    lat_hi, 2), ORACLE_OK);
  expect("apply rows", dspark_oracle_apply_rows(base, dt, lat, w2, dt, rows, V, r, out, 2), ORACLE_OK);
  expect("bounds rows", dspark_oracle_logit_bounds_rows(base, dt, lat, w2, dt, V, r, 8, prow, pcol, lo, mid, hi),
         ORACLE_OK);
  expect("gated apply", dspark_oracle_apply_block_gated(base, dt, tok_ids, hid, dt, d, w1, w2, gw, gb, dt, B, M, V,
                                                        r, out, lat, 2), ORACLE_OK);
  expect("gated apply, no hidden", dspark_oracle_apply_block_gated(base, dt, tok_ids, NULL, dt, 0, w1, w2, NULL, NULL,
                                                                   dt, B, M, V, r, out, NULL, 1), ORACLE_OK);
  expect("gated sample", dspark_oracle_sample_block_gated(base, dt, first, hid, dt, d, w1, w2, gw, gb, dt, B, M, V,
                                                          r, 0.7, 9, 0, 0, tokens, out, lat, 2), ORACLE_OK);
  expect("backward", dspark_oracle_apply_block_backward(grad, dt, tok_ids, w1, w2, dt, rows, V, r, dw1, dw2, 2),
         ORACLE_OK);
  expect("backward bounds dW2", dspark_oracle_backward_bounds(grad, dt, tok_ids, w1, w2, dt, rows, V, r, 2, 8, pcol,
                                                             prow, lo, mid, hi), ORACLE_OK);
  {
    int64_t which[2] = {tok_ids[0], tok_ids[3]}, cols[2] = {0, 15};
    expect("backward bounds dW1", dspark_oracle_backward_bounds(grad, dt, tok_ids, w1, w2, dt, rows, V, r, 1, 2,
                                                               which, cols, lo, mid, hi), ORACLE_OK);
  }

  /* argument errors: a status, never a crash */
  expect("null base", dspark_oracle_apply_block(NULL, dt, tok_ids, w1, w2, dt, B, M, V, r, out, 1), ORACLE_INVALID);
  expect("null ids", dspark_oracle_apply_block(base, dt, NULL, w1, w2, dt, B, M, V, r, out, 1), ORACLE_INVALID);
  expect("negative B", dspark_oracle_apply_block(base, dt, tok_ids, w1, w2, dt, -1, M, V, r, out, 1), ORACLE_INVALID);
  expect("rank 0", dspark_oracle_apply_block(base, dt, tok_ids, w1, w2, dt, B, M, V, 0, out, 1), ORACLE_INVALID);
  expect("bad dtype", dspark_oracle_apply_block(base, 7, tok_ids, w1, w2, dt, B, M, V, r, out, 1), ORACLE_UNSUPPORTED);
  expect("NaN temperature", dspark_oracle_sample_block(base, dt, first, w1, w2, dt, B, M, V, r, NAN, 1, 0, 0, tokens,
                                                       NULL, 1), ORACLE_INVALID);
  expect("null tokens", dspark_oracle_sample_block(base, dt, first, w1, w2, dt, B, M, V, r, 0.0, 1, 0, 0, NULL, NULL,
                                                   1), ORACLE_INVALID);
  {
    int64_t bad[10];
    memcpy(bad, tok_ids, sizeof(bad));
    bad[3] = V;
    expect("id out of range", dspark_oracle_apply_block(base, dt, bad, w1, w2, dt, B, M, V, r, out, 1),
           ORACLE_INVALID);
    expect("id out of range, bounds", dspark_oracle_logit_bounds(base, dt, bad, w1, w2, dt, V, r, 8, prow, pcol, lo,
                                                                 mid, hi), ORACLE_INVALID);
    expect("id out of range, latent", dspark_oracle_gated_latent(hid, dt, d, bad, w1, gw, gb, dt, rows, V, r, lat,
                                                                 NULL, NULL, 1), ORACLE_INVALID);
    expect("id out of range, gated", dspark_oracle_apply_block_gated(base, dt, bad, hid, dt, d, w1, w2, gw, gb, dt, B,
                                                                     M, V, r, out, NULL, 1), ORACLE_INVALID);
    expect("id out of range, backward", dspark_oracle_apply_block_backward(grad, dt, bad, w1, w2, dt, rows, V, r, dw1,
                                                                           dw2, 1), ORACLE_INVALID);
    bad[3] = -1;
    expect("negative id, backward bounds", dspark_oracle_backward_bounds(grad, dt, bad, w1, w2, dt, rows, V, r, 2, 8,
                                                                        pcol, prow, lo, mid, hi), ORACLE_INVALID);
    expect("negative id, backward bounds dW1", dspark_oracle_backward_bounds(grad, dt, bad, w1, w2, dt, rows, V, r, 1,
                                                                            8, pcol, prow, lo, mid, hi),
           ORACLE_INVALID);
    int64_t badfirst[2] = {first[0], -5};
    expect("first id out of range", dspark_oracle_sample_block(base, dt, badfirst, w1, w2, dt, B, M, V, r, 0.0, 1, 0,
                                                               0, tokens, NULL, 1), ORACLE_INVALID);
    expect("first id out of range, gated", dspark_oracle_sample_block_gated(base, dt, badfirst, hid, dt, d, w1, w2,
                                                                            gw, gb, dt, B, M, V, r, 0.0, 1, 0, 0,
                                                                            tokens, NULL, NULL, 1), ORACLE_INVALID);
  }
  expect("gated, missing gate", dspark_oracle_apply_block_gated(base, dt, tok_ids, hid, dt, d, w1, w2, NULL, gb, dt,
                                                                B, M, V, r, out, NULL, 1), ORACLE_INVALID);
  expect("backward, bad kind", dspark_oracle_backward_bounds(grad, dt, tok_ids, w1, w2, dt, rows, V, r, 3, 8, pcol,
                                                            prow, lo, mid, hi), ORACLE_INVALID);
  /* empty work */
  expect("empty apply", dspark_oracle_apply_block(base, dt, tok_ids, w1, w2, dt, 0, M, V, r, out, 1), ORACLE_OK);
  expect("empty sample", dspark_oracle_sample_block(base, dt, first, w1, w2, dt, B, 0, V, r, 0.0, 1, 0, 0, tokens,
                                                    NULL, 1), ORACLE_OK);

  free(base); free(w1); free(w2); free(hid); free(gw); free(gb); free(grad);
  free(tok_ids); free(first); free(out); free(lat); free(dw1); free(dw2);
}

int main(void) {
  run_dtype(ORACLE_F32);
  run_dtype(ORACLE_BF16);
  {
    const uint32_t ctr[4] = {0, 0, 0, 0}, key[2] = {0, 0};
    uint32_t o[4];
    dspark_oracle_philox4x32_10(ctr, key, o);
    (void)dspark_oracle_gumbel2(1, 0, 0, 5);
    (void)dspark_oracle_kappa(0.7);
  }
  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("oracle driver: all statuses as expected\n");
  return 0;
}
