/*
 * dspark_oracle.c -- plain, slow CPU oracle for the vanilla DSpark low-rank
 * Markov head.  TEST INFRASTRUCTURE: only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it.  It shares no code with the GPU
 * library.  Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math), so that
 * every float operation below is the IEEE operation it is written as.
 *
 * Each function names the passage of the DSpark pages that it follows:
 *   [P5] third-party markov_head.py (raw page): module docstring,
 *        _sample_tokens, VanillaMarkov and its methods, build_markov_head.
 *   [P3] NeMo AutoModel "speculative/dspark/markov_head" API page.
 *   [P1] NeMo AutoModel "models/deepseek_v41/dspark" API page.
 * Where the pages are silent the reading taken is stated at the function.
 */
#include "dspark_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                     */
/* ------------------------------------------------------------------ */

static float bits_to_float(uint32_t u) {
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

static uint32_t float_to_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return u;
}

/* bfloat16 keeps the upper 16 bits of an IEEE binary32 value. */
static float bf16_to_float(uint16_t h) { return bits_to_float((uint32_t)h << 16); }

/* Round a binary32 value to the nearest bfloat16, ties to the even
 * neighbour (the rounding torch uses for .to(torch.bfloat16)); every NaN
 * becomes the canonical quiet NaN 0x7FC0.  Written from the definition:
 * keep the upper half, then decide from the discarded lower half. */
uint16_t dspark_oracle_round_bf16(float x) {
  uint32_t u = float_to_bits(x);
  if (isnan(x)) return (uint16_t)0x7FC0u;
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept; /* a carry out of the mantissa steps the exponent */
}

/* Value of element i of an array of dtype `dt`, widened exactly to double. */
static double load_as_double(const void* p, int dt, int64_t i) {
  if (dt == ORACLE_F32) return (double)((const float*)p)[i];
  return (double)bf16_to_float(((const uint16_t*)p)[i]);
}

static float load_as_float(const void* p, int dt, int64_t i) {
  if (dt == ORACLE_F32) return ((const float*)p)[i];
  return bf16_to_float(((const uint16_t*)p)[i]);
}

/* Round a float to dtype dt and return the rounded value as a float. */
static float round_to(float x, int dt) {
  if (dt == ORACLE_F32) return x;
  return bf16_to_float(dspark_oracle_round_bf16(x));
}

static void store_from_float(void* p, int dt, int64_t i, float x) {
  /* x is already representable in dt */
  if (dt == ORACLE_F32)
    ((float*)p)[i] = x;
  else
    ((uint16_t*)p)[i] = (uint16_t)(float_to_bits(x) >> 16);
}

static int valid_dtype(int dt) { return dt == ORACLE_F32 || dt == ORACLE_BF16; }

/* ------------------------------------------------------------------ */
/* The bias and the corrected logit  ([P5] module docstring:          */
/* B(x_{k-1},:) = W2(W1[x_{k-1}]), corrected logit U_k + B)            */
/* ------------------------------------------------------------------ */

/* [P5] VanillaMarkov.get_prev_embeddings: e = W1[x]  (Embedding lookup). */
static void gather_w1_row(const void* w1, int wdt, int64_t r, int64_t x, double* e) {
  for (int64_t j = 0; j < r; ++j) e[j] = load_as_double(w1, wdt, x * r + j);
}

/* [P5] VanillaMarkov.project_bias: Linear(r, V, bias=False) applied to e,
 * i.e. a_v = sum_j e_j * W2w[v, j] with W2w the Linear weight [V, r].
 * Reading: fp32 accumulation is modelled by its best value, the double sum
 * (products of bf16/fp32 values are exact in double) rounded once to fp32.
 * The Linear emits the weight dtype W. */
static float projected_bias(const double* e, const double* w2_row, int64_t r) {
  double a = 0.0;
  for (int64_t j = 0; j < r; ++j) a += e[j] * w2_row[j];
  return (float)a;
}

/* [P5] apply_step_logits / apply_block_logits: logits + bias.to(logits.dtype).
 * Reading: the bias is first rounded to W (Linear output), then to L (the
 * .to cast), then added in fp32 and rounded once to L (torch's
 * reduced-precision add: upcast, add, round). */
static float corrected_value(float base_v, float acc_v, int ldt, int wdt) {
  float bias = round_to(round_to(acc_v, wdt), ldt);
  float sum = base_v + bias;
  return round_to(sum, ldt);
}

/* W2w converted once to double, [V, r]. */
static double* w2_as_double(const void* w2, int wdt, int64_t V, int64_t r) {
  double* d = (double*)malloc((size_t)(V * r) * sizeof(double));
  if (!d) return NULL;
  for (int64_t i = 0; i < V * r; ++i) d[i] = load_as_double(w2, wdt, i);
  return d;
}

/* One corrected row: base row (length V, dtype ldt) biased by the
 * projection of the latent row e[r] (W1[x] for the vanilla head).  Writes
 * the L-typed results as floats into out[V]. */
static void corrected_row_from(const void* base, int ldt, int64_t base_row,
                               const double* w2d, int wdt, int64_t V, int64_t r,
                               const double* e, float* out) {
  for (int64_t v = 0; v < V; ++v) {
    float acc = projected_bias(e, w2d + v * r, r);
    float b = load_as_float(base, ldt, base_row * V + v);
    out[v] = corrected_value(b, acc, ldt, wdt);
  }
}

/* One corrected row biased by token x (vanilla head). */
static void corrected_row(const void* base, int ldt, int64_t base_row,
                          const void* w1, const double* w2d, int wdt, int64_t V,
                          int64_t r, int64_t x, double* e, float* out) {
  gather_w1_row(w1, wdt, r, x, e);
  corrected_row_from(base, ldt, base_row, w2d, wdt, V, r, e, out);
}


static int n_threads_or_default(int n) { return n > 0 ? n : omp_get_max_threads(); }

/* [P5] VanillaMarkov.apply_block_logits (teacher-forced): every row (b, k)
 * is biased by its own token_ids[b, k].  Shape-agnostic over leading dims,
 * so [B, M] rows are processed independently.  An empty input (numel()==0
 * or M==0) returns the input unchanged: nothing is written.
 * [P5] VanillaMarkov.__init__ asserts markov_rank > 0: r <= 0 is invalid.
 * Out-of-range ids (the Embedding lookup would raise) are invalid. */
int dspark_oracle_apply_block(const void* base_logits, int logits_dtype,
                              const int64_t* token_ids, const void* w1,
                              const void* w2, int weight_dtype, int64_t B,
                              int64_t M, int64_t V, int64_t r,
                              void* corrected_logits, int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (B < 0 || M < 0 || V < 0 || r <= 0) return ORACLE_INVALID;
  int64_t rows = B * M;
  if (rows == 0 || V == 0) return ORACLE_OK; /* numel() == 0: return base */
  if (!base_logits || !token_ids || !w1 || !w2 || !corrected_logits) return ORACLE_INVALID;
  for (int64_t n = 0; n < rows; ++n)
    if (token_ids[n] < 0 || token_ids[n] >= V) return ORACLE_INVALID;

  double* w2d = w2_as_double(w2, weight_dtype, V, r);
  if (!w2d) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
#pragma omp parallel num_threads(nt)
  {
    double* e = (double*)malloc((size_t)r * sizeof(double));
    float* out = (float*)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < rows; ++n) {
      corrected_row(base_logits, logits_dtype, n, w1, w2d, weight_dtype, V, r,
                    token_ids[n], e, out);
      for (int64_t v = 0; v < V; ++v)
        store_from_float(corrected_logits, logits_dtype, n * V + v, out[v]);
    }
    free(out);
    free(e);
  }
  free(w2d);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Sampling ([P5] _sample_tokens)                                      */
/* ------------------------------------------------------------------ */

/* Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds;
 * each round multiplies words 0 and 2 by the Philox multipliers, swaps and
 * xors the high halves with the other words and the round key; the key is
 * advanced by the Weyl constants (golden ratio, sqrt(3)-1) between rounds. */
void dspark_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                 uint32_t out[4]) {
  const uint32_t mul0 = 0xD2511F53u, mul1 = 0xCD9E8D57u;
  const uint32_t weyl0 = 0x9E3779B9u, weyl1 = 0xBB67AE85u;
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += weyl0;
      k1 += weyl1;
    }
    uint64_t p0 = (uint64_t)mul0 * (uint64_t)x0;
    uint64_t p2 = (uint64_t)mul1 * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi2 = (uint32_t)(p2 >> 32), lo2 = (uint32_t)p2;
    uint32_t y0 = hi2 ^ x1 ^ k0;
    uint32_t y1 = lo2;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0;
    x1 = y1;
    x2 = y2;
    x3 = y3;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

/* Base-2 Gumbel noise for vocabulary entry v of row (b_abs, k_abs).
 * Reading (the pages draw with torch.multinomial, which no two devices
 * reproduce): the 32-bit word (v mod 4) of Philox4x32-10 with counter
 * (v div 4, k_abs, b_abs, 0) and key (low, high halves of seed) gives the
 * odd 24-bit uniform u = (2*(w >> 9) + 1) * 2^-24, which is never 0 or 1;
 * the noise is -log2(-log2(u)). */
float dspark_oracle_gumbel2(uint64_t seed, int64_t b_abs, int64_t k_abs, int64_t v) {
  uint32_t ctr[4] = {(uint32_t)((uint64_t)v >> 2), (uint32_t)k_abs, (uint32_t)b_abs, 0u};
  uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
  uint32_t w[4];
  dspark_oracle_philox4x32_10(ctr, key, w);
  uint32_t word = w[v & 3];
  float u = ldexpf((float)(2u * (word >> 9) + 1u), -24);
  return -log2f(-log2f(u));
}

/* Scale of the base-2 Gumbel-max score: log2(e)/T computed in double and
 * rounded once to fp32. */
float dspark_oracle_kappa(double temperature) {
  return (float)(1.4426950408889634 / temperature);
}

/* True when a ranks above b under argmax: NaN above everything (torch's
 * argmax returns a NaN's index), otherwise the usual order; +0 and -0 tie. */
static int ranks_above(float a, float b) {
  if (isnan(b)) return 0;
  if (isnan(a)) return 1;
  return a > b;
}

/* [P5] _sample_tokens.  Greedy when temperature < 1e-5 (the pages also map
 * None to greedy): argmax over the L-typed corrected values, first index on
 * ties (torch.argmax's convention).  Otherwise the pages draw one sample
 * from softmax(logits / T); this oracle draws the same law by Gumbel-max:
 * the smallest v maximising fmaf(c_v, log2(e)/T, g_v), which is argmax of
 * c_v/T + Gumbel noise scaled by log2(e) (Gumbel 1954; Maddison, Tarlow and
 * Minka 2014). */
static void select_from_row(const float* c, int64_t V, double temperature,
                            uint64_t seed, int64_t b_abs, int64_t k_abs,
                            int64_t* token, float* best_second, int64_t* second_idx) {
  int greedy = temperature < 1e-5;
  float kappa = greedy ? 0.0f : dspark_oracle_kappa(temperature);
  int64_t best = -1, second = -1;
  float sb = 0.0f, ss = 0.0f;
  for (int64_t v = 0; v < V; ++v) {
    float s = greedy ? c[v] : fmaf(c[v], kappa, dspark_oracle_gumbel2(seed, b_abs, k_abs, v));
    if (best < 0 || ranks_above(s, sb)) {
      second = best;
      ss = sb;
      best = v;
      sb = s;
    } else if (second < 0 || ranks_above(s, ss)) {
      second = v;
      ss = s;
    }
  }
  *token = best;
  if (best_second) {
    best_second[0] = sb;
    best_second[1] = ss;
  }
  if (second_idx) *second_idx = second;
}

int dspark_oracle_select_token(const void* row, int logits_dtype, int64_t V,
                               double temperature, uint64_t seed, int64_t b_abs,
                               int64_t k_abs, int64_t* token, float* score_out,
                               int64_t* runner_up) {
  if (!valid_dtype(logits_dtype)) return ORACLE_UNSUPPORTED;
  if (!row || !token || V <= 0 || isnan(temperature)) return ORACLE_INVALID;
  float* c = (float*)malloc((size_t)V * sizeof(float));
  if (!c) return ORACLE_INVALID;
  for (int64_t v = 0; v < V; ++v) c[v] = load_as_float(row, logits_dtype, v);
  select_from_row(c, V, temperature, seed, b_abs, k_abs, token, score_out, runner_up);
  free(c);
  return ORACLE_OK;
}

/* dspark_oracle_select_token for n rows [n, V] at once (rows in parallel):
 * row i draws with noise indices (b_abs[i], k_abs[i]); scores [n, 2] and
 * runner_up [n] may be NULL. */
int dspark_oracle_select_tokens(const void* rows, int logits_dtype, int64_t n, int64_t V,
                                double temperature, uint64_t seed, const int64_t* b_abs,
                                const int64_t* k_abs, int64_t* tokens, float* scores,
                                int64_t* runner_up, int n_threads) {
  if (!valid_dtype(logits_dtype)) return ORACLE_UNSUPPORTED;
  if (n < 0 || V <= 0 || isnan(temperature)) return ORACLE_INVALID;
  if (n == 0) return ORACLE_OK;
  if (!rows || !b_abs || !k_abs || !tokens) return ORACLE_INVALID;
  const size_t esz = logits_dtype == ORACLE_F32 ? 4 : 2;
  int nt = n_threads_or_default(n_threads);
#pragma omp parallel num_threads(nt)
  {
    float* c = (float*)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n; ++i) {
      const void* row = (const char*)rows + (size_t)(i * V) * esz;
      for (int64_t v = 0; v < V; ++v) c[v] = load_as_float(row, logits_dtype, v);
      select_from_row(c, V, temperature, seed, b_abs[i], k_abs[i], tokens + i,
                      scores ? scores + 2 * i : NULL, runner_up ? runner_up + i : NULL);
    }
    free(c);
  }
  return ORACLE_OK;
}

/* [P5] VanillaMarkov.sample_block_tokens: left to right, step k biases
 * base[:, k, :] by the previous token (first_prev for k = 0, the token just
 * drawn at k-1 after that), keeps the corrected row and draws the next token
 * with _sample_tokens.  proposal_len == 0 returns an empty token array and
 * the input.  NaN temperature is rejected (reading: the pages would sample
 * from NaN probabilities). */
int dspark_oracle_sample_block(const void* base_logits, int logits_dtype,
                               const int64_t* first_prev_token_ids,
                               const void* w1, const void* w2, int weight_dtype,
                               int64_t B, int64_t M, int64_t V, int64_t r,
                               double temperature, uint64_t seed,
                               int64_t position_offset, int64_t batch_offset,
                               int64_t* sampled_tokens, void* corrected_logits,
                               int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (B < 0 || M < 0 || V < 0 || r <= 0 || isnan(temperature)) return ORACLE_INVALID;
  if (B == 0 || M == 0) return ORACLE_OK;
  if (V == 0) return ORACLE_INVALID; /* nothing to draw from */
  if (!base_logits || !first_prev_token_ids || !w1 || !w2 || !sampled_tokens)
    return ORACLE_INVALID;
  for (int64_t b = 0; b < B; ++b)
    if (first_prev_token_ids[b] < 0 || first_prev_token_ids[b] >= V) return ORACLE_INVALID;

  double* w2d = w2_as_double(w2, weight_dtype, V, r);
  if (!w2d) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
  for (int64_t k = 0; k < M; ++k) {
#pragma omp parallel num_threads(nt)
    {
      double* e = (double*)malloc((size_t)r * sizeof(double));
      float* out = (float*)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
      for (int64_t b = 0; b < B; ++b) {
        int64_t prev = (k == 0) ? first_prev_token_ids[b] : sampled_tokens[b * M + k - 1];
        int64_t row = b * M + k;
        corrected_row(base_logits, logits_dtype, row, w1, w2d, weight_dtype, V, r, prev, e, out);
        if (corrected_logits)
          for (int64_t v = 0; v < V; ++v)
            store_from_float(corrected_logits, logits_dtype, row * V + v, out[v]);
        int64_t tok;
        select_from_row(out, V, temperature, seed, batch_offset + b, position_offset + k,
                        &tok, NULL, NULL);
        sampled_tokens[row] = tok;
      }
      free(out);
      free(e);
    }
  }
  free(w2d);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Admissible interval of one corrected element                        */
/* ------------------------------------------------------------------ */

/* Reading: a device that accumulates the r products in fp32 in any order
 * (exact products, up to r roundings) lands within
 * |acc' - a| <= r * 2^-24 * sum_j |e_j W2w[v,j]|; twice that bound is used.
 * Every step after the dot product (round to fp32, to W, to L, fp32 add,
 * round to L) is monotone, so pushing a -/+ delta through it bounds every
 * admissible result. */
int dspark_oracle_logit_bounds(const void* base_logits, int logits_dtype,
                               const int64_t* token_ids, const void* w1,
                               const void* w2, int weight_dtype, int64_t V,
                               int64_t r, int64_t n, const int64_t* rows,
                               const int64_t* cols, float* lo, float* mid,
                               float* hi) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (V <= 0 || r <= 0 || n < 0) return ORACLE_INVALID;
  if (n == 0) return ORACLE_OK;
  if (!base_logits || !token_ids || !w1 || !w2 || !rows || !cols || !lo || !mid || !hi)
    return ORACLE_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    int64_t row = rows[i], v = cols[i];
    if (row < 0 || v < 0 || v >= V) return ORACLE_INVALID;
    int64_t x = token_ids[row];
    if (x < 0 || x >= V) return ORACLE_INVALID;
    double a = 0.0, s = 0.0;
    for (int64_t j = 0; j < r; ++j) {
      double t = load_as_double(w1, weight_dtype, x * r + j) *
                 load_as_double(w2, weight_dtype, v * r + j);
      a += t;
      s += fabs(t);
    }
    double delta = 2.0 * (double)r * ldexp(1.0, -24) * s;
    float b = load_as_float(base_logits, logits_dtype, row * V + v);
    lo[i] = corrected_value(b, (float)(a - delta), logits_dtype, weight_dtype);
    mid[i] = corrected_value(b, (float)a, logits_dtype, weight_dtype);
    hi[i] = corrected_value(b, (float)(a + delta), logits_dtype, weight_dtype);
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Gated head ([P5] / [P3] GatedMarkovHead)                            */
/* ------------------------------------------------------------------ */

/* Logistic function of a W-typed value, evaluated in double and rounded
 * once to fp32 (torch's sigmoid on a reduced-precision tensor computes in
 * fp32), then to W. */
static float gate_value(float z, int wdt) {
  double s = 1.0 / (1.0 + exp(-(double)z));
  return round_to((float)s, wdt);
}

/* [P5] GatedMarkovHead.compute_gate and compute_step_bias, for one row:
 *   in   = [h.to(W); W1[x].to(W)]            (concatenation, hidden first)
 *   z_j  = gate_proj(in)_j = sum_i in_i Gw[j, i] + gb_j   (Linear(d + r, r))
 *   g_j  = sigmoid(z_j)                       (then .to(e.dtype) = W)
 *   u_j  = g_j * e_j                          (what project_bias receives)
 * Reading: the Linear's fp32 accumulator (bias included) is modelled by
 * its best value, the double sum rounded once to fp32, then rounded to W;
 * the sigmoid as in gate_value; the product in fp32, then rounded to W.
 * When lo/hi are given they receive the admissible interval of u_j: the
 * sum pushed to -/+ 2 (d + r + 1) 2^-24 (sum_i |in_i Gw[j, i]| + |gb_j|)
 * (fp32 accumulation in any order, split or not) and the fp32 sigmoid
 * widened by a relative 2^-20, through the monotone chain. */
static void gated_row(const void* hidden, int hdt, int64_t h_row, int64_t d,
                      const void* w1, int64_t x, const void* gw, const void* gb,
                      int wdt, int64_t r, double* in, float* u, float* lo, float* hi) {
  const int64_t K = d + r;
  for (int64_t i = 0; i < d; ++i)
    in[i] = (double)round_to(load_as_float(hidden, hdt, h_row * d + i), wdt);
  for (int64_t j = 0; j < r; ++j) in[d + j] = load_as_double(w1, wdt, x * r + j);
  for (int64_t j = 0; j < r; ++j) {
    double a = 0.0, s = 0.0;
    for (int64_t i = 0; i < K; ++i) {
      double t = in[i] * load_as_double(gw, wdt, j * K + i);
      a += t;
      s += fabs(t);
    }
    const double bj = load_as_double(gb, wdt, j);
    const float ej = (float)in[d + j];
    const float z = round_to((float)(a + bj), wdt);
    const float g = gate_value(z, wdt);
    u[j] = round_to(g * ej, wdt);
    if (lo && hi) {
      const double delta = 2.0 * (double)(K + 1) * ldexp(1.0, -24) * (s + fabs(bj));
      const float zl = round_to((float)(a + bj - delta), wdt);
      const float zh = round_to((float)(a + bj + delta), wdt);
      const double sl = (1.0 / (1.0 + exp(-(double)zl))) * (1.0 - ldexp(1.0, -20));
      const double sh = (1.0 / (1.0 + exp(-(double)zh))) * (1.0 + ldexp(1.0, -20));
      const float gl = round_to((float)sl, wdt), gh = round_to((float)sh, wdt);
      const float ul = round_to(gl * ej, wdt), uh = round_to(gh * ej, wdt);
      lo[j] = ul < uh ? ul : uh;
      hi[j] = ul < uh ? uh : ul;
    }
  }
}

static int gated_args_ok(int hdt, int wdt, int64_t d, int64_t r) {
  return valid_dtype(hdt) && valid_dtype(wdt) && d > 0 && r > 0;
}

/* Latent rows u[n, :] of the gated head for rows n with hidden state
 * hidden[n, :] ([rows, d]) and predecessor token_ids[n].  Gw is the
 * gate_proj weight [r, d + r], gb its bias [r]; both in the weight dtype.
 * latent [rows, r] in the weight dtype; lo/hi [rows, r] float or NULL. */
int dspark_oracle_gated_latent(const void* hidden, int hidden_dtype, int64_t d,
                               const int64_t* token_ids, const void* w1,
                               const void* gate_w, const void* gate_b,
                               int weight_dtype, int64_t rows, int64_t V,
                               int64_t r, void* latent, float* lo, float* hi,
                               int n_threads) {
  if (!gated_args_ok(hidden_dtype, weight_dtype, d, r)) return ORACLE_INVALID;
  if (rows < 0 || V <= 0) return ORACLE_INVALID;
  if (rows == 0) return ORACLE_OK;
  if (!hidden || !token_ids || !w1 || !gate_w || !gate_b || !latent) return ORACLE_INVALID;
  for (int64_t n = 0; n < rows; ++n)
    if (token_ids[n] < 0 || token_ids[n] >= V) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
#pragma omp parallel num_threads(nt)
  {
    double* in = (double*)malloc((size_t)(d + r) * sizeof(double));
    float* u = (float*)malloc((size_t)r * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < rows; ++n) {
      gated_row(hidden, hidden_dtype, n, d, w1, token_ids[n], gate_w, gate_b, weight_dtype, r,
                in, u, lo ? lo + n * r : NULL, hi ? hi + n * r : NULL);
      for (int64_t j = 0; j < r; ++j) store_from_float(latent, weight_dtype, n * r + j, u[j]);
    }
    free(u);
    free(in);
  }
  return ORACLE_OK;
}

/* [P5] project_bias applied to given latent rows, then the add of
 * apply_block_logits: row n of base [rows, V] is biased by latent[n, :]. */
int dspark_oracle_apply_rows(const void* base_logits, int logits_dtype,
                             const void* latent, const void* w2, int weight_dtype,
                             int64_t rows, int64_t V, int64_t r,
                             void* corrected_logits, int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (rows < 0 || V < 0 || r <= 0) return ORACLE_INVALID;
  if (rows == 0 || V == 0) return ORACLE_OK;
  if (!base_logits || !latent || !w2 || !corrected_logits) return ORACLE_INVALID;
  double* w2d = w2_as_double(w2, weight_dtype, V, r);
  if (!w2d) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
#pragma omp parallel num_threads(nt)
  {
    double* e = (double*)malloc((size_t)r * sizeof(double));
    float* out = (float*)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < rows; ++n) {
      gather_w1_row(latent, weight_dtype, r, n, e);
      corrected_row_from(base_logits, logits_dtype, n, w2d, weight_dtype, V, r, e, out);
      for (int64_t v = 0; v < V; ++v)
        store_from_float(corrected_logits, logits_dtype, n * V + v, out[v]);
    }
    free(out);
    free(e);
  }
  free(w2d);
  return ORACLE_OK;
}

/* dspark_oracle_logit_bounds for elements biased by latent rows:
 * element i is (rows[i], cols[i]) of base [*, V], biased by latent[rows[i]]. */
int dspark_oracle_logit_bounds_rows(const void* base_logits, int logits_dtype,
                                    const void* latent, const void* w2,
                                    int weight_dtype, int64_t V, int64_t r,
                                    int64_t n, const int64_t* rows,
                                    const int64_t* cols, float* lo, float* mid,
                                    float* hi) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (V <= 0 || r <= 0 || n < 0) return ORACLE_INVALID;
  if (n == 0) return ORACLE_OK;
  if (!base_logits || !latent || !w2 || !rows || !cols || !lo || !mid || !hi)
    return ORACLE_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    int64_t row = rows[i], v = cols[i];
    if (row < 0 || v < 0 || v >= V) return ORACLE_INVALID;
    double a = 0.0, s = 0.0;
    for (int64_t j = 0; j < r; ++j) {
      double t = load_as_double(latent, weight_dtype, row * r + j) *
                 load_as_double(w2, weight_dtype, v * r + j);
      a += t;
      s += fabs(t);
    }
    double delta = 2.0 * (double)r * ldexp(1.0, -24) * s;
    float b = load_as_float(base_logits, logits_dtype, row * V + v);
    lo[i] = corrected_value(b, (float)(a - delta), logits_dtype, weight_dtype);
    mid[i] = corrected_value(b, (float)a, logits_dtype, weight_dtype);
    hi[i] = corrected_value(b, (float)(a + delta), logits_dtype, weight_dtype);
  }
  return ORACLE_OK;
}

/* [P5] GatedMarkovHead through VanillaMarkov.apply_block_logits: every row
 * (b, k) is biased by project_bias(gate * W1[token_ids[b, k]]), the gate
 * from hidden_states[b, k, :] ([B, M, d]).  hidden_states NULL is the
 * vanilla fallback of compute_step_bias.  latent_out [B, M, r] (weight
 * dtype, may be NULL) receives what project_bias consumed. */
int dspark_oracle_apply_block_gated(const void* base_logits, int logits_dtype,
                                    const int64_t* token_ids, const void* hidden,
                                    int hidden_dtype, int64_t d, const void* w1,
                                    const void* w2, const void* gate_w,
                                    const void* gate_b, int weight_dtype, int64_t B,
                                    int64_t M, int64_t V, int64_t r,
                                    void* corrected_logits, void* latent_out,
                                    int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (B < 0 || M < 0 || V < 0 || r <= 0) return ORACLE_INVALID;
  int64_t rows = B * M;
  if (rows == 0 || V == 0) return ORACLE_OK;
  if (!base_logits || !token_ids || !w1 || !w2 || !corrected_logits) return ORACLE_INVALID;
  for (int64_t n = 0; n < rows; ++n)
    if (token_ids[n] < 0 || token_ids[n] >= V) return ORACLE_INVALID;
  size_t wb = weight_dtype == ORACLE_F32 ? 4 : 2;
  void* lat = malloc((size_t)(rows * r) * wb);
  if (!lat) return ORACLE_INVALID;
  int st = ORACLE_OK;
  if (hidden) {
    st = dspark_oracle_gated_latent(hidden, hidden_dtype, d, token_ids, w1, gate_w, gate_b,
                                    weight_dtype, rows, V, r, lat, NULL, NULL, n_threads);
  } else {
    for (int64_t n = 0; n < rows; ++n)
      memcpy((char*)lat + (size_t)(n * r) * wb, (const char*)w1 + (size_t)(token_ids[n] * r) * wb,
             (size_t)r * wb);
  }
  if (st == ORACLE_OK)
    st = dspark_oracle_apply_rows(base_logits, logits_dtype, lat, w2, weight_dtype, rows, V, r,
                                  corrected_logits, n_threads);
  if (st == ORACLE_OK && latent_out) memcpy(latent_out, lat, (size_t)(rows * r) * wb);
  free(lat);
  return st;
}

/* [P5] VanillaMarkov.sample_block_tokens with a GatedMarkovHead: step k
 * gates with hidden_states[:, k, :] and the previous token (first_prev at
 * k = 0, the token drawn at k - 1 after that).  hidden NULL is the vanilla
 * fallback.  latent_out [B, M, r] may be NULL. */
int dspark_oracle_sample_block_gated(const void* base_logits, int logits_dtype,
                                     const int64_t* first_prev_token_ids,
                                     const void* hidden, int hidden_dtype, int64_t d,
                                     const void* w1, const void* w2, const void* gate_w,
                                     const void* gate_b, int weight_dtype, int64_t B,
                                     int64_t M, int64_t V, int64_t r, double temperature,
                                     uint64_t seed, int64_t position_offset,
                                     int64_t batch_offset, int64_t* sampled_tokens,
                                     void* corrected_logits, void* latent_out,
                                     int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (B < 0 || M < 0 || V < 0 || r <= 0 || isnan(temperature)) return ORACLE_INVALID;
  if (hidden && !gated_args_ok(hidden_dtype, weight_dtype, d, r)) return ORACLE_INVALID;
  if (B == 0 || M == 0) return ORACLE_OK;
  if (V == 0) return ORACLE_INVALID;
  if (!base_logits || !first_prev_token_ids || !w1 || !w2 || !sampled_tokens)
    return ORACLE_INVALID;
  if (hidden && (!gate_w || !gate_b)) return ORACLE_INVALID;
  for (int64_t b = 0; b < B; ++b)
    if (first_prev_token_ids[b] < 0 || first_prev_token_ids[b] >= V) return ORACLE_INVALID;
  double* w2d = w2_as_double(w2, weight_dtype, V, r);
  if (!w2d) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
  for (int64_t k = 0; k < M; ++k) {
#pragma omp parallel num_threads(nt)
    {
      double* in = (double*)malloc((size_t)((hidden ? d : 0) + r) * sizeof(double));
      double* e = (double*)malloc((size_t)r * sizeof(double));
      float* u = (float*)malloc((size_t)r * sizeof(float));
      float* out = (float*)malloc((size_t)V * sizeof(float));
#pragma omp for schedule(dynamic, 1)
      for (int64_t b = 0; b < B; ++b) {
        int64_t prev = (k == 0) ? first_prev_token_ids[b] : sampled_tokens[b * M + k - 1];
        int64_t row = b * M + k;
        if (hidden) {
          gated_row(hidden, hidden_dtype, row, d, w1, prev, gate_w, gate_b, weight_dtype, r, in,
                    u, NULL, NULL);
          for (int64_t j = 0; j < r; ++j) e[j] = (double)u[j];
        } else {
          gather_w1_row(w1, weight_dtype, r, prev, e);
        }
        if (latent_out)
          for (int64_t j = 0; j < r; ++j) store_from_float(latent_out, weight_dtype, row * r + j, (float)e[j]);
        corrected_row_from(base_logits, logits_dtype, row, w2d, weight_dtype, V, r, e, out);
        if (corrected_logits)
          for (int64_t v = 0; v < V; ++v)
            store_from_float(corrected_logits, logits_dtype, row * V + v, out[v]);
        int64_t tok;
        select_from_row(out, V, temperature, seed, batch_offset + b, position_offset + k,
                        &tok, NULL, NULL);
        sampled_tokens[row] = tok;
      }
      free(out);
      free(u);
      free(e);
      free(in);
    }
  }
  free(w2d);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Backward of the teacher-forced apply ([P5] module docstring: at     */
/* train time the head runs teacher-forced; autograd of                 */
/* apply_block_logits: logits + bias.to(logits.dtype), the Linear and  */
/* the Embedding)                                                       */
/* ------------------------------------------------------------------ */

/* Given G = dloss/dcorrected [rows, V] (logits dtype L):
 *   g[n, v]   = G[n, v] cast to W          (backward of the .to(L) cast)
 *   dW2w[v, j] = sum_n g[n, v] e_n[j]       (Linear weight gradient, W)
 *   de[n, j]  = sum_v g[n, v] W2w[v, j]     (Linear input gradient, W)
 *   dW1[x, j] = sum over rows n with x_n = x of de[n, j]   (Embedding, W)
 * Reading: each sum is modelled by its best fp32 value (double sum rounded
 * once to fp32) and rounded to W; the Embedding gradient adds the W-typed
 * de rows in row order; rows of W1 no id refers to get zero.  The base
 * logits' gradient is G itself and is not computed. */
static float grad_in_w(const void* grad, int ldt, int wdt, int64_t i) {
  return round_to(load_as_float(grad, ldt, i), wdt);
}

int dspark_oracle_apply_block_backward(const void* grad, int logits_dtype,
                                       const int64_t* token_ids, const void* w1,
                                       const void* w2, int weight_dtype, int64_t rows,
                                       int64_t V, int64_t r, void* dw1, void* dw2,
                                       int n_threads) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (rows < 0 || V <= 0 || r <= 0) return ORACLE_INVALID;
  if (!dw1 || !dw2 || (rows > 0 && (!grad || !token_ids || !w1 || !w2))) return ORACLE_INVALID;
  for (int64_t n = 0; n < rows; ++n)
    if (token_ids[n] < 0 || token_ids[n] >= V) return ORACLE_INVALID;
  const int ldt = logits_dtype, wdt = weight_dtype;
  int nt = n_threads_or_default(n_threads);
  /* g in double, [rows, V] */
  double* g = (double*)malloc((size_t)(rows * V + 1) * sizeof(double));
  double* de = (double*)malloc((size_t)(rows * r + 1) * sizeof(double));
  if (!g || !de) {
    free(g);
    free(de);
    return ORACLE_INVALID;
  }
  for (int64_t i = 0; i < rows * V; ++i) g[i] = (double)grad_in_w(grad, ldt, wdt, i);
  /* dW2w */
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t v = 0; v < V; ++v)
    for (int64_t j = 0; j < r; ++j) {
      double a = 0.0;
      for (int64_t n = 0; n < rows; ++n) a += g[n * V + v] * load_as_double(w1, wdt, token_ids[n] * r + j);
      store_from_float(dw2, wdt, v * r + j, round_to((float)a, wdt));
    }
  /* de, rounded to W */
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t n = 0; n < rows; ++n)
    for (int64_t j = 0; j < r; ++j) {
      double a = 0.0;
      for (int64_t v = 0; v < V; ++v) a += g[n * V + v] * load_as_double(w2, wdt, v * r + j);
      de[n * r + j] = (double)round_to((float)a, wdt);
    }
  /* dW1: zero, then the rows of each id summed in row order */
  for (int64_t i = 0; i < V * r; ++i) store_from_float(dw1, wdt, i, 0.0f);
  for (int64_t n = 0; n < rows; ++n) {
    int first = 1;
    for (int64_t m = 0; m < n; ++m)
      if (token_ids[m] == token_ids[n]) first = 0;
    if (!first) continue;
    for (int64_t j = 0; j < r; ++j) {
      double a = 0.0;
      for (int64_t m = n; m < rows; ++m)
        if (token_ids[m] == token_ids[n]) a += de[m * r + j];
      store_from_float(dw1, wdt, token_ids[n] * r + j, round_to((float)a, wdt));
    }
  }
  free(de);
  free(g);
  return ORACLE_OK;
}

/* Admissible intervals of the backward's outputs for a device that sums in
 * fp32 in any order (twice Higham's bound, as for the forward):
 *  dW2 element (v, j): the row sum pushed to -/+ 2 rows 2^-24 sum_n|g e|;
 *  dW1 element (x, j): each contributing de[n, j] pushed to -/+ 2 V 2^-24
 *  sum_v|g w| and rounded to W, the ends summed and widened by
 *  2 cnt 2^-24 sum|de| for the fp32 row sum, then rounded to W.
 * kind 2: elements are (v, j) of dW2; kind 1: (x, j) of dW1.  mid is the
 * oracle's own value. */
int dspark_oracle_backward_bounds(const void* grad, int logits_dtype,
                                  const int64_t* token_ids, const void* w1,
                                  const void* w2, int weight_dtype, int64_t rows,
                                  int64_t V, int64_t r, int kind, int64_t n,
                                  const int64_t* which, const int64_t* cols, float* lo,
                                  float* mid, float* hi) {
  if (!valid_dtype(logits_dtype) || !valid_dtype(weight_dtype)) return ORACLE_UNSUPPORTED;
  if (rows < 0 || V <= 0 || r <= 0 || n < 0 || (kind != 1 && kind != 2)) return ORACLE_INVALID;
  if (n == 0) return ORACLE_OK;
  if (!grad || !token_ids || !w1 || !w2 || !which || !cols || !lo || !mid || !hi) return ORACLE_INVALID;
  for (int64_t m = 0; m < rows; ++m)
    if (token_ids[m] < 0 || token_ids[m] >= V) return ORACLE_INVALID;   /* Embedding lookup would raise */
  const int ldt = logits_dtype, wdt = weight_dtype;
  const double u = ldexp(1.0, -24);
  for (int64_t i = 0; i < n; ++i) {
    const int64_t a0 = which[i], j = cols[i];
    if (j < 0 || j >= r || a0 < 0 || a0 >= V) return ORACLE_INVALID;
    if (kind == 2) {
      double a = 0.0, s = 0.0;
      for (int64_t m = 0; m < rows; ++m) {
        double t = (double)grad_in_w(grad, ldt, wdt, m * V + a0) *
                   load_as_double(w1, wdt, token_ids[m] * r + j);
        a += t;
        s += fabs(t);
      }
      const double d = 2.0 * (double)rows * u * s;
      lo[i] = round_to((float)(a - d), wdt);
      mid[i] = round_to((float)a, wdt);
      hi[i] = round_to((float)(a + d), wdt);
    } else {
      double sl = 0.0, sm = 0.0, sh = 0.0, sa = 0.0;
      int64_t cnt = 0;
      for (int64_t m = 0; m < rows; ++m) {
        if (token_ids[m] != a0) continue;
        double a = 0.0, s = 0.0;
        for (int64_t v = 0; v < V; ++v) {
          double t = (double)grad_in_w(grad, ldt, wdt, m * V + v) * load_as_double(w2, wdt, v * r + j);
          a += t;
          s += fabs(t);
        }
        const double d = 2.0 * (double)V * u * s;
        const double l = round_to((float)(a - d), wdt), h = round_to((float)(a + d), wdt);
        sl += l;
        sh += h;
        sm += round_to((float)a, wdt);
        sa += fabs(l) > fabs(h) ? fabs(l) : fabs(h);
        ++cnt;
      }
      const double d2 = 2.0 * (double)cnt * u * sa;
      lo[i] = round_to((float)(sl - d2), wdt);
      mid[i] = round_to((float)sm, wdt);
      hi[i] = round_to((float)(sh + d2), wdt);
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* LM head fused with the bias ([P1] DeepseekV41DSparkModel.compute_logits */
/* followed by [P5] apply_block_logits)                                */
/* ------------------------------------------------------------------ */

/* [P1] compute_logits projects the hidden states through the frozen
 * vocabulary head in FP32 and returns FP32 logits U [rows, V]; [P5]
 * apply_block_logits then adds bias.to(U.dtype).  Reading: "in FP32" is an
 * fp32 accumulation of the products of the hidden row and the head's
 * weight row ([V, d], the Linear layout) with their values widened exactly;
 * the oracle models it by its best value, the double sum in index order
 * rounded once to fp32.  The bias follows the vanilla reading (fp32
 * accumulator rounded to the weight dtype W, then to fp32), and the
 * corrected logit is the fp32 sum U + bias. */
static float lm_head_value(const void* hidden, int hdt, int64_t n, const void* lm, int lmdt, int64_t v,
                           int64_t d, double* s_abs) {
  double a = 0.0, s = 0.0;
  for (int64_t i = 0; i < d; ++i) {
    const double t = load_as_double(hidden, hdt, n * d + i) * load_as_double(lm, lmdt, v * d + i);
    a += t;
    s += fabs(t);
  }
  if (s_abs) *s_abs = s;
  return (float)a;
}

int dspark_oracle_apply_block_lm_head(const void* hidden, int hidden_dtype, const void* lm_head,
                                      int lm_dtype, int64_t d, const int64_t* token_ids,
                                      const void* w1, const void* w2, int weight_dtype, int64_t rows,
                                      int64_t V, int64_t r, float* corrected, float* base_out,
                                      int n_threads) {
  if (!valid_dtype(hidden_dtype) || !valid_dtype(lm_dtype) || !valid_dtype(weight_dtype))
    return ORACLE_UNSUPPORTED;
  if (rows < 0 || V < 0 || r <= 0 || d <= 0) return ORACLE_INVALID;
  if (rows == 0 || V == 0) return ORACLE_OK;
  if (!hidden || !lm_head || !token_ids || !w1 || !w2 || !corrected) return ORACLE_INVALID;
  for (int64_t n = 0; n < rows; ++n)
    if (token_ids[n] < 0 || token_ids[n] >= V) return ORACLE_INVALID;
  double* w2d = w2_as_double(w2, weight_dtype, V, r);
  if (!w2d) return ORACLE_INVALID;
  int nt = n_threads_or_default(n_threads);
#pragma omp parallel num_threads(nt)
  {
    double* e = (double*)malloc((size_t)r * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < rows; ++n) {
      gather_w1_row(w1, weight_dtype, r, token_ids[n], e);
      for (int64_t v = 0; v < V; ++v) {
        const float u = lm_head_value(hidden, hidden_dtype, n, lm_head, lm_dtype, v, d, NULL);
        const float acc = projected_bias(e, w2d + v * r, r);
        corrected[n * V + v] = corrected_value(u, acc, ORACLE_F32, weight_dtype);
        if (base_out) base_out[n * V + v] = u;
      }
    }
    free(e);
  }
  free(w2d);
  return ORACLE_OK;
}

/* Admissible interval of fused elements (rows[i], cols[i]) for a device that
 * accumulates both products in fp32 in any order: U pushed to
 * -/+ 2 d 2^-24 sum|h w| and the bias accumulator to -/+ 2 r 2^-24 sum|e w2|
 * (twice Higham's bound each), through the monotone chain (round to fp32,
 * bias rounded to W then fp32, fp32 add). */
int dspark_oracle_lm_head_bounds(const void* hidden, int hidden_dtype, const void* lm_head, int lm_dtype,
                                 int64_t d, const int64_t* token_ids, const void* w1, const void* w2,
                                 int weight_dtype, int64_t V, int64_t r, int64_t n, const int64_t* rows,
                                 const int64_t* cols, float* lo, float* mid, float* hi) {
  if (!valid_dtype(hidden_dtype) || !valid_dtype(lm_dtype) || !valid_dtype(weight_dtype))
    return ORACLE_UNSUPPORTED;
  if (V <= 0 || r <= 0 || d <= 0 || n < 0) return ORACLE_INVALID;
  if (n == 0) return ORACLE_OK;
  if (!hidden || !lm_head || !token_ids || !w1 || !w2 || !rows || !cols || !lo || !mid || !hi)
    return ORACLE_INVALID;
  const double u24 = ldexp(1.0, -24);
  for (int64_t i = 0; i < n; ++i) {
    if (rows[i] < 0 || cols[i] < 0 || cols[i] >= V) return ORACLE_INVALID;
    if (token_ids[rows[i]] < 0 || token_ids[rows[i]] >= V) return ORACLE_INVALID;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t row = rows[i], v = cols[i];
    const int64_t x = token_ids[row];
    double a = 0.0, s = 0.0, ub = 0.0, su = 0.0;
    for (int64_t j = 0; j < r; ++j) {
      const double t = load_as_double(w1, weight_dtype, x * r + j) * load_as_double(w2, weight_dtype, v * r + j);
      a += t;
      s += fabs(t);
    }
    for (int64_t k = 0; k < d; ++k) {
      const double t = load_as_double(hidden, hidden_dtype, row * d + k) * load_as_double(lm_head, lm_dtype, v * d + k);
      ub += t;
      su += fabs(t);
    }
    const double db = 2.0 * (double)r * u24 * s, du = 2.0 * (double)d * u24 * su;
    lo[i] = corrected_value((float)(ub - du), (float)(a - db), ORACLE_F32, weight_dtype);
    mid[i] = corrected_value((float)ub, (float)a, ORACLE_F32, weight_dtype);
    hi[i] = corrected_value((float)(ub + du), (float)(a + db), ORACLE_F32, weight_dtype);
  }
  return ORACLE_OK;
}
