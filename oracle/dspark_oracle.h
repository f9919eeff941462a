/*
 * dspark_oracle.h -- plain, slow CPU oracle for the vanilla DSpark low-rank
 * Markov head.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product path never does.
 * It shares no code, header, table or constant generator with the GPU library.
 *
 * Sources (web pages on the DSpark Markov head):
 *   [P5] raw markov_head.py of a third-party DSpark draft repository:
 *        module docstring (transition formula B(x_{k-1},:) = W2(W1[x_{k-1}]),
 *        corrected logit U_k + B), _sample_tokens, VanillaMarkov
 *        (get_prev_embeddings, project_bias, compute_step_bias,
 *        apply_step_logits, apply_block_logits, sample_block_tokens),
 *        build_markov_head.
 *   [P3] NeMo AutoModel API page "speculative/dspark/markov_head",
 *        class VanillaMarkov (markov_w1 = nn.Embedding(V, r)).
 *   [P1] NeMo AutoModel API page "models/deepseek_v41/dspark",
 *        class _DeepseekV41DSparkMarkovHead.
 *   Gated head: [P5] GatedMarkovHead (compute_gate, compute_step_bias) and
 *        the [P3] API page's GatedMarkovHead (gate_proj = Linear(d + r, r)).
 *   Backward: [P5] module docstring (train time is teacher-forced), taken
 *        through autograd of apply_block_logits.
 *
 * Numeric reading (every step is written out in dspark_oracle.c):
 *   e      = W1[x, :]                                (exact, widened to double)
 *   a_v    = sum_j e_j * W2w[v, j]   in double, j in index order
 *   acc_v  = (float) a_v                              (one round to nearest even)
 *   bias_v = rnd_L(rnd_W(acc_v))                      (Linear emits W, .to(L))
 *   c_v    = rnd_L((float)base_v + (float)bias_v)     (fp32 add, one rounding)
 *   greedy (T < 1e-5): smallest v with c_v == max c
 *   else   : smallest v maximising fmaf(c_v, kappa_T, g_v),
 *            kappa_T = (float)(log2(e) / T), g_v = -log2f(-log2f(u_v)),
 *            u_v from Philox4x32-10 (Salmon et al., SC'11).
 *
 * Layouts: base/corrected [B, M, V] row-major; token_ids [B, M];
 * W1 [V, r] (the Embedding weight) and W2w [V, r] (the Linear(r, V) weight,
 * i.e. the transpose of the mathematical W2) both row-major.
 * dtype tags: 0 = float32, 1 = bfloat16 (stored as uint16 bit patterns).
 * Return codes: 0 ok, 1 invalid argument, 2 unsupported dtype pair.
 */
#ifndef DSPARK_ORACLE_H
#define DSPARK_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_OK 0
#define ORACLE_INVALID 1
#define ORACLE_UNSUPPORTED 2

/* Teacher-forced block bias (VanillaMarkov.apply_block_logits). */
int dspark_oracle_apply_block(const void* base_logits, int logits_dtype,
                              const int64_t* token_ids, const void* w1,
                              const void* w2, int weight_dtype, int64_t B,
                              int64_t M, int64_t V, int64_t r,
                              void* corrected_logits, int n_threads);

/* Left-to-right block sampling (VanillaMarkov.sample_block_tokens).
 * Noise for batch row b, step k uses the absolute indices
 * (batch_offset + b, position_offset + k).  corrected_logits may be NULL. */
int dspark_oracle_sample_block(const void* base_logits, int logits_dtype,
                               const int64_t* first_prev_token_ids,
                               const void* w1, const void* w2, int weight_dtype,
                               int64_t B, int64_t M, int64_t V, int64_t r,
                               double temperature, uint64_t seed,
                               int64_t position_offset, int64_t batch_offset,
                               int64_t* sampled_tokens, void* corrected_logits,
                               int n_threads);

/* The reduction step of _sample_tokens alone, applied to one corrected row
 * (dtype logits_dtype, length V) that the caller supplies.  Writes the token
 * and, if score_out is not NULL, the winning and runner-up scores (the
 * corrected values for greedy, the Gumbel scores otherwise) and the
 * runner-up index. */
int dspark_oracle_select_token(const void* row, int logits_dtype, int64_t V,
                               double temperature, uint64_t seed, int64_t b_abs,
                               int64_t k_abs, int64_t* token, float* score_out,
                               int64_t* runner_up);

/* dspark_oracle_select_token over n rows [n, V] (rows in parallel, n_threads
 * 0 = all cores); row i uses noise indices (b_abs[i], k_abs[i]).  scores
 * [n, 2] and runner_up [n] may be NULL. */
int dspark_oracle_select_tokens(const void* rows, int logits_dtype, int64_t n, int64_t V,
                                double temperature, uint64_t seed, const int64_t* b_abs,
                                const int64_t* k_abs, int64_t* tokens, float* scores,
                                int64_t* runner_up, int n_threads);

/* Bounds on one corrected element under any fp32 accumulation order:
 * for each of n (row, v) pairs, with row indexing the flattened [B*M] rows,
 * writes lo/hi (as float values of the L-typed results) obtained by pushing
 * the dot product to a -/+ 2r*2^-24*sum|e_j*W2w[v,j]| through the monotone
 * rounding chain.  Also writes the oracle's own value to mid. */
int dspark_oracle_logit_bounds(const void* base_logits, int logits_dtype,
                               const int64_t* token_ids, const void* w1,
                               const void* w2, int weight_dtype, int64_t V,
                               int64_t r, int64_t n, const int64_t* rows,
                               const int64_t* cols, float* lo, float* mid,
                               float* hi);

/* Gated head ([P5]/[P3] GatedMarkovHead): hidden [rows, d] (or [B, M, d]),
 * gate_w = gate_proj.weight [r, d + r], gate_b = gate_proj.bias [r], both
 * in the weight dtype.  The latent row u = sigmoid(gate_proj([h; e])) * e,
 * e = W1[x], is what project_bias consumes.  lo/hi (may be NULL) receive
 * each latent element's admissible interval for a device that accumulates
 * in fp32 in any order. */
int dspark_oracle_gated_latent(const void* hidden, int hidden_dtype, int64_t d,
                               const int64_t* token_ids, const void* w1,
                               const void* gate_w, const void* gate_b,
                               int weight_dtype, int64_t rows, int64_t V,
                               int64_t r, void* latent, float* lo, float* hi,
                               int n_threads);

/* Row n of base [rows, V] biased by project_bias(latent[n, :]). */
int dspark_oracle_apply_rows(const void* base_logits, int logits_dtype,
                             const void* latent, const void* w2, int weight_dtype,
                             int64_t rows, int64_t V, int64_t r,
                             void* corrected_logits, int n_threads);

/* dspark_oracle_logit_bounds with row rows[i] biased by latent[rows[i]]. */
int dspark_oracle_logit_bounds_rows(const void* base_logits, int logits_dtype,
                                    const void* latent, const void* w2,
                                    int weight_dtype, int64_t V, int64_t r,
                                    int64_t n, const int64_t* rows,
                                    const int64_t* cols, float* lo, float* mid,
                                    float* hi);

/* apply_block_logits / sample_block_tokens of a GatedMarkovHead; hidden
 * NULL is the vanilla fallback.  latent_out [B, M, r] may be NULL. */
int dspark_oracle_apply_block_gated(const void* base_logits, int logits_dtype,
                                    const int64_t* token_ids, const void* hidden,
                                    int hidden_dtype, int64_t d, const void* w1,
                                    const void* w2, const void* gate_w,
                                    const void* gate_b, int weight_dtype, int64_t B,
                                    int64_t M, int64_t V, int64_t r,
                                    void* corrected_logits, void* latent_out,
                                    int n_threads);
int dspark_oracle_sample_block_gated(const void* base_logits, int logits_dtype,
                                     const int64_t* first_prev_token_ids,
                                     const void* hidden, int hidden_dtype, int64_t d,
                                     const void* w1, const void* w2, const void* gate_w,
                                     const void* gate_b, int weight_dtype, int64_t B,
                                     int64_t M, int64_t V, int64_t r, double temperature,
                                     uint64_t seed, int64_t position_offset,
                                     int64_t batch_offset, int64_t* sampled_tokens,
                                     void* corrected_logits, void* latent_out,
                                     int n_threads);

/* Backward of the teacher-forced apply (training): given the gradient of
 * the loss w.r.t. the corrected logits, grad [rows, V] (logits dtype), the
 * gradients of W1 (dense [V, r], zero where no id refers) and of W2w
 * ([V, r]), both in the weight dtype.  The base logits' gradient is grad. */
int dspark_oracle_apply_block_backward(const void* grad, int logits_dtype,
                                       const int64_t* token_ids, const void* w1,
                                       const void* w2, int weight_dtype, int64_t rows,
                                       int64_t V, int64_t r, void* dw1, void* dw2,
                                       int n_threads);
/* Admissible intervals of chosen backward outputs: kind 2 = dW2w elements
 * (which[i] = v), kind 1 = dW1 elements (which[i] = token x); cols[i] = j. */
int dspark_oracle_backward_bounds(const void* grad, int logits_dtype,
                                  const int64_t* token_ids, const void* w1,
                                  const void* w2, int weight_dtype, int64_t rows,
                                  int64_t V, int64_t r, int kind, int64_t n,
                                  const int64_t* which, const int64_t* cols, float* lo,
                                  float* mid, float* hi);

/* LM head fused with the bias: U = the FP32 projection of hidden [rows, d]
 * through the vocabulary head lm_head [V, d] ([P1] compute_logits), then
 * corrected = U + bias.to(fp32) with bias = project_bias(W1[token_ids[n]])
 * ([P5] apply_block_logits).  corrected [rows, V] fp32; base_out [rows, V]
 * fp32 receives U when not NULL. */
int dspark_oracle_apply_block_lm_head(const void* hidden, int hidden_dtype, const void* lm_head,
                                      int lm_dtype, int64_t d, const int64_t* token_ids,
                                      const void* w1, const void* w2, int weight_dtype, int64_t rows,
                                      int64_t V, int64_t r, float* corrected, float* base_out,
                                      int n_threads);
/* Admissible interval of fused elements (rows[i], cols[i]) under any fp32
 * accumulation order of both products; mid is the oracle's value. */
int dspark_oracle_lm_head_bounds(const void* hidden, int hidden_dtype, const void* lm_head, int lm_dtype,
                                 int64_t d, const int64_t* token_ids, const void* w1, const void* w2,
                                 int weight_dtype, int64_t V, int64_t r, int64_t n, const int64_t* rows,
                                 const int64_t* cols, float* lo, float* mid, float* hi);

/* Building blocks exposed for pinning. */
void dspark_oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                                 uint32_t out[4]);
float dspark_oracle_gumbel2(uint64_t seed, int64_t b_abs, int64_t k_abs,
                            int64_t v);
uint16_t dspark_oracle_round_bf16(float x);
float dspark_oracle_kappa(double temperature);

#ifdef __cplusplus
}
#endif

#endif
