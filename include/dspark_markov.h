/*
 * dspark_markov.h -- C ABI of the MI355X (gfx950) DSpark low-rank Markov head.
 *
 * The vanilla DSpark Markov head adds a first-order token-transition bias to
 * a block drafter's base logits:
 *
 *     B(x_{k-1}, :) = W2 . W1[x_{k-1}],   W1 in R^{V x r},  W2 in R^{r x V}
 *     corrected_k   = U_k + B(x_{k-1}, :)
 *
 * (third-party markov_head.py page, module docstring; NeMo AutoModel
 * "speculative/dspark/markov_head" page, class VanillaMarkov; NeMo AutoModel
 * "models/deepseek_v41/dspark" page, class _DeepseekV41DSparkMarkovHead).
 *
 * Two operations mirror VanillaMarkov's two methods (each also has a gated
 * form for GatedMarkovHead, declared further down):
 *   dspark_markov_apply_block   -- apply_block_logits (teacher-forced: every
 *                                  row biased by its own given predecessor);
 *   dspark_markov_sample_block  -- sample_block_tokens (left to right: each
 *                                  position biased by the token drawn at the
 *                                  previous position, greedy or temperature).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every pointer argument named as device memory must point to
 *           memory of the current HIP device; the caller owns all buffers.
 *           The library never allocates memory visible to the caller.
 * Streams.  `stream` is a hipStream_t (NULL = the null stream).  All work is
 *           enqueued asynchronously on it; no entry point synchronises except
 *           dspark_markov_read_device_error.
 * Layout.   Contiguous row-major.  base/corrected logits are [B, M, V]; the
 *           training layout [B, num_anchors, block_size, V] is passed as
 *           B' = B * num_anchors, M = block_size (the op is row-wise, so the
 *           result is identical).  W1 is the Embedding weight [V, r]; W2 is
 *           passed as the Linear(r, V) weight [V, r], i.e. the transpose of
 *           the mathematical W2.
 * Dtypes.   (logits, weights) may be any pair of F32 and BF16; the
 *           roundings below follow each tensor's own dtype (the pages'
 *           bias.to(logits.dtype) defines the mixed case).  Token ids are
 *           int64.
 * Numerics. bias = round_L(round_W(fp32 dot product of W1[x] and W2w[v]));
 *           corrected = round_L(fp32(base) + fp32(bias))  (Linear output in
 *           the weight dtype, then .to(logits dtype), then the add).
 * Errors.   Argument errors are detected on the host before anything is
 *           enqueued and leave every output untouched.  Token ids outside
 *           [0, V) are not checked on the host: such a row gets a zero bias
 *           and is counted in the workspace's device error word (see
 *           dspark_markov_read_device_error).
 * Workspace. Device memory of at least dspark_markov_workspace_bytes(...)
 *           bytes, zero-filled once before its first use (for instance by
 *           dspark_markov_workspace_init); the library leaves it ready for
 *           the next call, of any shape and operation that fits it (every
 *           call uses one layout).  Calls that share one workspace must be
 *           ordered on one stream; calls in flight at the same time need
 *           their own.
 */
#ifndef DSPARK_MARKOV_H
#define DSPARK_MARKOV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below have int as their underlying type, so every int a
 * C caller passes is a valid value for the library to inspect (and reject
 * when it names no dtype or status); C sees plain enums of int size. */
#ifdef __cplusplus
#define DSPARK_ENUM_BASE : int
#else
#define DSPARK_ENUM_BASE
#endif

typedef enum DSPARK_ENUM_BASE { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype_t;

typedef enum DSPARK_ENUM_BASE {
  DSPARK_OK = 0,
  DSPARK_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, r <= 0, NaN temperature, overlap */
  DSPARK_ERR_UNSUPPORTED = 2,        /* dtype pair or shape the library has no kernel for */
  DSPARK_ERR_WORKSPACE_TOO_SMALL = 3,
  DSPARK_ERR_DEVICE = 4              /* a HIP runtime call failed (see dspark_markov_last_error) */
} dspark_status_t;

/* Bytes of workspace an apply (sample_mode = 0) or sample (sample_mode = 1)
 * call of these sizes needs.  Pure host function.  This and the gated and
 * backward size queries return SIZE_MAX when the sizes cannot be
 * represented (no buffer can then satisfy the call). */
size_t dspark_markov_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r, int sample_mode);

/* Zero-fill `bytes` bytes of workspace on `stream` with a device kernel. */
dspark_status_t dspark_markov_workspace_init(void* workspace, size_t bytes, void* stream);

/* Teacher-forced block bias (VanillaMarkov.apply_block_logits, third-party
 * markov_head.py page).
 *   base_logits      device, [B, M, V], logits_dtype.
 *   token_ids        device, [B, M] int64: the predecessor x_{k-1} of each row.
 *   w1, w2           device, [V, r] each, weight_dtype.
 *   corrected_logits device, [B, M, V], logits_dtype; may equal base_logits
 *                    (in place); any other overlap with an input is invalid.
 * B, M, V >= 0; r > 0 (the page's constructor asserts a positive rank);
 * ranks above 16384 return DSPARK_ERR_UNSUPPORTED.
 * B*M*V == 0 is a successful no-op (the page returns base_logits itself). */
dspark_status_t dspark_markov_apply_block(const void* base_logits, dspark_dtype_t logits_dtype,
                                          const int64_t* token_ids, const void* w1,
                                          const void* w2, dspark_dtype_t weight_dtype,
                                          int64_t B, int64_t M, int64_t V, int64_t r,
                                          void* corrected_logits, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Left-to-right block sampling (VanillaMarkov.sample_block_tokens and
 * _sample_tokens, third-party markov_head.py page).
 *   base_logits          device, [B, M, V].
 *   first_prev_token_ids device, [B] int64: the verified token before position 0.
 *   sampled_tokens       device, [B, M] int64 output.
 *   corrected_logits     device, [B, M, V] output, or NULL for tokens only.
 *   temperature          greedy argmax (first index on ties) when < 1e-5,
 *                        negative values included; NaN is invalid.  Otherwise
 *                        one draw from softmax(corrected / T) per position by
 *                        Gumbel-max: the first v maximising
 *                        fmaf(c_v, (float)(log2(e)/T), -log2(-log2(u_v))),
 *                        u_v = (2*(w >> 9) + 1) * 2^-24 with w the word (v & 3)
 *                        of Philox4x32-10 (Salmon et al., SC'11) at counter
 *                        (v >> 2, position_offset + k, batch_offset + b, 0)
 *                        and key (seed & 0xffffffff, seed >> 32).
 *   position_offset,     absolute step and batch indices of position 0 / row 0
 *   batch_offset         for the noise, so that M one-step calls, or a batch
 *                        split across calls, reproduce one whole call.
 * M == 0 or B == 0 is a successful no-op.  V == 0 with B*M > 0 is invalid;
 * ranks above 16384 return DSPARK_ERR_UNSUPPORTED.
 *
 * Calls with bf16 weights (bf16 or fp32 logits) and r <= 256 run as one
 * persistent launch when they fit one of two chains: greedy calls with
 * B <= 64, M <= 16 and V <= 512 * CUs; then any call (temperature, or a
 * greedy call the first did not take) with B <= 256, M * B <= 4096 and
 * V <= 640 * CUs (bf16 logits) or V <= 608 * CUs (fp32 logits).  Their
 * workgroups (one per CU) exchange each step's tokens through the
 * workspace; the host takes that path only when the occupancy query says a
 * CU can hold one of its workgroups (other calls run one step kernel per
 * position).  The tokens are the same on both paths.  Should a workgroup
 * still be unable to start (CUs held by other streams' kernels), the
 * others give up waiting
 * after 1 s instead of hanging: the call then writes -1 to every token of
 * sampled_tokens (corrected_logits is then undefined) and records the
 * failure in the workspace.  Until dspark_markov_read_device_error reads
 * and clears that record, every later persistent launch on the same
 * workspace does no work and also returns -1 tokens, so a failure cannot
 * pass unnoticed.  The word at byte 128 of the workspace is a test hook:
 * nonzero makes every such wait give up at once (the failure path without a
 * stall); zero-filled workspaces leave it off. */
dspark_status_t dspark_markov_sample_block(const void* base_logits, dspark_dtype_t logits_dtype,
                                           const int64_t* first_prev_token_ids, const void* w1,
                                           const void* w2, dspark_dtype_t weight_dtype,
                                           int64_t B, int64_t M, int64_t V, int64_t r,
                                           double temperature, uint64_t seed,
                                           int64_t position_offset, int64_t batch_offset,
                                           int64_t* sampled_tokens, void* corrected_logits,
                                           void* workspace, size_t workspace_bytes, void* stream);

/* dspark_markov_sample_block for callers that cannot allocate: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and kernels, minus the workspace: the library
 * uses a static scratch array of 4 MiB per GPU (4,194,304 bytes, held until
 * the process ends) in place of the caller's workspace.  Sizes whose
 * dspark_markov_workspace_bytes(B, M, V, r, 1) exceeds that are rejected
 * with DSPARK_ERR_WORKSPACE_TOO_SMALL before anything is enqueued (the
 * message names both sizes); for instance B = 64, M = 5 at V = 129280 needs
 * 1.1 MB and B = 256, M = 8 at V = 151936 needs 3.0 MB.  Nothing is
 * allocated: the first call on a device zero-fills its scratch with a
 * kernel on `stream`, and every call clears the scratch's error words
 * first, so out-of-range ids are not counted and a failed persistent chain
 * shows only as -1 tokens.  Every call on a GPU shares that GPU's scratch,
 * which keeps the last call's contents: calls that overlap on one GPU (on
 * different streams or host threads) race and must be ordered by the
 * caller. */
dspark_status_t dspark_markov_sample_block_static(const void* base_logits, dspark_dtype_t logits_dtype,
                                                  const int64_t* first_prev_token_ids, const void* w1,
                                                  const void* w2, dspark_dtype_t weight_dtype, int64_t B,
                                                  int64_t M, int64_t V, int64_t r, double temperature,
                                                  uint64_t seed, int64_t position_offset, int64_t batch_offset,
                                                  int64_t* sampled_tokens, void* corrected_logits, void* stream);

/* Gated head (GatedMarkovHead, on the third-party markov_head.py page and
 * the NeMo AutoModel "speculative/dspark/markov_head" page).  The bias of a
 * row is W2 . u with the latent row
 *     u = sigmoid(gate_proj([h; W1[x]])) * W1[x],
 * gate_proj = Linear(d + r, r) with a bias; h is the row's backbone hidden
 * state [d] and both concatenated operands are cast to the weight dtype
 * (compute_gate).  Rounding (weight dtype W): the gate's fp32 accumulator
 * plus bias rounded to W, the fp32 logistic of that rounded to W, the fp32
 * product with W1[x] rounded to W; then the vanilla numerics with u in place
 * of W1[x].  hidden_states NULL is the pages' vanilla fallback (u = W1[x]);
 * gate_weight and gate_bias are then ignored and may be NULL.
 *   hidden_states  device, [B, M, d], hidden_dtype (F32 or BF16): row (b, k)
 *                  gates position k of row b.
 *   gate_weight    device, [r, d + r] (the Linear weight), weight_dtype.
 *   gate_bias      device, [r], weight_dtype.
 *   latent_out     device, [B, M, r], weight_dtype, or NULL: receives u
 *                  (the vector project_bias consumed) for every row; for
 *                  the vanilla fallback that is the embedding W1[x] the
 *                  DeepSeek-V4.1 head returns beside its logits.
 * Token ids outside [0, V) give u = 0 (a zero bias) and are counted as in
 * the vanilla calls.  Other arguments as in dspark_markov_apply_block and
 * dspark_markov_sample_block; d > 0 when hidden_states is given.  The
 * workspace must hold dspark_markov_gated_workspace_bytes(...) bytes; the
 * gated calls need it zero-filled once, like the vanilla ones. */
size_t dspark_markov_gated_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r, int64_t d,
                                           int sample_mode);

dspark_status_t dspark_markov_apply_block_gated(
    const void* base_logits, dspark_dtype_t logits_dtype, const int64_t* token_ids,
    const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d, const void* w1,
    const void* w2, const void* gate_weight, const void* gate_bias, dspark_dtype_t weight_dtype,
    int64_t B, int64_t M, int64_t V, int64_t r, void* corrected_logits, void* latent_out,
    void* workspace, size_t workspace_bytes, void* stream);

/* Left-to-right sampling with the gated head: step k gates with
 * hidden_states[:, k, :] and the previous token (sample_block_tokens hands
 * each step its position's hidden state).  Noise and outputs as in
 * dspark_markov_sample_block; latent_out [B, M, r] or NULL. */
dspark_status_t dspark_markov_sample_block_gated(
    const void* base_logits, dspark_dtype_t logits_dtype, const int64_t* first_prev_token_ids,
    const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d, const void* w1,
    const void* w2, const void* gate_weight, const void* gate_bias, dspark_dtype_t weight_dtype,
    int64_t B, int64_t M, int64_t V, int64_t r, double temperature, uint64_t seed,
    int64_t position_offset, int64_t batch_offset, int64_t* sampled_tokens,
    void* corrected_logits, void* latent_out, void* workspace, size_t workspace_bytes,
    void* stream);

/* Backward of the teacher-forced apply (training; the third-party
 * markov_head.py page trains the head teacher-forced, through
 * apply_block_logits).  Given the gradient of the loss w.r.t. the corrected
 * logits, grad_corrected (device, [B, M, V], logits_dtype), writes
 *   grad_w2 [V, r] (the Linear weight's gradient):  sum_n g[n, v] W1[x_n],
 *   grad_w1 [V, r] (the Embedding's gradient, dense): for each id x the sum
 *           over its rows n of de[n] = sum_v g[n, v] W2w[v], zero for ids
 *           no row refers to,
 * both in weight_dtype, with g = grad_corrected cast to the weight dtype,
 * each product summed in fp32 and rounded once to the weight dtype (de
 * too, before the rows of one id are added in row order).  The base
 * logits' gradient is grad_corrected itself.  Rows whose id is outside
 * [0, V) contribute nothing and are counted in the device error word.
 * B*M == 0 writes zero gradients.  The workspace must hold
 * dspark_markov_backward_workspace_bytes(...) bytes (no zero fill
 * needed beyond the vanilla rule for the error word).  Outputs must not
 * overlap inputs or each other. */
size_t dspark_markov_backward_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r);

dspark_status_t dspark_markov_apply_block_backward(const void* grad_corrected, dspark_dtype_t logits_dtype,
                                                   const int64_t* token_ids, const void* w1, const void* w2,
                                                   dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V,
                                                   int64_t r, void* grad_w1, void* grad_w2, void* workspace,
                                                   size_t workspace_bytes, void* stream);

/* The drafter's vocabulary head fused with the teacher-forced bias: the
 * base logits U = hidden . lm_head^T are computed in FP32 (NeMo AutoModel
 * "models/deepseek_v41/dspark" page, DeepseekV41DSparkModel.compute_logits:
 * the hidden states projected through the frozen vocabulary head in FP32,
 * FP32 logits out) and the Markov bias is added as in apply_block_logits
 * (third-party markov_head.py page: U + bias.to(U.dtype)), without U ever
 * being written:
 *     corrected[n, v] = fp32( U[n, v] + fp32(round_W(sum_j W1[x_n, j] W2w[v, j])) ),
 * U[n, v] = the fp32 accumulation of hidden[n, i] * lm_head[v, i] (exact
 * products of the widened operands).
 *   hidden_states    device, [B, M, d] (row (b, k) is the drafter's hidden
 *                    state of block position k), hidden_dtype.
 *   lm_head_weight   device, [V, d] (the head's Linear weight), lm_head_dtype.
 *   token_ids        device, [B, M] int64 teacher-forced predecessors.
 *   w1, w2           device, [V, r] each, weight_dtype.
 *   corrected_logits device, [B, M, V] float32 output; must not overlap an input.
 * The kernel takes bf16 hidden states, head and Markov weights with d, r
 * and V multiples of 8, 16-byte aligned buffers, and each buffer within
 * 2^31 bytes; other calls return DSPARK_ERR_UNSUPPORTED (the message names
 * the rule).  B*M*V == 0 is a successful no-op; out-of-range ids give a zero
 * bias and are counted as in dspark_markov_apply_block.  The workspace is
 * that of dspark_markov_apply_block (only its error word is used). */
dspark_status_t dspark_markov_apply_block_lm_head(const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d,
                                                  const void* lm_head_weight, dspark_dtype_t lm_head_dtype,
                                                  const int64_t* token_ids, const void* w1, const void* w2,
                                                  dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V,
                                                  int64_t r, float* corrected_logits, void* workspace,
                                                  size_t workspace_bytes, void* stream);

/* Synchronises `stream`, then returns in *bad_rows the number of rows whose
 * predecessor id was outside [0, V) in the calls made with this workspace
 * since the last read, and clears the count.  Returns DSPARK_ERR_DEVICE when
 * a persistent sampling launch on this workspace failed since the last read
 * (its tokens were -1, see dspark_markov_sample_block); the failure record
 * is cleared too, so the next call runs normally. */
dspark_status_t dspark_markov_read_device_error(void* workspace, void* stream, int64_t* bad_rows);

/* Static description of a status code. */
const char* dspark_status_string(dspark_status_t status);

/* Message of the last HIP runtime failure seen by this thread ("" if none). */
const char* dspark_markov_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_MARKOV_H */
