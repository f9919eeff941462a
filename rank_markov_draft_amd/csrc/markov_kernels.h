// markov_kernels.h -- interface between the C ABI (dspark_markov.hip) and the
// gfx950 kernels (markov_kernels.hip, markov_apply.hip, markov_step.hip,
// markov_gate.hip; the chain's own interface is markov_chain.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "markov_chain.h"

namespace dspark {

enum { MODE_APPLY = 0, MODE_GREEDY = 1, MODE_TEMPERATURE = 2 };

// Arguments of one launch.  Apply launches process `rows` = B*M rows whose
// predecessors are ids[n]; sampling-step launches process the B rows of step
// k, whose predecessor is ids[b] (first_prev) at k = 0 and tokens[b, k-1]
// after that.
struct KernelParams {
  const void* base;      // [B, M, V] logits
  void* out;             // [B, M, V] corrected logits, or null (tokens only)
  const int64_t* ids;    // apply: token_ids [B*M]; sampling: first_prev [B]
  int64_t* tokens;       // sampling: [B, M]
  const void* w1;        // [V, r]
  const void* w2;        // [V, r]
  uint64_t* partials;    // sampling: [rows, nparts] argmax keys
  uint32_t* bad_rows;    // device error word
  void* sink;            // apply: 16 bytes per thread of scratch for stores past the edges
  // Gated head: when latent is set, row n (apply) or batch row b (sampling
  // step) is biased by the projection of latent row n (b) -- [rows] rows of
  // latent_ld elements in the weight dtype -- instead of W1[predecessor];
  // the predecessor still decides whether the row is valid.
  const void* latent;
  int64_t latent_ld;
  int64_t rows;
  int64_t V;
  int64_t r;
  int64_t M;
  int64_t k;             // sampling step
  int64_t nparts;        // sampling: vocabulary slices per row
  int64_t batch_offset;  // absolute batch index of row 0 (noise counter)
  int mode;
  float kappa;           // (float)(log2(e) / T)
  uint32_t k_abs;        // absolute position index of step k (noise counter)
  uint32_t seed_lo;
  uint32_t seed_hi;
};



// The vocabulary head fused with the bias (bf16 operands, fp32 output):
// out[n, v] = fp32(hidden[n] . lm[v] + fp32(rnd_bf16(W1[ids[n]] . W2w[v]))).
struct LmHeadParams {
  const void* hidden;  // [rows, d] bf16
  const void* lm;      // [V, d] bf16 (the head's Linear weight)
  const int64_t* ids;  // [rows] predecessors
  const void* w1;      // [V, r] bf16
  const void* w2;      // [V, r] bf16
  float* out;          // [rows, V] fp32
  uint32_t* bad_rows;  // device error word
  int64_t rows;
  int64_t V;
  int64_t r;
  int64_t d;
};
hipError_t launch_lm_head(const LmHeadParams& p, int num_cus, hipStream_t s);

// The gate of the gated head, one launch per call (apply) or per step
// (sampling): the latent rows u = rnd_W(rnd_W(sigmoid(rnd_W(z + b))) * e),
// z = gate_proj's product with [h; e], e = W1[predecessor] (zero for
// invalid ids); without hidden states (gated == 0) u = e.
struct GateParams {
  const void* hidden;      // rows of d elements: apply row n, step (b, k) at b * M + k
  const int64_t* ids;      // apply: token_ids [rows]; sampling: first_prev [B]
  const int64_t* tokens;   // sampling: [B, M]
  const void* w1;          // [V, r]
  const void* gw;          // gate_proj weight [r, d + r]
  const void* gb;          // gate_proj bias [r]
  void* latent;            // [rows] rows of latent_ld elements
  float* partials;         // [S][rows][r] split sums (workspace), when S > 1
  int64_t rows;
  int64_t V;
  int64_t r;
  int64_t d;
  int64_t M;
  int64_t k;               // sampling step
  int64_t latent_ld;
  int64_t hidden_bytes;    // extent of the hidden tensor
  int64_t kchunk;          // inner columns of one split (set by launch_gate)
  int S;                   // splits (set by launch_gate)
  int mode;                // MODE_APPLY or a sampling mode
  int gated;               // 0: no hidden states (vanilla fallback), u = e
};

// Splits of the gate GEMM for `rows` rows (their column count in *kchunk).
int gate_splits(int64_t rows, int64_t r, int64_t d, int64_t* kchunk);

// Gate of the gated head: weights bf16 or fp32, hidden bf16 or fp32.  The
// matrix-core form needs bf16 weights, d % 8 == 0, r % 8 == 0 and 16-byte
// aligned hidden, W1 and gate weight; otherwise a scalar form runs.
hipError_t launch_gate(const GateParams& g, bool weights_bf16, bool hidden_f32, hipStream_t s);

// Backward of the teacher-forced apply (training).
struct BwdParams {
  const void* grad;        // [rows, V] gradient of the corrected logits (L)
  const int64_t* ids;      // [rows] predecessors
  const void* w1;          // [V, r] (W)
  const void* w2;          // [V, r] (W)
  void* dw1;               // [V, r] output (W): zero where no valid id refers
  void* dw2;               // [V, r] output (W)
  float* partials;         // [S][rows][r] fp32 split sums of de (workspace)
  void* de;                // [rows, r] (W) input gradient of the Linear (workspace)
  int32_t* link;           // [2 rows] row links of equal ids (workspace)
  uint32_t* bad_rows;      // device error word
  int64_t rows;
  int64_t V;
  int64_t r;
  int64_t S;               // vocabulary slices of the de product
  int64_t SL;              // columns per slice
};

// Vocabulary slices of the de product (columns per slice in *slice_cols).
int64_t backward_slices(int64_t V, int64_t* slice_cols);
// dW2w, then de, then dW1 (zero-filled, then the rows of each id).  The
// matrix-core form needs bf16 weights, r % 8 == 0, r <= 256, V % 8 == 0,
// G and V * r * 2 within 2^31 bytes and 16-byte aligned G, W1 and W2w;
// scalar forms (compensated sums) run otherwise.  rows > 0.
hipError_t launch_backward(const BwdParams& p, bool logits_bf16, bool weights_bf16, hipStream_t s);

hipError_t launch_tile(const KernelParams& p, hipStream_t s);
// Streaming teacher-forced apply (bf16); needs rows * V < 2^31 and a sink of
// apply_sink_bytes() bytes.
hipError_t launch_apply_wide(const KernelParams& p, hipStream_t s);
size_t apply_sink_bytes();
// Grouped teacher-forced apply (bf16 weights; bf16 logits, or fp32 logits
// when logits_f32): from 1024 rows each distinct predecessor's bias is
// computed once; needs 1 <= rows <= 4096 and the logits and V * r * 2 at
// most 2^31 bytes.
hipError_t launch_apply_grouped(const KernelParams& p, bool logits_f32, hipStream_t s);
constexpr int64_t kGroupedApplyMaxRows = 4096;
// One sampling step with bf16 weights and bf16 or fp32 (logits_f32) logits
// (greedy or temperature) of the p.rows = B rows at
// position p.k: argmax keys per (row, 512-column block) into p.partials with
// p.nparts = sample_step_parts(V); one workgroup per CU.  Needs r <= 256,
// B <= 4096 and the logits and V * r * 2 within 2^31 bytes (hipErrorNotSupported).
int64_t sample_step_parts(int64_t V);
hipError_t launch_sample_step(const KernelParams& p, bool logits_f32, int num_cus, hipStream_t s);
// fp32 weights on the matrix cores when r and V are multiples of 4 and the
// operands 16-byte aligned (64 rows x 128 columns per workgroup), else the
// row-tile FMA kernel for any dtype pair and rank (32 rows x 128 columns per
// workgroup, the rank in chunks through LDS); sampling writes
// generic_parts(V) keys per row (p.nparts must equal it).
int64_t generic_parts(int64_t V);
hipError_t launch_generic(const KernelParams& p, bool logits_bf16, bool weights_bf16, hipStream_t s);
hipError_t launch_reduce(const uint64_t* partials, int64_t nparts, int64_t B, int64_t M, int64_t k,
                         int64_t* tokens, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

}  // namespace dspark
