// markov_chain.h -- interface of the persistent greedy chain kernel
// (markov_chain.hip) and the rank-block rule it shares with the other
// kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dspark {

// Rank blocks (of 16) the tile kernel is instantiated for, covering r; 0 if none.
int tile_ks_for_rank(int64_t r);

// Arguments of the persistent greedy chain (bf16).  keys holds one 64-bit
// argmax key per (step, key group, row) at a stride of kKeyPad words; sync
// holds the arrival counters and release words (kChainSyncBytes); both are
// zero between calls.
constexpr int kKeyPad = 8;
constexpr size_t kChainSyncBytes = 4096;

struct ChainParams {
  const void* base;           // [B, M, V] bf16, or fp32 when lf32
  void* out;                  // [B, M, V] like base, or null
  const int64_t* first_prev;  // [B]
  int64_t* tokens;            // [B, M]
  const uint16_t* w1;         // [V, r]
  const uint16_t* w2;         // [V, r]
  uint64_t* keys;             // [M][chain_key_groups()][chain_max_rows()] * kKeyPad
  uint32_t* sync;             // kChainSyncBytes
  uint32_t* bad_rows;
  uint32_t* sync_failures;    // failed device-wide waits; nonzero at entry: the workspace is poisoned
  const uint32_t* test_hook;  // nonzero: every device-wide wait gives up at once (tests of the failure path)
  int64_t B;
  int64_t M;
  int64_t V;
  int64_t r;
  int64_t S;                  // 32-column vocabulary slices
  bool lf32;                  // fp32 logits (bf16 weights either way)
};

// Arguments of the persistent temperature chain (bf16): keys holds one
// 64-bit argmax key per (step, key group, row) in 16-byte slots, sync the
// arrival counters; both are zero between calls.
struct ChainSampleParams {
  const void* base;           // [B, M, V] bf16, or fp32 when lf32
  void* out;                  // [B, M, V] like base, or null
  const int64_t* first_prev;  // [B]
  int64_t* tokens;            // [B, M]
  const uint16_t* w1;         // [V, r]
  const uint16_t* w2;         // [V, r]
  uint64_t* keys;             // [M][key groups][B] * 2 words
  uint32_t* sync;             // kChainSyncBytes
  uint32_t* bad_rows;
  uint32_t* sync_failures;    // failed device-wide waits; nonzero at entry: the workspace is poisoned
  const uint32_t* test_hook;  // nonzero: every device-wide wait gives up at once (tests of the failure path)
  int64_t B;
  int64_t M;
  int64_t V;
  int64_t r;
  int64_t S;                  // 32-column vocabulary slices
  float kappa;                // log2(e) / T
  uint32_t k_abs0;            // absolute position of step 0 (noise counter)
  uint32_t batch_offset;      // absolute batch index of row 0 (noise counter)
  uint32_t seed_lo;
  uint32_t seed_hi;
  bool greedy;                // argmax of the corrected values (no noise)
  bool lf32;                  // fp32 logits (bf16 weights either way)
};

int chain_max_rows();
int chain_key_groups();
int chain_waves_per_group();
// hipErrorNotSupported when the shape does not fit the kernel or the device
// cannot hold one of its workgroups per CU.
hipError_t launch_chain_greedy(const ChainParams& p, int num_cus, hipStream_t s);

int chain_sample_max_rows();       // B at most
int chain_sample_max_step_rows();  // M * B at most
int chain_sample_slices_per_group(bool lf32);
// hipErrorNotSupported when the shape does not fit the kernel or the device
// cannot hold one of its workgroups per CU.
hipError_t launch_chain_sample(const ChainSampleParams& p, int num_cus, hipStream_t s);

}  // namespace dspark
