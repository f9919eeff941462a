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
  const uint16_t* base;       // [B, M, V]
  uint16_t* out;              // [B, M, V] or null
  const int64_t* first_prev;  // [B]
  int64_t* tokens;            // [B, M]
  const uint16_t* w1;         // [V, r]
  const uint16_t* w2;         // [V, r]
  uint64_t* keys;             // [M][chain_key_groups()][chain_max_rows()] * kKeyPad
  uint32_t* sync;             // kChainSyncBytes
  uint32_t* bad_rows;
  uint32_t* sync_failures;
  int64_t B;
  int64_t M;
  int64_t V;
  int64_t r;
  int64_t S;                  // 32-column vocabulary slices
};

int chain_max_rows();
int chain_key_groups();
int chain_waves_per_group();
hipError_t launch_chain_greedy(const ChainParams& p, int num_cus, hipStream_t s);

}  // namespace dspark
