// chain_common.h -- device-wide exchange helpers shared by the persistent
// chain kernels (markov_chain.hip: greedy, markov_chain_sample.hip:
// temperature).
//
// Each kernel runs one workgroup per CU.  After a workgroup has published its
// partial argmax keys of a unit (64-bit atomic max into one of kChainKeyGroups
// key slots per row), it adds one to an arrival counter of that unit's slot;
// the counters are cumulative over steps, so step k of a slot is complete
// when the kChainKeyGroups counters of the slot sum to (k + 1) times the
// grid size.  Every wait on other workgroups is bounded.
#pragma once

#include "device_common.h"

namespace dspark {

constexpr int kChainKeyGroups = 8;                // key slots / arrival counters per unit slot
constexpr uint64_t kChainSpinTicks = 100000000;  // 1 s of the 100 MHz realtime clock

// Lane x < kChainKeyGroups loads counter x of a slot, whose counters start at
// `slot` and lie `stride` words apart.
template <int stride>
__device__ __forceinline__ uint32_t chain_arrival_load(uint32_t* slot, int lane) {
  return lane < kChainKeyGroups
             ? __hip_atomic_load(slot + stride * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
             : 0u;
}

// Sum of the counters loaded by lanes 0 .. kChainKeyGroups - 1, uniform over
// the wave: read lane by lane into scalar registers (a few cycles each)
// rather than by shuffles through LDS (a round trip each, on the poll's
// critical path).
__device__ __forceinline__ uint32_t chain_arrival_sum(uint32_t v) {
  uint32_t s = 0;
#pragma unroll
  for (int x = 0; x < kChainKeyGroups; ++x) s += (uint32_t)__builtin_amdgcn_readlane((int)v, x);
  return s;
}

// Spins until the counters of a slot sum to at least target; false after
// kChainSpinTicks.
template <int stride>
__device__ bool chain_wait_arrivals(uint32_t* slot, int lane, uint32_t target) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (chain_arrival_sum(chain_arrival_load<stride>(slot, lane)) < target) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kChainSpinTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// s_waitcnt vmcnt(n) for a count known only at run time (0..16; more waits
// for 16).
__device__ __forceinline__ void wait_vmcnt_upto16(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    default: wait_vmcnt<16>(); break;
  }
}

}  // namespace dspark
