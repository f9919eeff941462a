// markov_chain.hip -- persistent left-to-right greedy chain (gfx950).
//
// sample_block_tokens (third-party markov_head.py page) is a strictly
// sequential loop over the M block positions: position k is biased by the
// token drawn at k-1.  Launching a kernel per position re-reads W2 (66 MB at
// V=129280, r=256) every step and pays a launch plus a separate reduction per
// step.  This kernel runs the whole chain in one cooperative launch:
//
//   * one workgroup of 16 waves per CU; the vocabulary is cut into 32-column
//     slices and each wave owns at most one slice, whose W2w rows it keeps in
//     VGPRs for all M steps (W2 is read from HBM once per call);
//   * per step every workgroup gathers the W1 rows of the B current
//     predecessors into LDS and multiplies them on the matrix cores
//     (v_mfma_f32_32x32x16_bf16, vocabulary on M, batch rows on N); the
//     rounded bias goes to LDS row-major, and each wave then streams whole
//     rows of the workgroup's columns (one 1 KB row segment per wave
//     instruction): base logits in, corrected logits out, and the row's
//     argmax key folded across the wave;
//   * the base logits of step k+1 are requested right after step k's are
//     consumed, so they arrive while the device-wide token exchange runs;
//   * the exchange: each workgroup merges its per-row keys into a device-wide
//     key per (step, row) with a 64-bit atomic max, then arrives on a counter;
//     the next step starts when all workgroups have arrived.  Every wait is
//     bounded: a workgroup that waits too long records a failure in the
//     workspace and leaves, so no launch can hang.
// The last workgroup to leave clears the keys and the counter, so the
// workspace is ready for the next call.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kMaxRows = 64;                 // batch rows per call of this kernel
constexpr int kGroups = 8;                   // key slots / arrival groups (one per XCD)
constexpr uint64_t kSpinTicks = 100000000;   // 1 s of the 100 MHz realtime clock

// Words of the synchronisation area (one 64-byte line each).
__device__ __forceinline__ uint32_t* group_counter(uint32_t* sync, int x) { return sync + 16 * x; }
__device__ __forceinline__ uint32_t* global_counter(uint32_t* sync) { return sync + 16 * kGroups; }
__device__ __forceinline__ uint32_t* release_word(uint32_t* sync, int x) { return sync + 16 * (kGroups + 1 + x); }
__device__ __forceinline__ uint32_t* exit_counter(uint32_t* sync) { return sync + 16 * (2 * kGroups + 1); }

__device__ __forceinline__ uint64_t* key_slot(uint64_t* keys, int64_t k, int x, int b) {
  return keys + ((k * kGroups + x) * kMaxRows + b) * kKeyPad;
}

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *w >= target.  Returns false after kSpinTicks.  The polls are
// relaxed device-scope loads: everything exchanged between workgroups (keys,
// counters, release words) goes through device-scope atomics, so no acquire
// (which would invalidate this XCD's L2 on every poll) is needed.
__device__ bool wait_word(const uint32_t* w, uint32_t target) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
    __builtin_amdgcn_s_sleep(1);
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) return false;
  }
  return true;
}

// Two-level arrival of workgroup g for step k (one thread): the last
// arrival of g's group bumps the global counter, and the last group to arrive
// publishes k+1 in every group's release word; the workgroup then waits on
// its own group's word (wait_word(release_word(sync, g % kGroups), k + 1)).
// With a single counter and a single word, 256 workgroups contend on one
// address; this halves the cost of a round on MI355X (measured).
__device__ void arrive(uint32_t* sync, int g, int G, int64_t k) {
  const int ngroups = G < kGroups ? G : kGroups;
  const int x = g % kGroups;
  const uint32_t in_group = (uint32_t)((G - x + kGroups - 1) / kGroups);
  const uint32_t step = (uint32_t)(k + 1);
  if (atomic_add_agent(group_counter(sync, x), 1u) == in_group * step - 1u) {
    if (atomic_add_agent(global_counter(sync), 1u) == (uint32_t)ngroups * step - 1u)
      for (int y = 0; y < ngroups; ++y)
        __hip_atomic_store(release_word(sync, y), step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

template <int KS>
__global__ __launch_bounds__(kThreads) void markov_chain_greedy_bf16(ChainParams p) {
  constexpr int CPR = 2 * KS;               // 16-byte chunks per gathered W1 row
  constexpr int ESTRIDE = 32 * KS + 16;     // LDS bytes per gathered row
  constexpr int COLS = 32 * kWaves;         // columns of a workgroup (at most)
  constexpr int BSTRIDE = 2 * COLS + 16;    // LDS bytes per bias row
  constexpr int RPW = kMaxRows / kWaves;    // rows streamed per wave
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[kMaxRows * ESTRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[kMaxRows * BSTRIDE];
  __shared__ uint64_t lds_key[kMaxRows];
  __shared__ int64_t lds_tok[kMaxRows];
  __shared__ int lds_flag;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 31;
  const int h = lane >> 5;
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int xg = g % kGroups;
  const int64_t B = p.B, M = p.M, V = p.V, r = p.r;
  const int nchunks = (int)((B + 31) / 32);
  const uint16_t* __restrict__ w1 = p.w1;
  const uint16_t* __restrict__ base = p.base;
  uint16_t* __restrict__ out = p.out;

  // The workgroup's columns [vbeg, vend): slices s_begin .. s_end-1.
  const int64_t s_begin = ((int64_t)g * p.S) / G;
  const int64_t s_end = ((int64_t)(g + 1) * p.S) / G;
  const uint32_t vbeg = (uint32_t)(s_begin * 32);
  const uint32_t vend = (uint32_t)(s_end * 32 < V ? s_end * 32 : V);
  // This wave's slice for the matrix work.
  const int64_t slice = s_begin + wave;
  const bool has = slice < s_end;

  // A operand (W2w rows of the slice), permuted so that the lane's 16
  // accumulators are the 16 consecutive columns slice*32 + 16h + i.
  bf16x8_t a[KS];
  {
    const int perm = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
    const int64_t vrow = slice * 32 + perm;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int64_t kof = kk * 16 + 8 * h;
      if (has && vrow < V && kof < r)
        a[kk] = *(const bf16x8_t*)(p.w2 + vrow * r + kof);
      else
        a[kk] = bf16x8_t{};
    }
  }

  // Streaming: wave w handles rows RPW*w + i; lane l the 8 columns
  // vbeg + 8l .. +7 of them (whole 16-byte vectors since V % 8 == 0).
  // Element offsets fit in 32 bits (the host requires B*M*V < 2^31).
  const uint32_t vl = vbeg + 8u * (uint32_t)lane;
  const bool col_ok = vl < vend;
  u32x4_t pre[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const uint32_t b = RPW * wave + i;
    pre[i] = (b < B && col_ok)
                 ? __builtin_nontemporal_load((const u32x4_t*)(base + (b * (uint32_t)M) * (uint32_t)V + vl))
                 : u32x4_t{0u, 0u, 0u, 0u};
  }

  // Stores the wave's corrected rows of step kd (held in pre[]) and requests
  // its base logits of step kd + 1.
  auto drain = [&](int64_t kd) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint32_t b = RPW * wave + i;
      if (b >= B) break;
      if (out != nullptr && col_ok)
        __builtin_nontemporal_store(pre[i], (u32x4_t*)(out + (b * (uint32_t)M + (uint32_t)kd) * (uint32_t)V + vl));
      if (kd + 1 < M)
        pre[i] = col_ok ? __builtin_nontemporal_load(
                              (const u32x4_t*)(base + (b * (uint32_t)M + (uint32_t)kd + 1u) * (uint32_t)V + vl))
                        : u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  for (int64_t k = 0; k < M; ++k) {
    // A1: predecessors of step k: first_prev, or the merge of the eight
    // group slots of step k-1.
    if (tid < kMaxRows) {
      int64_t x = -1;
      if (tid < B) {
        if (k == 0) {
          x = p.first_prev[tid];
          if (x < 0 || x >= V) {
            if (g == 0) atomicAdd(p.bad_rows, 1u);
            x = -1;
          }
        } else {
          uint64_t best = 0;
#pragma unroll
          for (int y = 0; y < kGroups; ++y)
            best = max_u64(best, __hip_atomic_load(key_slot(p.keys, k - 1, y, tid), __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT));
          x = key_index(best);
          if (g == 0) p.tokens[tid * M + k - 1] = x;
          if (x < 0 || x >= V) x = -1;  // never after a complete exchange
        }
      }
      lds_tok[tid] = x;
    }
    __syncthreads();

    // Wave 0 drains the previous step now, after its low-latency loads.
    if (wave == 0 && k > 0) drain(k - 1);

    // A2: gather the W1 rows (zero rows for padding and invalid ids), by
    // waves 1.. (wave 0's loads are queued behind its drain).
    for (int c = tid - 64; c < nchunks * 32 * CPR; c += kThreads - 64) {
      if (c < 0) break;
      const int row = c / CPR;
      const int part = c - row * CPR;
      const int64_t x = lds_tok[row];
      u32x4_t d = u32x4_t{0u, 0u, 0u, 0u};
      if (x >= 0 && part * 8 < r) d = *(const u32x4_t*)(w1 + x * r + part * 8);
      *(u32x4_t*)(lds_e + row * ESTRIDE + part * 16) = d;
    }
    __syncthreads();

    // A3: the bias of the wave's slice for every row, rounded to bf16 (the
    // Linear's output dtype), into LDS row-major.
    if (has) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c >= nchunks) break;
        f32x16_t acc = f32x16_t{};
        const unsigned char* eb = lds_e + (32 * c + m) * ESTRIDE + h * 16;
#pragma unroll
        for (int k2 = 0; k2 < KS; k2 += 2) {
          bf16x8_t bop[2];
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (k2 + j < KS) bop[j] = *(const bf16x8_t*)(eb + (k2 + j) * 32);
#pragma unroll
          for (int j = 0; j < 2; ++j)
            if (k2 + j < KS) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k2 + j], bop[j], acc, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        u32x4_t lo, hi;
        lo.x = pack_bf16x2(acc[0], acc[1]);
        lo.y = pack_bf16x2(acc[2], acc[3]);
        lo.z = pack_bf16x2(acc[4], acc[5]);
        lo.w = pack_bf16x2(acc[6], acc[7]);
        hi.x = pack_bf16x2(acc[8], acc[9]);
        hi.y = pack_bf16x2(acc[10], acc[11]);
        hi.z = pack_bf16x2(acc[12], acc[13]);
        hi.w = pack_bf16x2(acc[14], acc[15]);
        unsigned char* bp = lds_b + (32 * c + m) * BSTRIDE + (wave * 32 + 16 * h) * 2;
        *(u32x4_t*)bp = lo;
        *(u32x4_t*)(bp + 16) = hi;
      }
    }
    __syncthreads();

    // A4 + A5: corrected rows (kept in registers until the keys are out) and
    // each row's best column of this workgroup.
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint32_t b = RPW * wave + i;
      if (b >= B) break;  // uniform over the wave
      const u32x4_t bb = pre[i];
      const u32x4_t bs = *(const u32x4_t*)(lds_b + b * BSTRIDE + lane * 16);
      float c[8];
      c[0] = bf16_lo(bb.x) + bf16_lo(bs.x);
      c[1] = bf16_hi(bb.x) + bf16_hi(bs.x);
      c[2] = bf16_lo(bb.y) + bf16_lo(bs.y);
      c[3] = bf16_hi(bb.y) + bf16_hi(bs.y);
      c[4] = bf16_lo(bb.z) + bf16_lo(bs.z);
      c[5] = bf16_hi(bb.z) + bf16_hi(bs.z);
      c[6] = bf16_lo(bb.w) + bf16_lo(bs.w);
      c[7] = bf16_hi(bb.w) + bf16_hi(bs.w);
      u32x4_t o;
      o.x = pack_bf16x2(c[0], c[1]);
      o.y = pack_bf16x2(c[2], c[3]);
      o.z = pack_bf16x2(c[4], c[5]);
      o.w = pack_bf16x2(c[6], c[7]);
      pre[i] = o;
      // a NaN among the fp32 sums makes this NaN (+inf + -inf too: rechecked)
      const float s8 = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
      uint32_t col, code;
      wave_row_argmax_bf16(o, col_ok, s8 != s8, (uint32_t)lane, &col, &code);
      if (lane == 0)
        lds_key[b] = (col < 0xFFFFu) ? (((uint64_t)code << 32) | (uint64_t)(0xFFFFFFFFu - (vbeg + col))) : 0;
    }
    __syncthreads();

    // Exchange.  Wave 0 merges the row keys into this group's slots and
    // waits until its atomics are performed, then one thread arrives.  (No
    // release fence: it would write back the XCD's whole L2, dirty with
    // corrected logits, twice per step and workgroup.)
    if (wave == 0) {
      if (lane < B && vbeg < vend)
        __hip_atomic_fetch_max(key_slot(p.keys, k, xg, lane), lds_key[lane], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
    }
    if (tid == 0) arrive(p.sync, g, G, k);
    // Waves 1.. write their corrected rows and request the next step's base
    // logits while the exchange completes.  Wave 0 keeps its memory queue
    // empty until it has read the next tokens: its polls and key loads would
    // otherwise wait behind these (the vector memory counter is in order).
    if (wave != 0) drain(k);
    if (tid == 0) {
      const bool ok = wait_word(release_word(p.sync, xg), (uint32_t)(k + 1));
      if (!ok) atomicAdd(p.sync_failures, 1u);
      lds_flag = ok ? 1 : 0;
    }
    __syncthreads();
    if (!lds_flag) return;
  }

  if (wave == 0) drain(M - 1);

  // Tokens of the last step.
  if (tid < B && g == 0) {
    uint64_t best = 0;
#pragma unroll
    for (int y = 0; y < kGroups; ++y)
      best = max_u64(best, __hip_atomic_load(key_slot(p.keys, M - 1, y, tid), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT));
    p.tokens[tid * M + M - 1] = key_index(best);
  }
  __syncthreads();

  // Leave; the last workgroup out clears the keys and the synchronisation
  // words (every other workgroup has passed its last wait and read).
  if (tid == 0) lds_flag = (atomic_add_agent(exit_counter(p.sync), 1u) == (uint32_t)(G - 1)) ? 1 : 0;
  __syncthreads();
  if (lds_flag) {
    for (int64_t i = tid; i < M * kGroups * kMaxRows; i += kThreads)
      __hip_atomic_store(p.keys + i * kKeyPad, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < 2 * kGroups + 2)
      __hip_atomic_store(p.sync + 16 * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------- launcher
namespace {

// A plain launch of one 1024-thread workgroup per CU: the kernel's LDS and
// VGPR use admit one workgroup per CU, so on an idle device all of them are
// resident together (a cooperative launch would guarantee it, at about 17 us
// of extra launch latency measured on MI355X).  If a workgroup cannot start
// while the others wait, their bounded waits end the launch with a recorded
// synchronisation failure instead of a hang.
template <int KS>
hipError_t launch_chain_ks(const ChainParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((markov_chain_greedy_bf16<KS>), dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int chain_max_rows() { return kMaxRows; }
int chain_key_groups() { return kGroups; }
int chain_waves_per_group() { return kWaves; }

// Returns hipErrorNotSupported when the shape does not fit the kernel.
hipError_t launch_chain_greedy(const ChainParams& p, int num_cus, hipStream_t s) {
  const int ks = tile_ks_for_rank(p.r);
  if (p.B > kMaxRows || ks == 0 || ks > 16) return hipErrorNotSupported;
  if (p.B * p.M * p.V >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  if (p.S > (int64_t)num_cus * kWaves) return hipErrorNotSupported;
  switch (ks) {
    case 1: return launch_chain_ks<1>(p, num_cus, s);
    case 2: return launch_chain_ks<2>(p, num_cus, s);
    case 4: return launch_chain_ks<4>(p, num_cus, s);
    case 8: return launch_chain_ks<8>(p, num_cus, s);
    case 16: return launch_chain_ks<16>(p, num_cus, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace dspark
