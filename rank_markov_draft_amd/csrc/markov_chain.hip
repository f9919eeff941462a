// markov_chain.hip -- persistent left-to-right greedy chain (gfx950).
//
// sample_block_tokens (third-party markov_head.py page) is a strictly
// sequential loop over the M block positions: position k is biased by the
// token drawn at k-1.  Launching a kernel per position re-reads W2 (66 MB at
// V=129280, r=256) every step and pays a launch plus a separate reduction per
// step.  This kernel runs the whole chain in one launch, one workgroup of 16
// waves per CU:
//
//   * the vocabulary is cut into 32-column slices; each wave owns at most one
//     slice and keeps its W2w rows in VGPRs for all M steps, so W2 is read
//     from HBM once per call;
//   * the batch rows are independent chains.  They are dealt into at most
//     four row groups of up to 16 (the MFMA N tile), and the workgroup works
//     through units u = 5k + g (step k of the group in slot g) one per
//     window; slots g >= the number of groups are idle windows.  A group's
//     next step needs the tokens of its current one from every workgroup, so
//     each device-wide exchange has the four windows between a group's
//     units to complete in;
//   * window w: every wave multiplies group g's gathered W1 rows by its
//     slice on the matrix cores (v_mfma_f32_16x16x32_bf16), rounds the bias
//     to bf16, adds it to the group's base logits staged in LDS (bf16, or
//     fp32 as the drafter's vocabulary head produces them), writes the
//     corrected values back in place and folds each row's best column into
//     a per-row LDS key.  One barrier ends the window;
//   * the memory traffic is issued around the matrix work and overlaps that
//     of the other waves: waves 2..15 send the corrected rows of unit w-1 to
//     HBM and load the base logits that group needs next straight into the
//     freed LDS rows, four windows ahead of use; waves 0 and 1 run the
//     exchange, taking turns in two roles so that each waits on its own
//     memory counter only for what it issued.  One of them merges the key
//     slots of unit w+1 into tokens, gathers their W1 rows (in LDS before
//     the barrier), publishes the row keys of unit w-1 (a 64-bit atomic max
//     per row into one of eight key slots) and, after its matrix work,
//     counts the workgroup in for unit w-1; the other polls the arrival
//     counts of unit w+2's previous step and, after its matrix work, loads
//     those key slots into LDS, to merge them itself in the next window.
//     Waves 0 and 1 run at raised issue priority.
// Every wait on other workgroups is bounded: a workgroup that waits too long
// records a failure in the workspace and leaves, so no launch can hang.  The
// last workgroup to leave writes the last step's tokens (every key is in by
// then, so nobody waits for them), then clears the keys and counters, so the
// workspace is ready for the next call; when any wait failed it writes -1 to
// every token of the call instead, so a failed chain never returns plausible
// tokens.  A
// launch that finds the failure count already nonzero (a failure nobody has
// read back and cleared) does no work and also returns -1 tokens.
#include <type_traits>

#include "chain_common.h"
#include "device_common.h"
#include "markov_chain.h"

namespace dspark {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
// Pipeline slots per step: row groups plus idle slots.  A group's steps are
// kSlots windows apart; four (no idle slot for 64 rows) left too little time
// for the exchange (measured: the polls then wait on the slowest workgroup).
constexpr int kSlots = 5;
constexpr int kMaxGroups = 4;                 // row groups of a call at most
constexpr int kGroupRows = 16;                // rows of a group at most (the MFMA N tile)
constexpr int kMaxRows = 64;                  // batch rows of one call
constexpr int kGroups = kChainKeyGroups;      // key slots / arrival counters per row group
static_assert(kMaxGroups * kGroupRows >= kMaxRows && kMaxGroups <= kSlots, "row groups");

// Synchronisation area, one 64-byte line per word: the arrival counters
// [kSlots][kGroups] (cumulative over steps), then the exit counter.
static_assert((kSlots * kGroups + 1) * 64 <= (int)kChainSyncBytes, "sync area");
__device__ __forceinline__ uint32_t* arrival_counter(uint32_t* sync, int rg, int x) {
  return sync + 16 * (rg * kGroups + x);
}
__device__ __forceinline__ uint32_t* exit_counter(uint32_t* sync) { return sync + 16 * (kSlots * kGroups); }

// Byte offset of the key slot of (step k, key group x, row b).
__device__ __forceinline__ uint32_t key_offset(int k, int x, int b) {
  return (uint32_t)(((k * kGroups + x) * kMaxRows + b) * kKeyPad * 8);
}

// Order code of a bf16 value for argmax (16 bits, larger = later in the
// order): every NaN ranks highest (torch.argmax reports a NaN), -0 and +0
// share one code, otherwise the IEEE order.
__device__ __forceinline__ uint32_t argmax_code_bf16(uint32_t h) {
  const uint32_t mag = h & 0x7FFFu;
  uint32_t c = (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
  c = (mag == 0u) ? 0x8000u : c;
  c = (mag > 0x7F80u) ? 0xFFFFu : c;
  return c;
}

}  // namespace

template <int K32, bool LF32>
__global__ __launch_bounds__(kThreads) void markov_chain_greedy_bf16(ChainParams p) {
  // bf16 or (LF32) fp32 logits: bytes per logit, 1 KB segments of a staged
  // row of 512 columns, LDS bytes of a staged row
  constexpr int kEl = LF32 ? 4 : 2;
  constexpr int kSegs = LF32 ? 2 : 1;
  constexpr int kPitch = 32 * kWaves * kEl + 16;
  // Gathered W1 rows, in the B-operand order of the matrix instruction:
  // block kk holds at lane l's 16 bytes row l % 16, rank elements 32 kk +
  // 8 (l / 16) .. +7.  One buffer per group with bf16 logits; with fp32
  // logits (whose staged rows take twice the LDS) two, by unit parity.
  constexpr int kEBufs = LF32 ? 2 : kMaxGroups;
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[kEBufs][K32 * 1024];
  // Staged logits per group: base, then corrected in place.
  __shared__ __attribute__((aligned(16))) unsigned char lds_x[kMaxGroups][kGroupRows * kPitch];
  // Per-row best keys: bf16 packs a 16-bit order code and the column in the
  // workgroup into 32 bits; fp32 keeps the 64-bit argmax key.
  using key_t = typename std::conditional<LF32, unsigned long long, uint32_t>::type;
  __shared__ key_t lds_key[kMaxGroups][16];
  // Key slots loaded for a token merge, two buffers of [lane] 16 bytes each,
  // the key in the first 8 (row l % 16, key group 2 (l / 16) + j).
  __shared__ __attribute__((aligned(16))) unsigned char lds_kv[2][2 * 1024];
  __shared__ __attribute__((aligned(16))) unsigned char lds_poll[64 * 16];  // polled counter lines
  __shared__ int lds_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int xg = g % kGroups;
  // A workspace whose failure count is nonzero stays poisoned until the host
  // reads and clears it: skip all work (the exit below writes -1 tokens).
  const bool poisoned =
      __builtin_amdgcn_readfirstlane((int)__hip_atomic_load(p.sync_failures, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)) != 0;
  const bool force_timeout = __builtin_amdgcn_readfirstlane((int)*p.test_hook) != 0;
  // The host guarantees B <= 64, V <= 32 * 16 * CUs, B*M*V*kEl < 2^31 and
  // M <= 4096, so every index below fits in 32 bits.
  const int B = (int)p.B, M = (int)p.M, V = (int)p.V, r = (int)p.r;
  // Rows are dealt into NR <= kMaxGroups groups of rpg <= 16.  A step has
  // kSlots slots; slots NR.. are idle windows (a group's steps are kSlots
  // windows apart, which is the time its exchange has).
  const int NR = (B + kGroupRows - 1) / kGroupRows;
  const int rpg = (B + NR - 1) / NR;
  const int U = M * kSlots;  // windows
  auto real = [&](int u) __attribute__((always_inline)) { return u % kSlots < NR; };
  uint32_t* const sync = p.sync;

  // The workgroup's columns [vbeg, vend): slices s_begin .. s_end-1.
  const int s_begin = (int)(((int64_t)g * p.S) / G);
  const int s_end = (int)(((int64_t)(g + 1) * p.S) / G);
  const uint32_t vbeg = (uint32_t)(s_begin * 32);
  const uint32_t vend = (uint32_t)(s_end * 32 < V ? s_end * 32 : V);
  const int slice = s_begin + wave;
  const bool has = slice < s_end;

  const uint32_t bytes = (uint32_t)(B * M * V * kEl);
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(p.out, p.out != nullptr ? bytes : 0u);
  const BufferWords bw_w1 = buffer_words(p.w1, (uint32_t)(V * r * 2));
  const BufferWords bw_keys = buffer_words(p.keys, (uint32_t)(M * kGroups * kMaxRows * kKeyPad * 8));
  const BufferWords bw_sync = buffer_words(sync, (uint32_t)kChainSyncBytes);

  // A operands (columns on M, rows on N, rank on K): the slice's 32 columns
  // are two 16-column tiles t.  Lane (n16, g4) supplies W2w[col(t, n16)]
  // [32 kk + 8 g4 .. +7]; the map col(t, m) = 8 (m / 4) + 4 t + m % 4 makes
  // a lane's 4 + 4 accumulators the 8 consecutive columns 8 g4 .. 8 g4 + 7.
  bf16x8_t a[2][K32];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int vrow = slice * 32 + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const int kof = kk * 32 + 8 * g4;
      a[t][kk] = (has && vrow < V && kof < r) ? *(const bf16x8_t*)(p.w2 + (uint32_t)(vrow * r + kof)) : bf16x8_t{};
    }
  }

  // ---- row staging.  Waves 2..15 move the bulk rows, one 1 KB row segment
  // per instruction, lane l the 8 columns vbeg + 8 l .. +7: wave w moves row
  // w - 2 of every group, and waves 2 and 3 also rows 14 and 15.  Waves 0 and
  // 1 run the exchange, so their memory counters hold exchange operations
  // only.  Base rows go straight into LDS (buffer loads to LDS) as soon as a
  // group's row is flushed, four windows before the group's next unit needs
  // them; a wave waits for them only at the end of the window before that
  // unit.  Offsets of masked-off lanes, rows or steps point past the buffer
  // (see buffer_rsrc), so every instruction is issued unconditionally.
  // Segment h of a row is its columns vbeg + 1024 h / kEl ..: lane l moves
  // the 16 bytes of columns vbeg + (1024 h + 16 l) / kEl .. .
  const int nbulk = wave >= 2 ? (wave < 4 ? 2 : 1) : 0;
  const int brow0 = wave - 2, brow1 = wave + 12;
  auto row_offset = [&](int gg, int kd, int row, int h) __attribute__((always_inline)) -> uint32_t {
    const int b = gg * rpg + row;
    const uint32_t col = vbeg + (uint32_t)((1024 * h + 16 * lane) / kEl);
    const bool ok = row < rpg && b < B && kd < M && col < vend;
    return ok ? (uint32_t)((b * M + kd) * V) * (uint32_t)kEl + (uint32_t)kEl * col : kBufferOob;
  };
  const BufferWords bw_base = buffer_words(p.base, bytes);
  auto load_row_lds = [&](int gg, int kd, int row) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < kSegs; ++h)
      load_lds16(bw_base, row_offset(gg, kd, row, h), lds_address(&lds_x[gg][row * kPitch + 1024 * h]));
  };
  // Corrected row of unit (gg, kd) from LDS to HBM, then the group's next
  // base row into the same LDS row (the stores need the LDS data first).
  auto store_row = [&](int gg, int kd, int row) __attribute__((always_inline)) {
    u32x4_t v[kSegs];
#pragma unroll
    for (int h = 0; h < kSegs; ++h) v[h] = *(const u32x4_t*)&lds_x[gg][row * kPitch + 1024 * h + lane * 16];
#pragma unroll
    for (int h = 0; h < kSegs; ++h) buffer_store16(rs_out, row_offset(gg, kd, row, h), v[h]);
  };
  auto flush_row = [&](int gg, int kd, int row) __attribute__((always_inline)) {
    store_row(gg, kd, row);
    load_row_lds(gg, kd + 1, row);
  };

  // ---- gather: W1 rows of tokens x (lane l: the token of row l % 16 of the
  // unit's group, or -1 for a zero row) into lds_e[buf].
  auto gather = [&](int buf, int x) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const int kof = 32 * kk + 8 * g4;
      const uint32_t off = (x >= 0 && kof < r) ? 2u * (uint32_t)(x * r + kof) : kBufferOob;
      load_lds16(bw_w1, off, lds_address(&lds_e[buf][kk * 1024]));
    }
  };
  // Merge of the key slots in lds_kv[buf] into the tokens of group gg's
  // step kt, written to tokens[:, kt] (workgroup 0); returns lane l's token
  // (row l % 16) for the gather, or -1.  Every lane reads the eight slots of
  // its row itself (all in flight at once).
  auto merge = [&](int buf, int gg, int kt) __attribute__((always_inline)) -> int {
    uint64_t kv[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) kv[4 * j + q] = *(const uint64_t*)&lds_kv[buf][j * 1024 + (n16 + 16 * q) * 16];
    uint64_t merged = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) merged = max_u64(merged, kv[i]);
    const int b = gg * rpg + n16;
    const bool row_ok = n16 < rpg && b < B;
    const int64_t t = key_index(merged);
    if (g == 0 && g4 == 0 && row_ok) p.tokens[(uint32_t)(b * M + kt)] = t;
    return (row_ok && t >= 0 && t < V) ? (int)t : -1;
  };
  // Key slots of group gg's step kt into lds_kv[buf].
  auto load_keys = [&](int buf, int gg, int kt) __attribute__((always_inline)) {
    const int b = gg * rpg + n16;
    const bool row_ok = n16 < rpg && b < B;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      load_lds16_coherent(bw_keys, row_ok ? key_offset(kt, 2 * g4 + j, b) : kBufferOob,
                          lds_address(&lds_kv[buf][j * 1024]));
  };

  // Lane l's first token (row l % 16 of group gg), or -1 (an invalid one is
  // counted as a bad row once, by workgroup 0).
  auto first_token = [&](int gg) __attribute__((always_inline)) -> int {
    const int b = gg * rpg + n16;
    int x = -1;
    if (n16 < rpg && b < B) {
      const int64_t x0 = p.first_prev[(uint32_t)b];
      if (x0 >= 0 && x0 < V) x = (int)x0;
      else if (g == 0 && g4 == 0) atomicAdd(p.bad_rows, 1u);
    }
    return x;
  };
  // The gathered rows of unit u: per group with bf16 logits, by parity with
  // fp32 (where the first step's units past the first two are gathered in
  // the windows, like the later steps').
  auto ebuf = [&](int u) __attribute__((always_inline)) -> int { return LF32 ? (u & 1) : u % kSlots; };

  // ---- prologue: stage step 0 of every group, gather the first tokens.
  for (int gg = 0; gg < NR; ++gg) {
    if (nbulk >= 1) load_row_lds(gg, 0, brow0);
    if (nbulk >= 2) load_row_lds(gg, 0, brow1);
  }
  if (wave == 1 && !poisoned) {
    for (int gg = 0; gg < (LF32 ? (NR < 2 ? NR : 2) : NR); ++gg) gather(ebuf(gg), first_token(gg));
  } else if (wave == 0) {
    if (lane < 16) {
#pragma unroll
      for (int gg = 0; gg < kMaxGroups; ++gg) lds_key[gg][lane] = 0;
    }
    if (lane == 0) lds_flag = poisoned ? 0 : 1;
  }
  // Every group's step-0 rows are in before the first window (letting the
  // later groups' rows arrive during the first windows measured 10 us
  // slower per call: the windows then wait on loads that compete with W2's).
  wait_vmcnt<0>();
  lds_barrier();

  bool ok = true;  // this wave's exchange waits have not timed out
  // The exchange's memory operations are few and latency-bound; the bulk
  // traffic fills this CU's memory queue.  Waves 0 and 1 issue first.
  if (wave < 2) __builtin_amdgcn_s_setprio(3);

  // Row keys of unit u (lds_key of its group) into this workgroup's key
  // slots, one 64-bit atomic max per row; the group's next unit reuses
  // lds_key, so it is cleared here.
  auto publish = [&](int u) __attribute__((always_inline)) {
    if (lane < 16) {
      const int gp = u % kSlots, kp = u / kSlots;
      const key_t kw = lds_key[gp][lane];
      lds_key[gp][lane] = 0;
      const int b = gp * rpg + lane;
      if (kw != 0 && lane < rpg && b < B) {
        uint64_t key;
        if constexpr (LF32) {
          key = kw;
        } else {
          const uint64_t code = kw >> 16;
          const uint32_t col = vbeg + (0xFFFFu - (kw & 0xFFFFu));
          key = (code << 32) | (uint64_t)(0xFFFFFFFFu - col);
        }
        __hip_atomic_fetch_max((uint64_t*)((unsigned char*)p.keys + key_offset(kp, xg, b)), key, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };
  // This workgroup counted in for unit u (its key atomics are complete).
  auto count_in = [&](int u) __attribute__((always_inline)) {
    if (lane == 0)
      __hip_atomic_fetch_add(arrival_counter(sync, u % kSlots, xg), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- windows.  Window w computes unit w = 4k + g (step k of group g).
  // Waves 0 and 1 take turns in two exchange roles, so that each keeps its
  // own memory counter over the operations it has to wait for:
  //   role A (wave (w+1) & 1): merges the key slots of unit w+1 (which it
  //     loaded a window ago) into tokens and gathers their W1 rows, and
  //     publishes the row keys of unit w-1; after its matrix work it waits
  //     for both and counts the workgroup in for unit w-1;
  //   role B (wave w & 1): polls the arrivals of unit w+2's previous step
  //     (counted in at the end of the window before), and after its matrix
  //     work loads that step's key slots, which the same wave merges in the
  //     next window in role A.
  // A group's steps are kSlots windows apart: the hand-off of one step
  // (publish, count in, poll, load keys, merge and gather) takes the windows
  // between them, with one to spare for the slowest workgroup's count.
  for (int w = 0; w < (poisoned ? 0 : U); ++w) {
    const int gc = w % kSlots;  // slot of unit w (its group when real)
    const bool role_a = wave == ((w + 1) & 1);
    const bool role_b = wave == (w & 1);
    const int u1 = w + 1, u2 = w + 2;
    const bool pub = role_a && w >= 1 && real(w - 1);
    const bool do1 = role_a && u1 < U && u1 >= (LF32 ? 2 : kSlots) && real(u1);
    const bool do2 = role_b && ok && u2 < U && u2 >= kSlots && real(u2);

    // Bulk rows first: the corrected rows of unit w-1 to HBM, and that
    // group's next base rows (unit w+3) into the freed LDS rows.  They drain
    // during the matrix work and the windows after it.
    if (w >= 1 && real(w - 1)) {
      const int gp = (w - 1) % kSlots, kp = (w - 1) / kSlots;
      if (nbulk >= 1) flush_row(gp, kp, brow0);
      if (nbulk >= 2) flush_row(gp, kp, brow1);
    }

    if (role_a) {
      // the key slots of unit w+1 are in LDS; the gather first: its round
      // trip has the rest of the window
      wait_vmcnt<0>();
      if (do1) {
        int x;
        if constexpr (LF32) x = u1 < kSlots ? first_token(u1) : merge(u1 & 1, u1 % kSlots, u1 / kSlots - 1);
        else x = merge(u1 & 1, u1 % kSlots, u1 / kSlots - 1);
        gather(ebuf(u1), x);
      }
      if (pub) publish(w - 1);
    } else if (do2) {
      // lane l < kGroups loads counter line l of unit w+2's slot
      load_lds16_coherent(bw_sync, lane < kGroups ? (uint32_t)(4 * 16 * ((u2 % kSlots) * kGroups + lane)) : kBufferOob,
                          lds_address(&lds_poll[0]));
    }

    // -- unit w: bias of the wave's slice for the group's rows, added to the
    // staged base logits in place; each row's best column into lds_key.
    if (has && real(w)) {
      f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
      const unsigned char* eb = &lds_e[ebuf(w)][lane * 16];
      constexpr int KB = (K32 < 4) ? K32 : 4;
#pragma unroll
      for (int k0 = 0; k0 < K32; k0 += KB) {
        bf16x8_t bop[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) bop[i] = *(const bf16x8_t*)(eb + (k0 + i) * 1024);
        __builtin_amdgcn_sched_barrier(0);  // the reads ahead of the products (one LDS round trip per KB blocks)
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][k0 + i], bop[i], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][k0 + i], bop[i], acc1, 0, 0, 0);
        }
      }
      const int colw = wave * 32 + 8 * g4;  // first of the lane's 8 columns in the workgroup
      // lanes of padding rows (past the group's rows or the batch) stay idle:
      // their all-zero values would send the wave down the exact pass below
      if constexpr (LF32) {
        if (n16 < rpg && gc * rpg + n16 < B) {
          // bias rounded to bf16 (the Linear's output dtype), widened and
          // added to the fp32 logits with one rounding
          unsigned char* xp = &lds_x[gc][n16 * kPitch + colw * 4];
          unsigned long long key = 0ull;
#pragma unroll
          for (int t = 0; t < 2; ++t) {  // columns colw + 4 t .. + 3 (accumulators of tile t)
            const f32x4_t a4 = t ? acc1 : acc0;
            const u32x4_t bq = *(const u32x4_t*)(xp + 16 * t);
            const uint32_t bw4[4] = {bq.x, bq.y, bq.z, bq.w};
            float c4[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              c4[q] = __uint_as_float(bw4[q]) + bf16_lo(pack_bf16x2(a4[q], 0.0f));
              key = max_u64(key, argmax_key(c4[q], vbeg + (uint32_t)(colw + 4 * t + q)));
            }
            *(u32x4_t*)(xp + 16 * t) =
                u32x4_t{__float_as_uint(c4[0]), __float_as_uint(c4[1]), __float_as_uint(c4[2]), __float_as_uint(c4[3])};
          }
          if (vbeg + (uint32_t)colw < vend) {
            // the row's key slot from the lane count (recomputed here rather
            // than kept live across the window)
            const int row = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & 15;
            atomicMax(&lds_key[gc][row], key);
          }
        }
      } else if (n16 < rpg && gc * rpg + n16 < B) {
        // bias rounded to bf16 (the Linear's output dtype)
        const uint32_t bw[4] = {pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]),
                                pack_bf16x2(acc1[0], acc1[1]), pack_bf16x2(acc1[2], acc1[3])};
        unsigned char* xp = &lds_x[gc][n16 * kPitch + colw * 2];
        const u32x4_t bb = *(const u32x4_t*)xp;
        const uint32_t xw[4] = {bb.x, bb.y, bb.z, bb.w};
        uint32_t ow[4];
        uint32_t key = 0;
        float sum = 0.0f;  // NaN if a value is NaN (or +inf and -inf meet): exact pass below
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bf16_lo(xw[q]) + bf16_lo(bw[q]);
          const float hi = bf16_hi(xw[q]) + bf16_hi(bw[q]);
          ow[q] = pack_bf16x2(lo, hi);
          __asm__("" : "+v"(ow[q]));  // keep the packed word (else the codes below repack it)
          sum += lo + hi;
          // order codes of both values at once; key = code << 16 | (0xFFFF - column)
          const uint32_t c2 = pair_order_codes(ow[q]);
          const uint32_t klo = (c2 << 16) | (0xFFFFu - (uint32_t)(colw + 2 * q));
          const uint32_t khi = (c2 & 0xFFFF0000u) | (0xFFFFu - (uint32_t)(colw + 2 * q + 1));
          key = max(key, max(klo, khi));
        }
        *(u32x4_t*)xp = u32x4_t{ow[0], ow[1], ow[2], ow[3]};
        // The plain order codes rank -0 below +0 and order NaNs by payload.
        // A lane whose best value is a zero or that may hold a NaN recomputes
        // its key with the exact codes (NaN highest, -0 == +0).
        const uint32_t cm = key >> 16;
        if (sum != sum || cm == 0x7FFFu || cm == 0x8000u) {
          key = 0;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t klo = (argmax_code_bf16(ow[q] & 0xFFFFu) << 16) | (0xFFFFu - (uint32_t)(colw + 2 * q));
            const uint32_t khi = (argmax_code_bf16(ow[q] >> 16) << 16) | (0xFFFFu - (uint32_t)(colw + 2 * q + 1));
            key = max(key, max(klo, khi));
          }
        }
        if (vbeg + (uint32_t)colw < vend) atomicMax(&lds_key[gc][n16], key);
      }
    }

    if (role_a) {
      // the key atomics of unit w-1 and the gather of unit w+1 are complete
      wait_vmcnt<0>();
      if (pub) count_in(w - 1);
    } else if (do2) {
      // complete when every workgroup has counted in unit w+2 - kSlots
      wait_vmcnt<0>();
      const uint32_t target = (uint32_t)(u2 / kSlots) * (uint32_t)G;
      // lane x < kGroups reads counter x; the sum goes through scalar registers
      const uint32_t cx = lane < kGroups ? *(const uint32_t*)&lds_poll[lane * 16] : 0u;
      uint32_t seen = 0;
#pragma unroll
      for (int x = 0; x < kGroups; ++x) seen += (uint32_t)__builtin_amdgcn_readlane((int)cx, x);
      if (force_timeout) ok = false;
      else if (seen < target) ok = chain_wait_arrivals<16>(arrival_counter(sync, u2 % kSlots, 0), lane, target);
      // the key slots arrive during the next window
      if (ok) load_keys(u2 & 1, u2 % kSlots, u2 / kSlots - 1);
      else if (lane == 0) {
        atomicAdd(p.sync_failures, 1u);
        lds_flag = 0;
      }
    }
    // bulk waves: the base rows of unit w+1 (loaded at window w-3, when unit
    // w-4 was flushed) are in LDS before the barrier.  Each flush window
    // since then issued a store and a load per row.
    if (nbulk > 0 && w + 1 < U && w + 1 >= kSlots && real(w + 1)) {
      int later = 0;
      for (int x = w - kSlots + 3; x <= w; ++x) later += (x >= 1 && real(x - 1)) ? 2 * kSegs * nbulk : 0;
      wait_vmcnt_upto16(later);
    }
    lds_barrier();
    if (!lds_flag) break;
  }
  // after the last window: corrected rows of the last unit, then its keys
  // and count (the last arrival)
  if (lds_flag && real(U - 1)) {
    const int gp = (U - 1) % kSlots, kp = (U - 1) / kSlots;
    if (nbulk >= 1) store_row(gp, kp, brow0);
    if (nbulk >= 2) store_row(gp, kp, brow1);
    if (wave == 0) {
      wait_vmcnt<0>();
      publish(U - 1);
      wait_vmcnt<0>();
      count_in(U - 1);
    }
  }
  if (wave < 2) __builtin_amdgcn_s_setprio(0);
  wait_vmcnt<0>();
  lds_barrier();

  // Leave.  The last workgroup out (every other one has made its last
  // publish and count, read its last keys and written its tokens, all
  // ordered before its exit count) writes the last step's tokens from the
  // complete keys, then clears the keys and the counters; after a failure
  // it writes -1 to every token instead.
  if (tid == 0) lds_flag = (__hip_atomic_fetch_add(exit_counter(sync), 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(G - 1)) ? 1 : 0;
  lds_barrier();
  if (lds_flag) {
    const bool failed =
        poisoned || __hip_atomic_load(p.sync_failures, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (!failed && wave < NR) {
      // wave gg: group gg's rows, lane (n16, g4) reads key slots 2 g4, 2 g4 + 1 of row n16
      const int gg = wave;
      const int b = gg * rpg + n16;
      const bool row_ok = n16 < rpg && b < B;
      const uint64_t k0 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_offset(M - 1, 2 * g4, b)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
      const uint64_t k1 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_offset(M - 1, 2 * g4 + 1, b)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
      const uint64_t best = max_u64(k0, k1);
      const uint64_t merged = max_row_lanes(best);
      if (g4 == 0 && row_ok) p.tokens[(uint32_t)(b * M + M - 1)] = key_index(merged);
    }
    lds_barrier();  // the last keys are read before they are cleared
    for (int i = tid; i < M * kGroups * kMaxRows; i += kThreads)
      __hip_atomic_store(p.keys + (uint32_t)(i * kKeyPad), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < kSlots * kGroups + 1)
      __hip_atomic_store(sync + 16 * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (failed)
      for (int i = tid; i < B * M; i += kThreads) p.tokens[(uint32_t)i] = -1;
  }
}

// ---------------------------------------------------------------- launcher
namespace {

// A plain launch of one 1024-thread workgroup per CU: the kernel's LDS and
// VGPR use admit one workgroup per CU, so on an idle device all of them are
// resident together (a cooperative launch would guarantee it, at about 17 us
// of extra launch latency measured on MI355X).  The host declines the chain
// when the occupancy query says a CU cannot hold a workgroup.  If a
// workgroup still cannot start while the others wait (CUs held by other
// streams' kernels), their bounded waits end the launch with a recorded
// synchronisation failure and -1 tokens instead of a hang.
// Workgroups of markov_chain_greedy_bf16<K32, LF32> one CU of the current
// device can hold, cached per device; the chain needs at least one.
template <int K32, bool LF32>
int chain_occupancy() {
  static int cache[64];
  static bool known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!known[dev]) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, markov_chain_greedy_bf16<K32, LF32>, kThreads, 0) !=
        hipSuccess)
      blocks = 0;
    cache[dev] = blocks;
    known[dev] = true;
  }
  return cache[dev];
}

template <int K32>
hipError_t launch_chain_k(const ChainParams& p, int grid, hipStream_t s) {
  if (p.lf32) {
    if (chain_occupancy<K32, true>() < 1) return hipErrorNotSupported;
    hipLaunchKernelGGL((markov_chain_greedy_bf16<K32, true>), dim3(grid), dim3(kThreads), 0, s, p);
  } else {
    if (chain_occupancy<K32, false>() < 1) return hipErrorNotSupported;
    hipLaunchKernelGGL((markov_chain_greedy_bf16<K32, false>), dim3(grid), dim3(kThreads), 0, s, p);
  }
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
  if (p.B * p.M * p.V * (p.lf32 ? 4 : 2) >= ((int64_t)1 << 31)) return hipErrorNotSupported;  // byte offsets below 2^31
  if (p.M > 4096) return hipErrorNotSupported;                              // key area below 2^31 bytes
  if (p.S > (int64_t)num_cus * kWaves) return hipErrorNotSupported;
  switch (ks) {  // rank blocks of 16 -> blocks of 32 (zero-padded)
    case 1:
    case 2: return launch_chain_k<1>(p, num_cus, s);
    case 4: return launch_chain_k<2>(p, num_cus, s);
    case 8: return launch_chain_k<4>(p, num_cus, s);
    case 16: return launch_chain_k<8>(p, num_cus, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace dspark
