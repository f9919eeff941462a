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
//     through units u = 6k + g (step k of the group in slot g) one per
//     window; slots g >= the number of groups are idle windows.  A group's
//     next step needs the tokens of its current one from every workgroup, so
//     each device-wide exchange has five windows of other work to hide in;
//   * window w: every wave multiplies group g's gathered W1 rows by its
//     slice on the matrix cores (v_mfma_f32_16x16x32_bf16), rounds the bias
//     to bf16, adds it to the group's base logits staged in LDS, writes the
//     corrected values back in place and folds each row's best column into
//     a per-row LDS key.  One barrier ends the window;
//   * everything else is issued at the start of a window and overlaps the
//     matrix work of the other waves: the corrected rows of unit w-1 go to
//     HBM and the base logits that group needs next are loaded (into
//     registers, written to the freed LDS rows a window later, four windows
//     ahead of use); wave 0 publishes the row keys of unit w-1 (a 64-bit
//     atomic max per row into one of eight key slots) and counts the
//     workgroup in for unit w-2, whose atomics it issued a window earlier;
//     wave 1 checks the arrival counts it polled a window ago for unit w+2's
//     previous step, loads those key slots into LDS, merges the slots it
//     loaded a window ago into the tokens of unit w+1, gathers their W1
//     rows (in LDS before the barrier) and polls for unit w+3.  Waves 0 and
//     1 run at raised issue priority.
// Every wait on other workgroups is bounded: a workgroup that waits too long
// records a failure in the workspace and leaves, so no launch can hang.  The
// last workgroup to leave clears the keys and counters, so the workspace is
// ready for the next call.
#include "device_common.h"
#include "markov_chain.h"

namespace dspark {

namespace {

constexpr int kWaves = 16;
constexpr int kThreads = kWaves * 64;
constexpr int kRowGroups = 6;                 // pipeline slots per step (row groups + idle slots)
constexpr int kMaxGroups = 4;                 // row groups of a call at most
constexpr int kGroupRows = 16;                // rows of a group at most (the MFMA N tile)
constexpr int kMaxRows = 64;                  // batch rows of one call
constexpr int kGroups = 8;                    // key slots / arrival counters per row group
constexpr int kPitch = 2 * 32 * kWaves + 16;  // LDS bytes of a staged row (512 columns + pad)
constexpr uint64_t kSpinTicks = 100000000;    // 1 s of the 100 MHz realtime clock
static_assert(kMaxGroups * kGroupRows >= kMaxRows && kMaxGroups <= kRowGroups, "row groups");

// Synchronisation area, one 64-byte line per word: the arrival counters
// [kRowGroups][kGroups] (cumulative over steps), then the exit counter.
static_assert((kRowGroups * kGroups + 1) * 64 <= (int)kChainSyncBytes, "sync area");
__device__ __forceinline__ uint32_t* arrival_counter(uint32_t* sync, int rg, int x) {
  return sync + 16 * (rg * kGroups + x);
}
__device__ __forceinline__ uint32_t* exit_counter(uint32_t* sync) { return sync + 16 * (kRowGroups * kGroups); }

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

// Arrival counters of row group rg: lanes 0..kGroups-1 load one each
// (arrival_load), arrival_sum adds them up, uniform over the wave.  Split so
// that a poll can be issued early and summed later.
__device__ __forceinline__ uint32_t arrival_load(uint32_t* sync, int rg, int lane) {
  return lane < kGroups ? __hip_atomic_load(arrival_counter(sync, rg, lane), __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0u;
}
__device__ __forceinline__ uint32_t arrival_sum(uint32_t v) {
#pragma unroll
  for (int d = 1; d < kGroups; d <<= 1) v += (uint32_t)__shfl_xor((int)v, d);
  return (uint32_t)__builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ uint32_t arrivals(uint32_t* sync, int rg, int lane) {
  return arrival_sum(arrival_load(sync, rg, lane));
}

// Spins until the arrival counters of row group rg sum to at least target;
// false after kSpinTicks.
__device__ bool wait_arrivals(uint32_t* sync, int rg, int lane, uint32_t target) {
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  while (arrivals(sync, rg, lane) < target) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kSpinTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

}  // namespace

template <int K32>
__global__ __launch_bounds__(kThreads) void markov_chain_greedy_bf16(ChainParams p) {
  // Gathered W1 rows per group, in the B-operand order of the matrix
  // instruction: block kk holds at lane l's 16 bytes row l % 16, rank
  // elements 32 kk + 8 (l / 16) .. +7.
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[kMaxGroups][K32 * 1024];
  // Staged logits per group: base, then corrected in place.
  __shared__ __attribute__((aligned(16))) unsigned char lds_x[kMaxGroups][kGroupRows * kPitch];
  __shared__ uint32_t lds_key[kMaxGroups][16];
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
  // The host guarantees B <= 64, V <= 32 * 16 * CUs, B*M*V < 2^30 and
  // M <= 4096, so every index below fits in 32 bits.
  const int B = (int)p.B, M = (int)p.M, V = (int)p.V, r = (int)p.r;
  // Rows are dealt into NR <= kMaxGroups groups of rpg <= 16.  A step has
  // kRowGroups slots; slots NR.. are idle windows that give each group's
  // exchange time to complete (a group's steps are kRowGroups windows apart).
  const int NR = (B + kGroupRows - 1) / kGroupRows;
  const int rpg = (B + NR - 1) / NR;
  const int U = M * kRowGroups;  // windows
  auto real = [&](int u) __attribute__((always_inline)) { return u % kRowGroups < NR; };
  uint32_t* const sync = p.sync;

  // The workgroup's columns [vbeg, vend): slices s_begin .. s_end-1.
  const int s_begin = (int)(((int64_t)g * p.S) / G);
  const int s_end = (int)(((int64_t)(g + 1) * p.S) / G);
  const uint32_t vbeg = (uint32_t)(s_begin * 32);
  const uint32_t vend = (uint32_t)(s_end * 32 < V ? s_end * 32 : V);
  const int slice = s_begin + wave;
  const bool has = slice < s_end;

  const uint32_t bytes = (uint32_t)(B * M * V * 2);
  const __amdgpu_buffer_rsrc_t rs_base = buffer_rsrc(p.base, bytes);
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

  // ---- row staging: wave w moves row w of every group, one 1 KB row
  // segment per instruction, lane l the 8 columns vbeg + 8 l .. +7.  Offsets
  // of masked-off lanes, rows or steps point past the buffer (see
  // buffer_rsrc), so every instruction is issued unconditionally.
  const int srow = wave;
  const bool col_ok = vbeg + 8u * (uint32_t)lane < vend;
  const uint32_t lane_off = 2u * (vbeg + 8u * (uint32_t)lane);
  auto row_offset = [&](int gg, int kd) __attribute__((always_inline)) -> uint32_t {
    const int b = gg * rpg + srow;
    const bool ok = srow < rpg && b < B && kd < M && col_ok;
    return ok ? (uint32_t)((b * M + kd) * V) * 2u + lane_off : kBufferOob;
  };
  // The bulk rows travel through registers (plain buffer loads issue far
  // faster than loads to LDS): a base row is loaded into pre in one window
  // and written to its LDS row at the start of the next.
  u32x4_t pre = u32x4_t{0u, 0u, 0u, 0u};
  auto load_row = [&](int gg, int kd) __attribute__((always_inline)) {
    pre = buffer_load16(rs_base, row_offset(gg, kd));
  };
  auto store_row_lds = [&](int gg) __attribute__((always_inline)) {
    *(u32x4_t*)&lds_x[gg][srow * kPitch + lane * 16] = pre;
  };

  // ---- gather (wave 1): W1 rows of tokens x (lane l: the token of row
  // l % 16 of group gg, or -1 for a zero row) into lds_e[gg].
  auto gather = [&](int gg, int x) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const int kof = 32 * kk + 8 * g4;
      const uint32_t off = (x >= 0 && kof < r) ? 2u * (uint32_t)(x * r + kof) : kBufferOob;
      load_lds16(bw_w1, off, lds_address(&lds_e[gg][kk * 1024]));
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

  // ---- prologue: stage step 0 of every group, gather the first tokens.
  for (int gg = 0; gg < NR; ++gg) {
    load_row(gg, 0);
    store_row_lds(gg);
  }
  if (wave == 1) {
    for (int gg = 0; gg < NR; ++gg) {
      const int b = gg * rpg + n16;
      int x = -1;
      if (n16 < rpg && b < B) {
        const int64_t x0 = p.first_prev[(uint32_t)b];
        if (x0 >= 0 && x0 < V) x = (int)x0;
        else if (g == 0 && g4 == 0) atomicAdd(p.bad_rows, 1u);
      }
      gather(gg, x);
    }
  } else if (wave == 0) {
    if (lane < 16) {
#pragma unroll
      for (int gg = 0; gg < kMaxGroups; ++gg) lds_key[gg][lane] = 0u;
    }
    if (lane == 0) lds_flag = 1;
  }
  wait_vmcnt<0>();
  lds_barrier();

  bool ok = true;  // wave 1: no exchange wait has timed out
  // The exchange's memory operations are few and latency-bound; the bulk
  // traffic fills this CU's memory queue.  Waves 0 and 1 issue first.
  if (wave < 2) __builtin_amdgcn_s_setprio(3);

  // ---- windows.  Window w starts with the exchange and bulk work for
  // earlier units, which overlaps the matrix work of the other waves, then
  // computes unit w = 6k + g (step k of group g); one barrier ends it.
  for (int w = 0; w < U; ++w) {
    const int gc = w % kRowGroups;  // slot of unit w (its group when real)
    int after_gather = 0;           // wave 1

    // Bulk rows first: the base row loaded a window ago (unit w+4) into its
    // LDS row, the corrected row of unit w-1 to HBM, then that group's next
    // base row (unit w+5) into registers.  It drains during the matrix work.
    if (w >= 2 && real(w - 2)) store_row_lds((w - 2) % kRowGroups);
    const bool flush = w >= 1 && real(w - 1);
    if (flush) {
      const int gp = (w - 1) % kRowGroups, kp = (w - 1) / kRowGroups;
      const u32x4_t v = *(const u32x4_t*)&lds_x[gp][srow * kPitch + lane * 16];
      buffer_store16(rs_out, row_offset(gp, kp), v);
      load_row(gp, kp + 1);
    }

    if (wave == 0) {
      // count this workgroup in for unit w-2 (its key atomics were issued a
      // window ago; the two bulk operations just issued may stay in flight),
      // then publish the row keys of unit w-1
      if (flush) wait_vmcnt<2>();
      else wait_vmcnt<0>();
      if (w >= 2 && real(w - 2) && lane == 0)
        __hip_atomic_fetch_add(arrival_counter(sync, (w - 2) % kRowGroups, xg), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      if (w >= 1 && real(w - 1) && lane < 16) {
        const int gp = (w - 1) % kRowGroups, kp = (w - 1) / kRowGroups;
        const uint32_t kw = lds_key[gp][lane];
        lds_key[gp][lane] = 0u;
        const int b = gp * rpg + lane;
        if (kw != 0u && lane < rpg && b < B) {
          const uint64_t code = kw >> 16;
          const uint32_t col = vbeg + (0xFFFFu - (kw & 0xFFFFu));
          __hip_atomic_fetch_max((uint64_t*)((unsigned char*)p.keys + key_offset(kp, xg, b)),
                                 (code << 32) | (uint64_t)(0xFFFFFFFFu - col), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    } else if (wave == 1) {
      // Targets: unit w+2 (poll issued a window ago; key slots) and unit w+1
      // (key slots loaded a window ago; merge and gather).  The wait below
      // completes the poll and key slots issued a window ago (the two bulk
      // operations just issued may stay in flight).
      const int u2 = w + 2, u1 = w + 1, u3 = w + 3;
      const bool do2 = ok && u2 < U && u2 >= kRowGroups && real(u2);
      const bool do1 = u1 < U && u1 >= kRowGroups && real(u1);
      const bool do3 = u3 < U && u3 >= kRowGroups && real(u3);
      if (flush) wait_vmcnt<2>();
      else wait_vmcnt<0>();
      // the gather first: its round trip has the rest of the window
      if (do1) gather(u1 % kRowGroups, merge(u1 & 1, u1 % kRowGroups, u1 / kRowGroups - 1));
      if (do2) {
        // complete when every workgroup has counted in unit u2 - kRowGroups
        const uint32_t target = (uint32_t)(u2 / kRowGroups) * (uint32_t)G;
        // lane x < kGroups reads counter x; the sum goes through scalar registers
        const uint32_t cx = lane < kGroups ? *(const uint32_t*)&lds_poll[lane * 16] : 0u;
        uint32_t seen = 0;
#pragma unroll
        for (int x = 0; x < kGroups; ++x) seen += (uint32_t)__builtin_amdgcn_readlane((int)cx, x);
        if (seen < target) ok = wait_arrivals(sync, u2 % kRowGroups, lane, target);
      }
      if (do2 && ok) load_keys(u2 & 1, u2 % kRowGroups, u2 / kRowGroups - 1);
      // poll the arrivals of unit w+3's previous step into LDS (lane
      // l < kGroups loads counter line l)
      if (do3 && ok)
        load_lds16_coherent(bw_sync, lane < kGroups ? (uint32_t)(4 * 16 * ((u3 % kRowGroups) * kGroups + lane)) : kBufferOob,
                            lds_address(&lds_poll[0]));
      // operations issued after the gather (waited for before the barrier)
      after_gather = (do2 && ok ? 2 : 0) + (do3 && ok ? 1 : 0);
      if (!ok && lane == 0) {
        atomicAdd(p.sync_failures, 1u);
        lds_flag = 0;
      }
    }

    // -- unit w: bias of the wave's slice for the group's rows, added to the
    // staged base logits in place; each row's best column into lds_key.
    if (has && real(w)) {
      f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
      const unsigned char* eb = &lds_e[gc][lane * 16];
#pragma unroll
      for (int kk = 0; kk < K32; ++kk) {
        const bf16x8_t bop = *(const bf16x8_t*)(eb + kk * 1024);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][kk], bop, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][kk], bop, acc1, 0, 0, 0);
      }
      const int colw = wave * 32 + 8 * g4;  // first of the lane's 8 columns in the workgroup
      // lanes of padding rows (past the group's rows or the batch) stay idle:
      // their all-zero values would send the wave down the exact pass below
      if (n16 < rpg && gc * rpg + n16 < B) {
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
    // wave 1: the gather of unit w+1 (issued this window, before the key
    // slots and the poll) is in LDS before the barrier
    if (wave == 1) {
      switch (after_gather) {
        case 5: wait_vmcnt<5>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 1: wait_vmcnt<1>(); break;
        default: wait_vmcnt<0>(); break;
      }
    }
    lds_barrier();
    if (!lds_flag) break;
  }
  // after the last window: corrected rows of the last unit, the keys of the
  // last unit, and the last two arrivals
  if (lds_flag) {
    if (real(U - 1)) {
      const int gp = (U - 1) % kRowGroups, kp = (U - 1) / kRowGroups;
      const u32x4_t v = *(const u32x4_t*)&lds_x[gp][srow * kPitch + lane * 16];
      buffer_store16(rs_out, row_offset(gp, kp), v);
    }
    if (wave == 0) {
      wait_vmcnt<0>();
      if (lane == 0 && U >= 2 && real(U - 2))
        __hip_atomic_fetch_add(arrival_counter(sync, (U - 2) % kRowGroups, xg), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      if (real(U - 1)) {
        if (lane < 16) {
          const int gp = (U - 1) % kRowGroups, kp = (U - 1) / kRowGroups;
          const uint32_t kw = lds_key[gp][lane];
          const int b = gp * rpg + lane;
          if (kw != 0u && lane < rpg && b < B) {
            const uint64_t code = kw >> 16;
            const uint32_t col = vbeg + (0xFFFFu - (kw & 0xFFFFu));
            __hip_atomic_fetch_max((uint64_t*)((unsigned char*)p.keys + key_offset(kp, xg, b)),
                                   (code << 32) | (uint64_t)(0xFFFFFFFFu - col), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        wait_vmcnt<0>();
        if (lane == 0)
          __hip_atomic_fetch_add(arrival_counter(sync, (U - 1) % kRowGroups, xg), 1u, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (wave < 2) __builtin_amdgcn_s_setprio(0);

  // Workgroup 0 writes the last step's tokens once every workgroup has
  // counted in every group.
  if (g == 0 && wave == 1 && lds_flag) {
    const uint32_t target = (uint32_t)M * (uint32_t)G;
    bool fin = true;
    for (int gg = 0; gg < NR; ++gg) {
      fin = fin && wait_arrivals(sync, gg, lane, target);
      const int b = gg * rpg + n16;
      const bool row_ok = n16 < rpg && b < B;
      const uint64_t k0 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_offset(M - 1, 2 * g4, b)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
      const uint64_t k1 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_offset(M - 1, 2 * g4 + 1, b)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0;
      const uint64_t best = max_u64(k0, k1);
      const uint64_t b2 = max_u64(best, (uint64_t)__shfl_xor((long long)best, 16));
      const uint64_t merged = max_u64(b2, (uint64_t)__shfl_xor((long long)b2, 32));
      if (g4 == 0 && row_ok) p.tokens[(uint32_t)(b * M + M - 1)] = key_index(merged);
    }
    if (!fin && lane == 0) atomicAdd(p.sync_failures, 1u);
    wait_vmcnt<0>();
  }
  wait_vmcnt<0>();
  lds_barrier();

  // Leave; the last workgroup out clears the keys and the counters (every
  // other workgroup has passed its last wait and read).
  if (tid == 0) lds_flag = (__hip_atomic_fetch_add(exit_counter(sync), 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(G - 1)) ? 1 : 0;
  lds_barrier();
  if (lds_flag) {
    for (int i = tid; i < M * kGroups * kMaxRows; i += kThreads)
      __hip_atomic_store(p.keys + (uint32_t)(i * kKeyPad), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid < kRowGroups * kGroups + 1)
      __hip_atomic_store(sync + 16 * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
template <int K32>
hipError_t launch_chain_k(const ChainParams& p, int grid, hipStream_t s) {
  hipLaunchKernelGGL((markov_chain_greedy_bf16<K32>), dim3(grid), dim3(kThreads), 0, s, p);
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
  if (p.B * p.M * p.V >= ((int64_t)1 << 30)) return hipErrorNotSupported;  // byte offsets below 2^31
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
