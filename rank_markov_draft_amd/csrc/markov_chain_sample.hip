// markov_chain_sample.hip -- persistent left-to-right temperature chain (gfx950).
//
// Temperature sampling in sample_block_tokens (third-party markov_head.py
// page, _sample_tokens) draws the token of position k from softmax(c / T),
// c the corrected logits biased by the token drawn at k-1.  Here the draw is
// the Gumbel-max form the step kernels use: the first argmax over v of
// fmaf(c_v, log2(e) / T, g_v), g_v base-2 Gumbel noise from Philox4x32-10 of
// (v / 4, k_abs, b_abs, 0) under the seed.  A kernel per position re-reads W2
// (78 MB at V=151936, r=256) every step; this kernel runs all M positions in
// one launch with W2 resident on the CUs, one workgroup of 16 waves per CU:
//
//   * the workgroup's columns are cut into 32-column slices (up to 20);
//     wave w keeps the W2 rows of slice w in VGPRs for all M steps, and the
//     rows of slices 16.. sit in LDS, each multiplied as two 16-column tiles
//     by two of waves 4..11, so that no wave scores more than one and a half
//     slices and the SIMDs carrying the exchange waves get the fewest tiles.
//     Four waves per SIMD (128 VGPRs each) hide the latency of the scoring's
//     dependent chains (the Philox rounds);
//   * the batch rows are dealt into row groups of up to 16 (the MFMA N
//     tile); unit u = S k + g is step k of group g, S = max(groups, 5)
//     slots per step (slots past the groups are idle), and window w
//     computes unit w: every wave multiplies the group's gathered W1 rows
//     by its slices on the matrix cores, rounds the bias to bf16, adds it to
//     the staged base logits, scores every column and folds each row's best
//     key into LDS.  One barrier ends the window;
//   * waves 2..15 stage the base rows of unit w+2 into LDS (buffer loads to
//     LDS), and when the corrected logits are returned they first send the
//     rows of unit w-1 from LDS to HBM;
//   * waves 0 and 1 run the exchange of the greedy chain (markov_chain.hip):
//     in turns, one merges the key slots of unit w+1 into tokens, gathers
//     their W1 rows, publishes the row keys of unit w-1 and counts the
//     workgroup in; the other polls the arrival counts of unit w+2's
//     previous step and loads its key slots.  A group's steps are S windows
//     apart, so at 16 groups the exchange has fifteen windows of slack.
// Every wait on other workgroups is bounded; the last workgroup to leave
// writes the last step's tokens, clears the keys and counters, and writes -1
// to every token instead when a wait failed (or the workspace was already
// poisoned by an unread failure).  Instantiated with GREEDY the kernel
// selects the first argmax of the corrected values, without noise: the
// greedy calls the greedy chain does not take (more rows, or more columns
// per CU) run on it.  Instantiated with LF32 it reads and writes fp32
// logits (bf16 weights either way): the bf16 bias is widened and added in
// fp32, a workgroup takes up to 19 slices, and the base rows of unit w+1
// load during window w (a ring of two units, as the rows are twice as wide).
#include "chain_common.h"
#include "device_common.h"
#include "markov_chain.h"

namespace dspark {

namespace {

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTWaves = 16;
constexpr int kTThreads = kTWaves * 64;
constexpr int kTBulk = kTWaves - 2;          // staging waves (2 .. 15)
// LDS layout by logits dtype: bf16 rows of up to 640 columns (four LDS
// slices) in a ring of three units (the rows of unit w+2 load during window
// w); fp32 rows, twice the bytes, of up to 608 columns (three LDS slices) in
// a ring of two (the rows of unit w+1 load during window w).
template <bool LF32>
struct TLayout {
  static constexpr int El = LF32 ? 4 : 2;              // bytes per logit
  static constexpr int Extra = LF32 ? 3 : 4;           // slices whose W2 rows sit in LDS
  static constexpr int Slices = kTWaves + Extra;       // slices of a workgroup at most
  static constexpr int Pitch = 32 * Slices * El + 16;  // LDS bytes of a staged row (+ pad)
  static constexpr int Ring = LF32 ? 2 : 3;            // staged units
  static constexpr int SegCols = 1024 / El;            // columns of a 1 KB row segment
};
constexpr int kTGroupRows = 16;              // rows of a group at most
constexpr int kTMaxGroups = 16;              // row groups of a call at most (256 rows)
constexpr int kTMinSlots = 5;                // slots per step at least
constexpr int kTKeyWords = 2;                // words per key slot (16 bytes: the DMA unit)
constexpr int kTStride = 4;                  // words between arrival counters
constexpr int kTMaxStepRows = 4096;        // M * B at most (key area)

// Arrival counter x of slot rg, and the exit counter after all of them.
__device__ __forceinline__ uint32_t* t_counter(uint32_t* sync, int rg, int x) {
  return sync + kTStride * (rg * kChainKeyGroups + x);
}
__device__ __forceinline__ uint32_t* t_exit_counter(uint32_t* sync) {
  return sync + kTStride * (kTMaxGroups * kChainKeyGroups);
}
static_assert((kTMaxGroups * kChainKeyGroups + 1) * kTStride * 4 <= (int)kChainSyncBytes, "sync area");
// The 16-column tile q = 2 e + t of LDS slice e (tile t: columns 16 t ..
// 16 t + 15 in the matrix instruction's order) is multiplied by wave
// 6, 7, 10, 11, 4, 5, 8, 9 (q = 0..7): with three LDS slices SIMDs 2 and 3
// take two tiles and SIMDs 0 and 1, whose waves 0 and 1 run the exchange,
// one each.  -1 for the other waves.
__device__ __forceinline__ int extra_tile_of_wave(int wave) {
  switch (wave) {
    case 6: return 0;
    case 7: return 1;
    case 10: return 2;
    case 11: return 3;
    case 4: return 4;
    case 5: return 5;
    case 8: return 6;
    case 9: return 7;
    default: return -1;
  }
}
// The best key of a lane's N consecutive columns vcol .. vcol + N - 1 with
// corrected values cv and noise words w: the first column of the highest
// score fmaf(cv, kappa, g); a NaN corrected value (the only source of a NaN
// score, the noise being finite) ranks above all, the first one winning.
template <int N>
__device__ __forceinline__ uint64_t score_key(const float (&cv)[N], const uint32_t (&w)[N], float kappa,
                                              uint32_t vcol) {
  float sc[N];
#pragma unroll
  for (int q = 0; q < N; ++q) sc[q] = __builtin_fmaf(cv[q], kappa, gumbel2_from_word(w[q]));
  // NaN-propagating maximum (v_maximum3_f32): a score is NaN exactly when
  // its corrected value is (the noise and kappa are finite), so a NaN best
  // flags the lane's NaN columns at no extra cost
  float best = sc[0];
#pragma unroll
  for (int q = 1; q < N; ++q) best = __builtin_elementwise_maximum(best, sc[q]);
  uint32_t bi = N - 1;
#pragma unroll
  for (int q = N - 2; q >= 0; --q) bi = sc[q] == best ? (uint32_t)q : bi;
  uint64_t k = argmax_key(best, vcol + bi);
  if (best != best) {
    uint32_t first = N - 1;
#pragma unroll
    for (int q = N - 2; q >= 0; --q)
      if (cv[q] != cv[q]) first = (uint32_t)q;
    k = (0xFFFFFFFFull << 32) | (uint64_t)(0xFFFFFFFFu - (vcol + first));
  }
  return k;
}
// The same for greedy selection: the score is the corrected value itself.
template <int N>
__device__ __forceinline__ uint64_t value_key(const float (&cv)[N], uint32_t vcol) {
  float best = cv[0];
#pragma unroll
  for (int q = 1; q < N; ++q) best = fmaxf(best, cv[q]);
  uint32_t bi = N - 1;
#pragma unroll
  for (int q = N - 2; q >= 0; --q) bi = cv[q] == best ? (uint32_t)q : bi;
  uint64_t k = argmax_key(best, vcol + bi);
  uint32_t first = N;
#pragma unroll
  for (int q = N - 1; q >= 0; --q)
    if (cv[q] != cv[q]) first = (uint32_t)q;
  if (first < N) k = (0xFFFFFFFFull << 32) | (uint64_t)(0xFFFFFFFFu - (vcol + first));
  return k;
}
// the key slots of M * B <= kTMaxStepRows step-rows fit the chain area's keys
// (16 steps x 8 key groups x 64 rows of 64-byte slots)
static_assert(kTMaxStepRows * kChainKeyGroups * kTKeyWords * 8 <= 16 * 8 * 64 * kKeyPad * 8, "key area");

}  // namespace

// GREEDY: the same chain selecting the argmax of the corrected values (no
// noise); it serves greedy calls of more rows than the greedy chain takes.
// LF32: fp32 logits (bf16 weights either way).
template <int K32, bool GREEDY, bool LF32>
__global__ __launch_bounds__(kTThreads) void markov_chain_sample_bf16(ChainSampleParams p) {
  using L = TLayout<LF32>;
  constexpr int kTExtra = L::Extra, kTPitch = L::Pitch, kTRing = L::Ring;
  // Gathered W1 rows of units u (buffer u % 2), in the B-operand order of the
  // matrix instruction: block kk holds at lane l's 16 bytes row l % 16,
  // rank elements 32 kk + 8 (l / 16) .. +7.
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[2][K32 * 1024];
  // Staged logits of units u (slot u % kTRing): base, then corrected.
  __shared__ __attribute__((aligned(16))) unsigned char lds_x[kTRing][kTGroupRows * kTPitch];
  // W2 rows of the LDS slices, block (kk, t) at (2 kk + t) * 1024 in the
  // A-operand order of the register slices (lane l's 16 bytes).
  __shared__ __attribute__((aligned(16))) unsigned char lds_w2[kTExtra][2 * K32 * 1024];
  __shared__ uint64_t lds_key[2][16];  // row keys of units u (buffer u % 2)
  // Key slots loaded for a merge, two buffers of [lane] 16 bytes each, the
  // key in the first 8 (row l % 16, key group 2 (l / 16) + j).
  __shared__ __attribute__((aligned(16))) unsigned char lds_kv[2][2 * 1024];
  __shared__ __attribute__((aligned(16))) unsigned char lds_poll[64 * 16];
  __shared__ int lds_flag;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int xg = g % kChainKeyGroups;
  const bool poisoned =
      __builtin_amdgcn_readfirstlane((int)__hip_atomic_load(p.sync_failures, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT)) != 0;
  const bool force_timeout = __builtin_amdgcn_readfirstlane((int)*p.test_hook) != 0;
  // The host guarantees B <= 256, M * B <= 4096, V % 8 == 0, V <= 640 * CUs
  // and B * M * V < 2^30, so every index below fits in 32 bits.
  const int B = (int)p.B, M = (int)p.M, V = (int)p.V, r = (int)p.r;
  const int NR = (B + kTGroupRows - 1) / kTGroupRows;
  const int rpg = (B + NR - 1) / NR;
  const int NS = NR > kTMinSlots ? NR : kTMinSlots;  // slots per step
  const int U = M * NS;                               // windows
  auto real = [&](int u) __attribute__((always_inline)) { return u % NS < NR; };
  uint32_t* const sync = p.sync;
  const bool ret = p.out != nullptr;

  // The workgroup's columns [vbeg, vend): slices s_begin .. s_end - 1;
  // wave w's register slice is slice w of the workgroup, its LDS tile (if
  // any) tile extra_tile_of_wave(w) of slices 16...
  const int s_begin = (int)(((int64_t)g * p.S) / G);
  const int s_end = (int)(((int64_t)(g + 1) * p.S) / G);
  const uint32_t vbeg = (uint32_t)(s_begin * 32);
  const uint32_t vend = (uint32_t)(s_end * 32 < V ? s_end * 32 : V);
  const int ncols = (int)(vend - vbeg);               // <= 640, a multiple of 8
  // 1 KB row segments (bf16: one or two, fp32: one to three)
  const int nseg = LF32 ? (ncols > L::SegCols ? (ncols + L::SegCols - 1) / L::SegCols : 1) : (ncols > L::SegCols ? 2 : 1);
  const int xq = extra_tile_of_wave(wave);

  const uint32_t bytes = (uint32_t)(B * M * V * L::El);
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(p.out, ret ? bytes : 0u);
  const BufferWords bw_base = buffer_words(p.base, bytes);
  const BufferWords bw_w1 = buffer_words(p.w1, (uint32_t)(V * r * 2));
  const BufferWords bw_keys = buffer_words(p.keys, (uint32_t)(M * kChainKeyGroups * B * kTKeyWords * 8));
  const BufferWords bw_sync = buffer_words(sync, (uint32_t)kChainSyncBytes);
  auto key_off = [&](int k, int x, int b) __attribute__((always_inline)) -> uint32_t {
    return (uint32_t)(((k * kChainKeyGroups + x) * B + b) * kTKeyWords * 8);
  };

  // A operands of slice i (columns on M, rows on N, rank on K): its 32
  // columns are two 16-column tiles t; lane (n16, g4) supplies
  // W2w[col(t, n16)][32 kk + 8 g4 .. +7] with col(t, m) = 8 (m / 4) + 4 t +
  // m % 4, so a lane's 4 + 4 accumulators are the 8 consecutive columns
  // 8 g4 .. 8 g4 + 7 of the slice.
  bf16x8_t a[2][K32];
  {
    const int slice = s_begin + wave;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int vrow = slice * 32 + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
      for (int kk = 0; kk < K32; ++kk) {
        const int kof = kk * 32 + 8 * g4;
        a[t][kk] = (slice < s_end && vrow < V && kof < r) ? *(const bf16x8_t*)(p.w2 + (uint32_t)(vrow * r + kof))
                                                         : bf16x8_t{};
      }
    }
  }
  // the LDS slices' blocks, dealt over all waves (loads to LDS)
  const BufferWords bw_w2 = buffer_words(p.w2, (uint32_t)(V * r * 2));
  for (int d = wave; d < kTExtra * 2 * K32; d += kTWaves) {
    const int e = d / (2 * K32), kk = (d % (2 * K32)) >> 1, t = d & 1;
    const int slice = s_begin + kTWaves + e;
    if (slice >= s_end) continue;
    const int vrow = slice * 32 + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
    const int kof = kk * 32 + 8 * g4;
    load_lds16(bw_w2, (vrow < V && kof < r) ? (uint32_t)(vrow * r + kof) * 2u : kBufferOob,
               lds_address(&lds_w2[e][(2 * kk + t) * 1024]));
  }

  // ---- row staging by waves 2..15: row i (0..15) of a unit is moved by
  // wave 2 + i % 14 as nseg segments of SegCols columns (1 KB), lane l the
  // 16 bytes at column base + 16 l / El, base = SegCols h for all but the
  // last segment and ncols - SegCols for the last (which overlaps the one
  // before).  One wave moves a row's segments, so its corrected values are
  // read for the store before the next unit's loads overwrite any of them.
  // Offsets of masked-off lanes, rows or steps point past the buffer, so
  // every instruction is unconditional.
  const int bw = wave - 2;  // bulk index (negative for waves 0 and 1)
  auto seg_base = [&](int h) __attribute__((always_inline)) -> uint32_t {
    if constexpr (LF32) return h < nseg - 1 ? (uint32_t)(L::SegCols * h) : (nseg > 1 ? (uint32_t)(ncols - L::SegCols) : 0u);
    else return h ? (uint32_t)(ncols - L::SegCols) : 0u;
  };
  auto seg_offset = [&](int u, int row, int h) __attribute__((always_inline)) -> uint32_t {
    const int gg = u % NS, kd = u / NS;
    const int b = gg * rpg + row;
    const uint32_t col = vbeg + seg_base(h) + (uint32_t)(16 / L::El) * (uint32_t)lane;
    const bool ok = row < rpg && b < B && kd < M && col < vend;
    return ok ? (uint32_t)((b * M + kd) * V) * (uint32_t)L::El + (uint32_t)L::El * col : kBufferOob;
  };
  // the segment's LDS base (a load to LDS puts lane l's 16 bytes at base + 16 l)
  auto seg_lds = [&](int u, int row, int h) __attribute__((always_inline)) -> unsigned char* {
    return &lds_x[u % kTRing][row * kTPitch + L::El * seg_base(h)];
  };
  // bulk operations this wave issues per staged unit
  const int my_segs = bw < 0 ? 0 : nseg * ((kTGroupRows - bw + kTBulk - 1) / kTBulk);
  auto load_unit = [&](int u) __attribute__((always_inline)) {
    for (int i = bw; i < kTGroupRows; i += kTBulk)
      for (int h = 0; h < nseg; ++h) load_lds16(bw_base, seg_offset(u, i, h), lds_address(seg_lds(u, i, h)));
  };
  auto flush_unit = [&](int u) __attribute__((always_inline)) {
    for (int i = bw; i < kTGroupRows; i += kTBulk)
      for (int h = 0; h < nseg; ++h)
        buffer_store16(rs_out, seg_offset(u, i, h), *(const u32x4_t*)(seg_lds(u, i, h) + lane * 16));
  };

  // ---- exchange pieces (waves 0 and 1)
  // W1 rows of tokens x (lane l: the token of row l % 16, or -1 for a zero
  // row) into lds_e[buf].
  auto gather = [&](int buf, int x) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const int kof = 32 * kk + 8 * g4;
      const uint32_t off = (x >= 0 && kof < r) ? 2u * (uint32_t)(x * r + kof) : kBufferOob;
      load_lds16(bw_w1, off, lds_address(&lds_e[buf][kk * 1024]));
    }
  };
  // Predecessor tokens of unit u for its gather (lane l: row l % 16): the
  // first tokens for step 0 (invalid ones count as bad rows once, by
  // workgroup 0), else the merge of the key slots in lds_kv[u % 2], whose
  // tokens workgroup 0 writes to tokens[:, k - 1].
  auto predecessor = [&](int u) __attribute__((always_inline)) -> int {
    const int gg = u % NS, kd = u / NS;
    const int b = gg * rpg + n16;
    const bool row_ok = n16 < rpg && b < B;
    if (kd == 0) {
      int x = -1;
      if (row_ok) {
        const int64_t x0 = p.first_prev[(uint32_t)b];
        if (x0 >= 0 && x0 < V) x = (int)x0;
        else if (g == 0 && g4 == 0) atomicAdd(p.bad_rows, 1u);
      }
      return x;
    }
    uint64_t kv[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) kv[4 * j + q] = *(const uint64_t*)&lds_kv[u & 1][j * 1024 + (n16 + 16 * q) * 16];
    uint64_t merged = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) merged = max_u64(merged, kv[i]);
    const int64_t t = key_index(merged);
    if (g == 0 && g4 == 0 && row_ok) p.tokens[(uint32_t)(b * M + kd - 1)] = t;
    return (row_ok && t >= 0 && t < V) ? (int)t : -1;
  };
  // Key slots of unit u's previous step into lds_kv[u % 2].
  auto load_keys = [&](int u) __attribute__((always_inline)) {
    const int gg = u % NS, kt = u / NS - 1;
    const int b = gg * rpg + n16;
    const bool row_ok = n16 < rpg && b < B;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      load_lds16_coherent(bw_keys, row_ok ? key_off(kt, 2 * g4 + j, b) : kBufferOob,
                          lds_address(&lds_kv[u & 1][j * 1024]));
  };
  auto publish = [&](int u) __attribute__((always_inline)) {
    if (lane < 16) {
      const int gp = u % NS, kp = u / NS;
      const uint64_t kw = lds_key[u & 1][lane];
      lds_key[u & 1][lane] = 0ull;
      const int b = gp * rpg + lane;
      if (kw != 0ull && lane < rpg && b < B)
        __hip_atomic_fetch_max((uint64_t*)((unsigned char*)p.keys + key_off(kp, xg, b)), kw, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  auto count_in = [&](int u) __attribute__((always_inline)) {
    if (lane == 0)
      __hip_atomic_fetch_add(t_counter(sync, u % NS, xg), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // ---- prologue: the first units' rows, the first unit's W1 rows.
  for (int u = 0; u < kTRing - 1 && u < U; ++u)
    if (real(u)) load_unit(u);
  if (wave == 1 && !poisoned) gather(0, predecessor(0));
  if (wave == 0) {
    if (lane < 32) (&lds_key[0][0])[lane] = 0ull;
    if (lane == 0) lds_flag = poisoned ? 0 : 1;
  }
  wait_vmcnt<0>();
  lds_barrier();

  bool ok = true;  // this wave's exchange waits have not timed out
  // Issue priority: the exchange waves first, then the waves with an LDS
  // tile (one and a half slices), so that the waves with one slice, not
  // those with more, end the window.
  if (wave < 2) __builtin_amdgcn_s_setprio(3);
  else if (xq >= 0 && xq < 2 * (s_end - s_begin - kTWaves)) __builtin_amdgcn_s_setprio(2);

  for (int w = 0; w < (poisoned ? 0 : U); ++w) {
    const bool role_a = wave == ((w + 1) & 1);
    const bool role_b = wave == (w & 1);
    const int u1 = w + 1, u2 = w + 2;
    const bool pub = role_a && w >= 1 && real(w - 1);
    const bool do1 = role_a && u1 < U && real(u1);
    const bool do2 = role_b && ok && u2 < U && u2 >= NS && real(u2);

    // bulk: the corrected rows of unit w-1 out, then the base rows of unit
    // w+2 into the slot it freed
    int issued = 0;
    if (bw >= 0) {
      if (ret && w >= 1 && real(w - 1)) {
        flush_unit(w - 1);
        issued += my_segs;
      }
      if (w + kTRing - 1 < U && real(w + kTRing - 1)) {
        load_unit(w + kTRing - 1);
        issued += my_segs;
      }
    }

    if (role_a) {
      // the key slots of unit w+1 are in LDS (loaded by this wave a window ago)
      wait_vmcnt<0>();
      if (do1) gather(u1 & 1, predecessor(u1));
      if (pub) publish(w - 1);
    } else if (do2) {
      load_lds16_coherent(bw_sync, lane < kChainKeyGroups ? (uint32_t)(4 * kTStride * ((u2 % NS) * kChainKeyGroups + lane))
                                                         : kBufferOob,
                          lds_address(&lds_poll[0]));
    }

    // -- unit w: each slice's bias for the group's rows, the corrected
    // values, their scores and each row's best key into lds_key.
    if (real(w)) {
      const int gc = w % NS, kd = w / NS;
      const int row = gc * rpg + n16;
      const bool row_ok = n16 < rpg && row < B;
      const unsigned char* eb = &lds_e[w & 1][lane * 16];
      unsigned char* xrow = &lds_x[w % kTRing][n16 * kTPitch];
      const uint32_t brow = p.batch_offset + (uint32_t)row;
      const uint32_t kabs = p.k_abs0 + (uint32_t)kd;
      uint64_t key = 0ull;
      // opaque per window: else the compiler keeps loop-invariant Philox
      // products and the ten round keys live across the windows (and spills
      // them)
      uint32_t seed_lo = p.seed_lo, seed_hi = p.seed_hi;
      __asm__ volatile("" : "+s"(seed_lo), "+s"(seed_hi));
      const bool has_reg = s_begin + wave < s_end;
      const int xs = kTWaves + (xq >> 1);  // the LDS tile's slice within the workgroup
      const bool has_tile = xq >= 0 && s_begin + xs < s_end;
      const unsigned char* ab = &lds_w2[xq >= 0 ? xq >> 1 : 0][(xq & 1) * 1024 + lane * 16];
      f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{}, acc2 = f32x4_t{};
      constexpr int KB = (K32 < 2) ? K32 : 2;
#pragma unroll
      for (int k0 = 0; k0 < K32; k0 += KB) {
        bf16x8_t bop[KB], aop[KB];
#pragma unroll
        for (int q = 0; q < KB; ++q) bop[q] = *(const bf16x8_t*)(eb + (k0 + q) * 1024);
        if (has_tile) {
#pragma unroll
          for (int q = 0; q < KB; ++q) aop[q] = *(const bf16x8_t*)(ab + (k0 + q) * 2048);
        }
        __builtin_amdgcn_sched_barrier(0);  // the reads ahead of the products
#pragma unroll
        for (int q = 0; q < KB; ++q) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][k0 + q], bop[q], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][k0 + q], bop[q], acc1, 0, 0, 0);
        }
        if (has_tile) {
#pragma unroll
          for (int q = 0; q < KB; ++q) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop[q], bop[q], acc2, 0, 0, 0);
        }
      }
      // corrected values: the bias rounded to bf16 (the Linear's output
      // dtype), the sum rounded to the bf16 logits
      // the register slice: the lane's 8 columns 32 wave + 8 g4 .. +7
      const uint32_t colw = (uint32_t)(wave * 32 + 8 * g4);
      if (has_reg && row_ok && vbeg + colw < vend) {
        float cv[8];
        if constexpr (LF32) {
          // fp32 logits: the bf16 bias widened and added with one rounding
          unsigned char* xp = xrow + colw * 4;
          const u32x4_t b0 = *(const u32x4_t*)xp, b1 = *(const u32x4_t*)(xp + 16);
          const uint32_t xw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
          const float a8[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
#pragma unroll
          for (int q = 0; q < 8; ++q) cv[q] = __uint_as_float(xw[q]) + bf16_rne(a8[q]);
          if (ret) {
            *(u32x4_t*)xp = u32x4_t{__float_as_uint(cv[0]), __float_as_uint(cv[1]), __float_as_uint(cv[2]), __float_as_uint(cv[3])};
            *(u32x4_t*)(xp + 16) =
                u32x4_t{__float_as_uint(cv[4]), __float_as_uint(cv[5]), __float_as_uint(cv[6]), __float_as_uint(cv[7])};
          }
        } else {
          // both roundings in the float domain (one instruction each)
          unsigned char* xp = xrow + colw * 2;
          const u32x4_t bb = *(const u32x4_t*)xp;
          const uint32_t xw[4] = {bb.x, bb.y, bb.z, bb.w};
          const float a8[8] = {acc0[0], acc0[1], acc0[2], acc0[3], acc1[0], acc1[1], acc1[2], acc1[3]};
#pragma unroll
          for (int q = 0; q < 8; ++q)
            cv[q] = bf16_rne(((q & 1) ? bf16_hi(xw[q >> 1]) : bf16_lo(xw[q >> 1])) + bf16_rne(a8[q]));
          if (ret)
            *(u32x4_t*)xp = u32x4_t{join_bf16(cv[0], cv[1]), join_bf16(cv[2], cv[3]), join_bf16(cv[4], cv[5]),
                                    join_bf16(cv[6], cv[7])};
        }
        uint32_t vcol = vbeg + colw;
        if constexpr (GREEDY) {
          key = value_key<8>(cv, vcol);
        } else {
          __asm__ volatile("" : "+v"(vcol));  // opaque, as the seeds
          // columns vcol .. + 3 and vcol + 4 .. + 7 are the words of two
          // Philox blocks, computed as two interleaved chains
          Philox4 qa, qb;
          philox4x32_10_pair(vcol >> 2, (vcol >> 2) + 1u, kabs, brow, 0u, seed_lo, seed_hi, qa, qb);
          const uint32_t words[8] = {qa.x0, qa.x1, qa.x2, qa.x3, qb.x0, qb.x1, qb.x2, qb.x3};
          key = score_key<8>(cv, words, p.kappa, vcol);
        }
      }
      // the LDS tile: the lane's 4 columns 32 xs + 8 g4 + 4 t .. +3 (one
      // Philox block)
      const uint32_t colt = (uint32_t)(xs * 32 + 8 * g4 + 4 * (xq & 1));
      if (has_tile && row_ok && vbeg + colt < vend) {
        float cv[4];
        if constexpr (LF32) {
          unsigned char* xp = xrow + colt * 4;
          const u32x4_t bb = *(const u32x4_t*)xp;
          const uint32_t xw[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) cv[q] = __uint_as_float(xw[q]) + bf16_rne(acc2[q]);
          if (ret)
            *(u32x4_t*)xp = u32x4_t{__float_as_uint(cv[0]), __float_as_uint(cv[1]), __float_as_uint(cv[2]), __float_as_uint(cv[3])};
        } else {
          unsigned char* xp = xrow + colt * 2;
          const u32x2_t bb = *(const u32x2_t*)xp;
          const uint32_t xw[2] = {bb.x, bb.y};
#pragma unroll
          for (int q = 0; q < 4; ++q)
            cv[q] = bf16_rne(((q & 1) ? bf16_hi(xw[q >> 1]) : bf16_lo(xw[q >> 1])) + bf16_rne(acc2[q]));
          if (ret) *(u32x2_t*)xp = u32x2_t{join_bf16(cv[0], cv[1]), join_bf16(cv[2], cv[3])};
        }
        uint32_t vcol = vbeg + colt;
        if constexpr (GREEDY) {
          key = max_u64(key, value_key<4>(cv, vcol));
        } else {
          __asm__ volatile("" : "+v"(vcol));
          const Philox4 q4 = philox4x32_10(vcol >> 2, kabs, brow, 0u, seed_lo, seed_hi);
          const uint32_t words[4] = {q4.x0, q4.x1, q4.x2, q4.x3};
          key = max_u64(key, score_key<4>(cv, words, p.kappa, vcol));
        }
      }
      // the row's four lanes (n16 + 16 j), then one LDS max per row and wave
      key = max_row_lanes(key);
      if (g4 == 0 && key != 0ull) atomicMax((unsigned long long*)&lds_key[w & 1][n16], (unsigned long long)key);
    }

    if (role_a) {
      // the key atomics of unit w-1 and the gather of unit w+1 are complete
      wait_vmcnt<0>();
      if (pub) count_in(w - 1);
    } else if (do2) {
      // complete when every workgroup has counted in unit w+2 - NS
      wait_vmcnt<0>();
      const uint32_t target = (uint32_t)(u2 / NS) * (uint32_t)G;
      const uint32_t cx = lane < kChainKeyGroups ? *(const uint32_t*)&lds_poll[lane * 16] : 0u;
      uint32_t seen = 0;
#pragma unroll
      for (int x = 0; x < kChainKeyGroups; ++x) seen += (uint32_t)__builtin_amdgcn_readlane((int)cx, x);
      if (force_timeout) ok = false;
      else if (seen < target) ok = chain_wait_arrivals<kTStride>(t_counter(sync, u2 % NS, 0), lane, target);
      if (ok) load_keys(u2);  // merged by this wave in the next window
      else if (lane == 0) {
        atomicAdd(p.sync_failures, 1u);
        lds_flag = 0;
      }
    }
    // bulk: the rows of unit w+1 are in LDS before the barrier: with a ring
    // of three they were loaded a window ago and this window's operations
    // may stay in flight; with two they were loaded in this window
    if (bw >= 0) {
      if constexpr (kTRing == 2) wait_vmcnt<0>();
      else wait_vmcnt_upto16(issued);
    }
    lds_barrier();
    if (!lds_flag) break;
  }
  // after the last window: the corrected rows of the last unit, then its
  // keys and count
  if (lds_flag && real(U - 1)) {
    if (ret && bw >= 0) flush_unit(U - 1);
    if (wave == 0) {
      wait_vmcnt<0>();
      publish(U - 1);
      wait_vmcnt<0>();
      count_in(U - 1);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  wait_vmcnt<0>();
  lds_barrier();

  // Leave.  The last workgroup out writes the last step's tokens from the
  // complete keys, then clears the keys and the counters; after a failure
  // it writes -1 to every token instead.
  if (tid == 0)
    lds_flag = (__hip_atomic_fetch_add(t_exit_counter(sync), 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(G - 1))
                   ? 1
                   : 0;
  lds_barrier();
  if (lds_flag) {
    const bool failed =
        poisoned || __hip_atomic_load(p.sync_failures, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (!failed) {
      for (int gg = wave; gg < NR; gg += kTWaves) {
        // lane (n16, g4) reads key slots 2 g4, 2 g4 + 1 of row n16
        const int b = gg * rpg + n16;
        const bool row_ok = n16 < rpg && b < B;
        const uint64_t k0 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_off(M - 1, 2 * g4, b)),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0;
        const uint64_t k1 = row_ok ? __hip_atomic_load((uint64_t*)((unsigned char*)p.keys + key_off(M - 1, 2 * g4 + 1, b)),
                                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0;
        const uint64_t best = max_u64(k0, k1);
        const uint64_t merged = max_row_lanes(best);
        if (g4 == 0 && row_ok) p.tokens[(uint32_t)(b * M + M - 1)] = key_index(merged);
      }
    }
    lds_barrier();  // the last keys are read before they are cleared
    for (int i = tid; i < M * kChainKeyGroups * B; i += kTThreads)
      __hip_atomic_store(p.keys + (uint32_t)(i * kTKeyWords), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid <= kTMaxGroups * kChainKeyGroups)
      __hip_atomic_store(sync + kTStride * tid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (failed)
      for (int i = tid; i < B * M; i += kTThreads) p.tokens[(uint32_t)i] = -1;
  }
}

// ---------------------------------------------------------------- launcher
namespace {

// Workgroups of markov_chain_sample_bf16<K32, GREEDY, LF32> one CU of the
// current device can hold, cached per device; the chain needs at least one.
template <int K32, bool GREEDY, bool LF32>
int chain_sample_occupancy() {
  static int cache[64];
  static bool known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!known[dev]) {
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, markov_chain_sample_bf16<K32, GREEDY, LF32>, kTThreads,
                                                     0) != hipSuccess)
      blocks = 0;
    cache[dev] = blocks;
    known[dev] = true;
  }
  return cache[dev];
}

template <int K32, bool GREEDY, bool LF32>
hipError_t launch_chain_sample_i(const ChainSampleParams& p, int grid, hipStream_t s) {
  if (chain_sample_occupancy<K32, GREEDY, LF32>() < 1) return hipErrorNotSupported;
  hipLaunchKernelGGL((markov_chain_sample_bf16<K32, GREEDY, LF32>), dim3(grid), dim3(kTThreads), 0, s, p);
  return hipGetLastError();
}

template <int K32>
hipError_t launch_chain_sample_k(const ChainSampleParams& p, int grid, hipStream_t s) {
  if (p.lf32) return p.greedy ? launch_chain_sample_i<K32, true, true>(p, grid, s)
                              : launch_chain_sample_i<K32, false, true>(p, grid, s);
  return p.greedy ? launch_chain_sample_i<K32, true, false>(p, grid, s)
                  : launch_chain_sample_i<K32, false, false>(p, grid, s);
}

}  // namespace

int chain_sample_max_rows() { return kTGroupRows * kTMaxGroups; }
int chain_sample_max_step_rows() { return kTMaxStepRows; }
int chain_sample_slices_per_group(bool lf32) { return lf32 ? TLayout<true>::Slices : TLayout<false>::Slices; }

hipError_t launch_chain_sample(const ChainSampleParams& p, int num_cus, hipStream_t s) {
  const int ks = tile_ks_for_rank(p.r);
  if (p.B < 1 || p.B > chain_sample_max_rows() || p.M < 1 || p.M * p.B > kTMaxStepRows || ks == 0 || ks > 16)
    return hipErrorNotSupported;
  // byte offsets below 2^31
  if (p.V % 8 != 0 || p.B * p.M * p.V * (p.lf32 ? 4 : 2) >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  if (p.S > (int64_t)num_cus * chain_sample_slices_per_group(p.lf32)) return hipErrorNotSupported;
  switch (ks) {  // rank blocks of 16 -> blocks of 32 (zero-padded)
    case 1:
    case 2: return launch_chain_sample_k<1>(p, num_cus, s);
    case 4: return launch_chain_sample_k<2>(p, num_cus, s);
    case 8: return launch_chain_sample_k<4>(p, num_cus, s);
    case 16: return launch_chain_sample_k<8>(p, num_cus, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace dspark
