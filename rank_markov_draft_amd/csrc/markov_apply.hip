// markov_apply.hip -- teacher-forced block bias, streaming form (gfx950).
//
// apply_block_logits (third-party markov_head.py page) biases every row
// (b, k) of base[B, M, V] by W2 . W1[token_ids[b, k]] and adds the result to
// the base logits.  The bytes are the base logits in and the corrected
// logits out; W2 is read once.  Layout of the work:
//
//   * a workgroup owns 32*WAVES consecutive vocabulary columns; each wave
//     keeps the W2w rows of one 32-column slice in VGPRs for the whole
//     launch (so W2 is read from HBM exactly once);
//   * the rows are walked in chunks of RC rows.  For chunk c the W1 rows of
//     the predecessors sit in LDS; the waves multiply them on the matrix
//     cores (v_mfma_f32_16x16x32_bf16: columns on M, rows on N, rank on K)
//     and write the bias, rounded to bf16 (the Linear's output dtype), to
//     LDS row-major;
//   * then every thread streams 16-byte vectors of whole row segments
//     (consecutive lanes, consecutive columns): base in, fp32 add, one
//     rounding, corrected out;
//   * software pipeline: the base logits are loaded into a two-slot register
//     ring two chunks ahead of use, and the W1 rows of chunk c+1 into
//     registers (written to LDS at the end of chunk c), while chunk c is
//     multiplied and streamed.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

template <int K32, int WAVES, int RC>
__global__ __launch_bounds__(WAVES * 64) void markov_apply_wide_bf16(KernelParams p) {
  constexpr int THREADS = WAVES * 64;
  constexpr int CPR = 4 * K32;                 // 16-byte chunks of a gathered W1 row (rank padded to 32*K32)
  constexpr int ESTRIDE = 64 * K32 + 16;       // LDS bytes per gathered row
  constexpr int COLS = 32 * WAVES;             // columns of the workgroup
  constexpr int BSTRIDE = 2 * COLS + 16;       // LDS bytes per bias row
  constexpr int VPR = COLS / 8;                // 16-byte vectors per row segment
  constexpr int VPT = RC * VPR / THREADS;      // streamed vectors per thread and chunk
  constexpr int GTOT = RC * CPR;               // gathered vectors per chunk
  constexpr int GPT = (GTOT + THREADS - 1) / THREADS;
  constexpr int NT = RC / 16;                  // 16-row MFMA tiles per chunk
  static_assert(VPT * THREADS == RC * VPR, "stream mapping");
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[RC * ESTRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[RC * BSTRIDE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int64_t V = p.V, r = p.r, rows = p.rows;
  const int64_t S = (V + 31) / 32;
  const int64_t vbeg = (int64_t)blockIdx.x * COLS;
  const int64_t vend = (vbeg + COLS < V) ? vbeg + COLS : V;
  const int64_t slice = (int64_t)blockIdx.x * WAVES + wave;
  const bool has = slice < S;
  const uint16_t* __restrict__ w1 = (const uint16_t*)p.w1;
  const uint16_t* __restrict__ base = (const uint16_t*)p.base;
  uint16_t* __restrict__ out = (uint16_t*)p.out;
  const int64_t nchunks = (rows + RC - 1) / RC;

  // A operands (v_mfma_f32_16x16x32_bf16: columns on M, rows on N, rank on
  // K): the slice's 32 columns are two 16-column tiles t.  Lane (n = l%16,
  // g = l/16) supplies W2w[col(t, n)][32kk + 8g .. +7]; the tile-row ->
  // column map col(t, m) = 8(m/4) + 4t + m%4 makes a lane's 4 + 4
  // accumulators of the two tiles the 8 consecutive columns 8g .. 8g+7.
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  bf16x8_t a[2][K32];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int64_t vrow = slice * 32 + 8 * (n16 >> 2) + 4 * t + (n16 & 3);
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const int64_t kof = kk * 32 + 8 * g4;
      a[t][kk] = (has && vrow < V && kof < r) ? *(const bf16x8_t*)((const uint16_t*)p.w2 + vrow * r + kof)
                                              : bf16x8_t{};
    }
  }

  // Every global access of the chunk loop is unconditional: lanes past the
  // last row or column load from clamped (valid) addresses and store into a
  // per-thread sink vector of the workspace.  Loads or stores in branches
  // make the compiler wait for every outstanding memory operation at the
  // join, which serialises the pipeline.  Element offsets fit in 32 bits
  // (the host requires rows * V < 2^31).
  const uint32_t Vu = (uint32_t)V;
  const uint32_t last_row = (uint32_t)(rows - 1);
  const uint32_t last_vec = (uint32_t)(vend - 8);
  u32x4_t* sink = (u32x4_t*)p.sink + tid;

  // Token ids: gather vector q of chunk c is row (tid + q*THREADS) / CPR,
  // part (tid + q*THREADS) % CPR.  nid[] holds the ids of the next chunk.
  int64_t nid[GPT];
  auto load_ids = [&](int64_t c) {
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int e = tid + q * THREADS;
      const int64_t n = c * RC + (e < GTOT ? e / CPR : 0);
      nid[q] = p.ids[n < (int64_t)last_row ? n : (int64_t)last_row];
    }
  };
  uint32_t bad = 0;  // out-of-range ids seen by this thread (workgroup 0 only)
  bool g_ok[GPT];
  auto gather = [&](int64_t c, u32x4_t g[GPT]) {
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int e = tid + q * THREADS;
      const int row = e < GTOT ? e / CPR : 0;
      const int part = e < GTOT ? e - row * CPR : 0;
      const int64_t x = nid[q];
      const bool x_ok = x >= 0 && x < V;
      const bool part_ok = part * 8 < r;
      g[q] = *(const u32x4_t*)(w1 + (x_ok ? x : 0) * r + (part_ok ? part * 8 : 0));
      g_ok[q] = x_ok && part_ok;
      if (blockIdx.x == 0 && e < GTOT && part == 0 && !x_ok && c * RC + row < rows) ++bad;
    }
  };
  // Zeroing of invalid ids and rank padding happens here, at the end of the
  // chunk, so the select does not wait for the load early.
  auto gather_to_lds = [&](const u32x4_t g[GPT]) {
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int e = tid + q * THREADS;
      const int row = e / CPR;
      const int part = e - row * CPR;
      if (e < GTOT)
        *(u32x4_t*)(&lds_e[row * ESTRIDE + part * 16]) = g_ok[q] ? g[q] : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  // Stream vector q of this thread in chunk c: row c*RC + (tid+q*THREADS)/VPR,
  // vector (tid+q*THREADS) % VPR of the workgroup's row segment.
  auto stream_row = [&](int64_t c, int q) { return c * RC + (tid + q * THREADS) / VPR; };
  auto stream_col = [&](int q) {
    const int e = tid + q * THREADS;
    return (uint32_t)vbeg + 8u * (uint32_t)(e - (e / VPR) * VPR);
  };
  auto load_base = [&](int64_t c, int q) {
    const int64_t n = stream_row(c, q);
    const uint32_t v = stream_col(q);
    const uint32_t off = (n < (int64_t)last_row ? (uint32_t)n : last_row) * Vu + (v < last_vec ? v : last_vec);
    return __builtin_nontemporal_load((const u32x4_t*)(base + off));
  };

  u32x4_t g[GPT];
  u32x4_t ring[2][VPT];  // base logits of chunks c (slot c & 1) and c + 1
  load_ids(0);
  gather(0, g);
  load_ids(1);
#pragma unroll
  for (int q = 0; q < VPT; ++q) ring[0][q] = load_base(0, q);
#pragma unroll
  for (int q = 0; q < VPT; ++q) ring[1][q] = load_base(1, q);
  gather_to_lds(g);
  __syncthreads();

  // One chunk; slot is compile-time so the ring stays in registers.
  auto chunk = [&](int64_t c, u32x4_t pre[VPT]) {
    // In flight during this chunk: W1 rows of chunk c+1 (ids loaded a chunk
    // ago) and the ids of chunk c+2; base logits of c+1 (issued last chunk).
    gather(c + 1, g);
    load_ids(c + 2);

    // A3: bias of the wave's slice for the chunk's rows, one 16-row tile at
    // a time (8 accumulators live), rounded to bf16 into LDS row-major.
    if (has) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
        const unsigned char* eb = &lds_e[(16 * nt + n16) * ESTRIDE + g4 * 16];
#pragma unroll
        for (int kk = 0; kk < K32; ++kk) {
          const bf16x8_t bop = *(const bf16x8_t*)(eb + kk * 64);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][kk], bop, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][kk], bop, acc1, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        u32x4_t w;
        w.x = pack_bf16x2(acc0[0], acc0[1]);
        w.y = pack_bf16x2(acc0[2], acc0[3]);
        w.z = pack_bf16x2(acc1[0], acc1[1]);
        w.w = pack_bf16x2(acc1[2], acc1[3]);
        *(u32x4_t*)(lds_b + (16 * nt + n16) * BSTRIDE + (wave * 32 + 8 * g4) * 2) = w;
      }
    }
    __syncthreads();

    // A4: stream the chunk; its register slot is refilled with chunk c+2.
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int e = tid + q * THREADS;
      const int row = e / VPR;
      const int vi = e - row * VPR;
      const int64_t n = stream_row(c, q);
      const uint32_t v = stream_col(q);
      const u32x4_t bb = pre[q];
      pre[q] = load_base(c + 2, q);
      const u32x4_t bs = *(const u32x4_t*)(lds_b + row * BSTRIDE + vi * 16);
      u32x4_t o;
      o.x = pack_bf16x2(bf16_lo(bb.x) + bf16_lo(bs.x), bf16_hi(bb.x) + bf16_hi(bs.x));
      o.y = pack_bf16x2(bf16_lo(bb.y) + bf16_lo(bs.y), bf16_hi(bb.y) + bf16_hi(bs.y));
      o.z = pack_bf16x2(bf16_lo(bb.z) + bf16_lo(bs.z), bf16_hi(bb.z) + bf16_hi(bs.z));
      o.w = pack_bf16x2(bf16_lo(bb.w) + bf16_lo(bs.w), bf16_hi(bb.w) + bf16_hi(bs.w));
      const bool real = n < rows && (int64_t)v < vend;
      __builtin_nontemporal_store(o, real ? (u32x4_t*)(out + ((uint32_t)n * Vu + v)) : sink);
    }
    gather_to_lds(g);  // lds_e was last read before the barrier above
    __syncthreads();
  };

  // Pairs of chunks; an odd count ends with one chunk past the last row,
  // whose stores all go to the sink.
  for (int64_t c = 0; c < nchunks; c += 2) {
    chunk(c, ring[0]);
    chunk(c + 1, ring[1]);
  }
  if (blockIdx.x == 0 && bad) atomicAdd(p.bad_rows, bad);
}

// ---------------------------------------------------------------- grouped form
// The bias is a function of the predecessor token alone (markov_head.py
// page, the Markov head's forward), so rows that share a predecessor share
// their bias.  Batches with repeated predecessors (Zipf-like token streams)
// take this form, which multiplies each distinct token once:
//
//   * plan, per workgroup in LDS: the ids go into a hash table (linear
//     probing), distinct tokens get dense ids u in table order, and a
//     counting sort lists the rows grouped by u;
//   * the sorted rows are walked in chunks of RC.  A chunk's rows need the
//     bias of at most three 16-token tiles of u; each tile is multiplied
//     once (v_mfma_f32_16x16x32_bf16, the wave's W2 slice in VGPRs) into a
//     five-tile bias ring in LDS, one chunk before the first chunk that
//     needs it, so that a wave's matrix work overlaps other waves'
//     streaming (one barrier per chunk);
//   * each thread streams 16-byte vectors of row segments: base in, the
//     bias of the row's token from the ring, corrected out.  Base vectors
//     are loaded D chunks ahead into a register ring;
//   * the last two waves load the W1 rows of new tiles straight into LDS (a
//     four-tile ring) two chunks ahead of the streaming.  A wave's memory
//     counter completes in issue order, so waiting for those rows also
//     waits for every base load the wave issued earlier: keeping the gather
//     in two waves keeps the other waves' rings full.
// Loads and stores past the edges carry out-of-range buffer offsets, so
// every memory operation is unconditional.
constexpr int kGroupedMaxRows = 4096;   // rows of one call (plan arrays in LDS)
constexpr int kGroupedHash = 8192;      // hash slots (load factor <= 1/2)
// Below this many rows the plan costs more than the repeats save (measured
// at V = 129280 with 320 rows of distinct ids), and the rows keep their
// own order.
constexpr int kGroupedMinRows = 1024;

// DEDUP: plan with the hash table (one bias per distinct token); without
// it every row is its own token id (rows in their own order), which costs
// nothing to plan and suits batches with few repeats.
// LF32: fp32 logits (the weights stay bf16); each 8-column vector of a row
// is then two 16-byte pieces, the sum is not rounded again.
template <int K32, int WAVES, int D, int KB, bool DEDUP, bool LF32>
__global__ __launch_bounds__(WAVES * 64) void markov_apply_grouped_bf16(KernelParams p) {
  constexpr int NV = LF32 ? 2 : 1;             // 16-byte pieces per 8-column vector
  constexpr uint32_t LB = LF32 ? 4u : 2u;      // bytes per logit
  constexpr int THREADS = WAVES * 64;
  constexpr int RC = 32;                       // sorted rows per chunk
  constexpr int COLS = 32 * WAVES;             // columns of the workgroup
  constexpr int VPR = COLS / 8;                // 16-byte vectors per row segment
  constexpr int VPT = RC * VPR / THREADS;      // streamed vectors per thread and chunk
  constexpr int BSTRIDE = 2 * COLS + 16;       // LDS bytes per bias row
  constexpr int IPT = kGroupedMaxRows / THREADS;
  constexpr int EBYTES = 4 * K32 * 1024;       // four gathered tiles
  constexpr int kBiasTiles = 5;                // bias ring: five 16-token tiles
  constexpr int RING_BYTES = kBiasTiles * 16 * BSTRIDE;
  constexpr int PLAN_TMP = kGroupedHash * 4 + kGroupedHash * 2 + kGroupedMaxRows * 4;
  constexpr int UNION = (EBYTES + RING_BYTES > PLAN_TMP) ? EBYTES + RING_BYTES : PLAN_TMP;
  static_assert(VPT * THREADS == RC * VPR && IPT * THREADS == kGroupedMaxRows, "thread mapping");
  static_assert(RC == 32, "a chunk spans at most three tiles and adds at most two");
  // KB: B-operand blocks read ahead in the matrix loop (D and KB fit the
  // VGPR budget: 256 per lane at 8 waves, 128 at 16)
  static_assert(K32 % KB == 0, "rank blocks");

  // Working area: the plan's temporaries, then the gathered W1 tiles and the
  // bias ring.
  __shared__ __attribute__((aligned(16))) unsigned char lds_u[UNION];
  __shared__ uint16_t plan_row[kGroupedMaxRows];   // sorted position -> row
  __shared__ uint16_t plan_uid[kGroupedMaxRows];   // sorted position -> token id u
  __shared__ int32_t plan_tok[kGroupedMaxRows + 16];  // u -> token (-1: zero bias)
  __shared__ uint32_t lds_part[WAVES];
  __shared__ uint32_t lds_part2[WAVES];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int rows = (int)p.rows;  // 1 .. kGroupedMaxRows (host)
  const uint32_t V = (uint32_t)p.V;
  const int r = (int)p.r;
  const uint32_t vbeg = blockIdx.x * (uint32_t)COLS;
  const uint32_t vend = (vbeg + COLS < V) ? vbeg + COLS : V;
  const uint32_t S = (V + 31) / 32;
  const bool has = blockIdx.x * WAVES + wave < S;
  const uint32_t lbytes = (uint32_t)rows * V * LB;  // <= 2^31 (host)
  const __amdgpu_buffer_rsrc_t rs_base = buffer_rsrc(p.base, lbytes);
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(p.out, lbytes);
  // gated head: the gathered row of row i is latent row i (rows in their own
  // order; the host never plans a gated call)
  const bool lat = p.latent != nullptr;
  const BufferWords bw_w1 = lat ? buffer_words(p.latent, (uint32_t)rows * (uint32_t)r * 2u)
                                : buffer_words(p.w1, V * (uint32_t)r * 2u);
  constexpr int GW = WAVES - 1;  // the gathering waves: GW and GW - 1

  // ids first; the W2 loads are issued in eight groups between the plan's
  // phases, so that the plan runs while they are in flight (a wave stalls
  // on issue once the memory pipeline is full).
  int64_t idv[IPT];
#pragma unroll
  for (int k = 0; k < IPT; ++k) {
    const int i = tid + k * THREADS;
    idv[k] = p.ids[i < rows ? i : rows - 1];
  }
  const __amdgpu_buffer_rsrc_t rs_w2 = buffer_rsrc(p.w2, V * (uint32_t)r * 2u);
  bf16x8_t a[2][K32];
  auto load_w2 = [&](int group) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t vrow = (blockIdx.x * WAVES + wave) * 32u + 8u * (n16 >> 2) + 4u * t + (n16 & 3);
#pragma unroll
      for (int kk = 0; kk < K32; ++kk) {
        if ((t * K32 + kk) * 8 / (2 * K32) != group) continue;
        const int kof = kk * 32 + 8 * g4;
        a[t][kk] = __builtin_bit_cast(
            bf16x8_t, buffer_load16(rs_w2, (has && vrow < V && kof < r) ? (vrow * (uint32_t)r + kof) * 2u : kBufferOob));
      }
    }
  };
  load_w2(0);

  if constexpr (DEDUP) {
    // ---- plan.  Invalid ids (outside [0, V)) become the key V, one more
    // group with a zero bias.
    uint32_t* const htab = (uint32_t*)lds_u;                                  // [kGroupedHash] key or ~0
    uint16_t* const huid = (uint16_t*)(lds_u + kGroupedHash * 4);             // [kGroupedHash] u of a slot
    uint32_t* const cnt = (uint32_t*)(lds_u + kGroupedHash * 6);              // [kGroupedMaxRows] rows of u
    for (int i = tid; i < kGroupedHash; i += THREADS) htab[i] = 0xFFFFFFFFu;
    for (int i = tid; i < kGroupedMaxRows; i += THREADS) cnt[i] = 0u;
    lds_barrier();
    load_w2(1);
    uint32_t bad = 0;
    uint32_t key[IPT], slot[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int i = tid + k * THREADS;
      const bool ok = idv[k] >= 0 && idv[k] < (int64_t)V;
      key[k] = ok ? (uint32_t)idv[k] : V;
      if (i < rows) {
        bad += ok ? 0u : 1u;
        uint32_t s = (key[k] * 0x9E3779B1u) >> (32 - 13);
        // at most rows < kGroupedHash keys: an empty slot always exists
        for (int probe = 0; probe < kGroupedHash; ++probe) {
          const uint32_t old = atomicCAS(&htab[s], 0xFFFFFFFFu, key[k]);
          if (old == 0xFFFFFFFFu || old == key[k]) break;
          s = (s + 1) & (kGroupedHash - 1);
        }
        slot[k] = s;
      }
    }
    if (blockIdx.x == 0 && bad) atomicAdd(p.bad_rows, bad);
    lds_barrier();
    load_w2(2);
    // Dense ids u in slot order.  Wave w owns slots [w SPW, (w + 1) SPW),
    // read 64 consecutive slots at a time (no bank conflicts); the ballot of
    // the occupied ones ranks them.
    constexpr int SPW = kGroupedHash / WAVES;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes under this one
    {
      uint32_t cw = 0;
#pragma unroll
      for (int j = 0; j < SPW / 64; ++j)
        cw += (uint32_t)__builtin_popcountll(__ballot(htab[wave * SPW + j * 64 + lane] != 0xFFFFFFFFu));
      if (lane == 0) lds_part[wave] = cw;
    }
    lds_barrier();
    load_w2(3);
    uint32_t U = 0, run = 0;
    for (int w = 0; w < WAVES; ++w) {
      const uint32_t pw = lds_part[w];
      run += w < wave ? pw : 0u;
      U += pw;
    }
    U = __builtin_amdgcn_readfirstlane(U);
    uint32_t hk[SPW / 64];
#pragma unroll
    for (int j = 0; j < SPW / 64; ++j) hk[j] = htab[wave * SPW + j * 64 + lane];
#pragma unroll
    for (int j = 0; j < SPW / 64; ++j) {
      const int sl = wave * SPW + j * 64 + lane;
      const uint32_t kk = hk[j];
      const uint64_t m = __ballot(kk != 0xFFFFFFFFu);
      if (kk != 0xFFFFFFFFu) {
        const uint32_t u = run + (uint32_t)__builtin_popcountll(m & below);
        huid[sl] = (uint16_t)u;
        plan_tok[u] = kk < V ? (int32_t)kk : -1;
      }
      run += (uint32_t)__builtin_popcountll(m);
    }
    if (tid < 16) plan_tok[U + tid] = -1;  // the last tile's padding
    lds_barrier();
    load_w2(4);
    // counting sort of the rows by u
    uint32_t ru[IPT];
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int i = tid + k * THREADS;
      if (i < rows) {
        ru[k] = huid[slot[k]];
        atomicAdd(&cnt[ru[k]], 1u);
      }
    }
    lds_barrier();
    load_w2(5);
    // exclusive scan of cnt[0 .. kGroupedMaxRows) in place, wave w owning
    // [w CPW, (w + 1) CPW) in runs of 64
    constexpr int CPW = kGroupedMaxRows / WAVES;
    {
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < CPW / 64; ++j) tot += cnt[wave * CPW + j * 64 + lane];
      tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_sum_u32(tot), 63);
      if (lane == 0) lds_part2[wave] = tot;
    }
    lds_barrier();
    load_w2(6);
    {
      uint32_t base = 0;
      for (int w = 0; w < wave; ++w) base += lds_part2[w];
      uint32_t v[CPW / 64];
#pragma unroll
      for (int j = 0; j < CPW / 64; ++j) v[j] = cnt[wave * CPW + j * 64 + lane];
#pragma unroll
      for (int j = 0; j < CPW / 64; ++j) {
        const uint32_t incl = wave_inclusive_sum_u32(v[j]);
        cnt[wave * CPW + j * 64 + lane] = base + incl - v[j];
        base += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      }
    }
    lds_barrier();
    load_w2(7);
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int i = tid + k * THREADS;
      if (i < rows) {
        const uint32_t pos = atomicAdd(&cnt[ru[k]], 1u);
        plan_row[pos] = (uint16_t)i;
        plan_uid[pos] = (uint16_t)ru[k];
      }
    }
    lds_barrier();
  } else {
#pragma unroll
    for (int g = 1; g < 8; ++g) load_w2(g);
    uint32_t bad = 0;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int i = tid + k * THREADS;
      if (i < rows) {
        const bool ok = idv[k] >= 0 && idv[k] < (int64_t)V;
        bad += ok ? 0u : 1u;
        plan_row[i] = (uint16_t)i;
        plan_uid[i] = (uint16_t)i;
        plan_tok[i] = ok ? (lat ? i : (int32_t)idv[k]) : -1;
      }
    }
    if (blockIdx.x == 0 && bad) atomicAdd(p.bad_rows, bad);
    if (tid < 16) plan_tok[rows + tid] = -1;  // the last tile's padding
    lds_barrier();
  }

  // ---- chunk loop over the sorted rows
  // Gathered tile t (slot t % 4): block kk holds at lane l's 16 bytes the
  // W1 row of token 16 t + l % 16, rank elements 32 kk + 8 (l / 16) .. +7
  // (the B operand of the matrix instruction).
  unsigned char* const lds_e = lds_u;             // [4 tiles][K32 blocks][1024]
  unsigned char* const lds_b = lds_u + EBYTES;    // [5 tiles x 16 tokens][BSTRIDE]
  const int nch = (rows + RC - 1) / RC;
  // last tile chunk c needs (chunks past the end: the last one)
  auto last_tile = [&](int c) __attribute__((always_inline)) -> int {
    const int pos = RC * c + RC - 1;
    return __builtin_amdgcn_readfirstlane((int)plan_uid[pos < rows ? pos : rows - 1] >> 4);
  };
  // stream vector q of the thread: sorted position RC c + prow(q), vector vi
  const int vi = tid % VPR;
  const uint32_t col = vbeg + 8u * (uint32_t)vi;
  const bool col_ok = col < vend;
  auto prow = [&](int q) __attribute__((always_inline)) { return (tid + q * THREADS) / VPR; };
  auto base_off = [&](int pos) __attribute__((always_inline)) -> uint32_t {
    return (pos < rows && col_ok) ? ((uint32_t)plan_row[pos] * V + col) * LB : kBufferOob;
  };
  // waves GW and GW - 1: W1 rows of tiles t0 .. t0 + nn - 1 into their LDS
  // slots, the even rank blocks by GW and the odd ones by GW - 1
  const int gpar = wave == GW ? 0 : 1;
  auto gather = [&](int t0, int nn) __attribute__((always_inline)) {
    for (int j = 0; j < nn; ++j) {
      const int t = t0 + j;
      const int x = plan_tok[16 * t + n16];
#pragma unroll
      for (int kk = 0; kk < K32; ++kk) {
        if ((kk & 1) != gpar) continue;
        const int kof = 32 * kk + 8 * g4;
        load_lds16(bw_w1, (x >= 0 && kof < r) ? ((uint32_t)x * (uint32_t)r + kof) * 2u : kBufferOob,
                   lds_address(lds_e + ((t & 3) * K32 + kk) * 1024));
      }
    }
  };

  // The ring is filled in the loop's own pattern of a store and a load per
  // vector (the stores here land past the buffer and are dropped), so the
  // compiler's count of the operations after each ring load is the loop's.
  u32x4_t ring[D][VPT][NV];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
#pragma unroll
      for (int h = 0; h < NV; ++h)
        buffer_store16(rs_out, kBufferOob + 16u * (uint32_t)((d * VPT + q) * NV + h), u32x4_t{0u, 0u, 0u, 0u});
      const uint32_t off = base_off(RC * d + prow(q));
#pragma unroll
      for (int h = 0; h < NV; ++h) ring[d][q][h] = buffer_load16(rs_base, off + 16u * h);
    }
  // W2 is complete before the chunk loop (the ring stays in flight), so that
  // no wait inside the loop is held back by it.
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) __asm__ volatile("" ::"v"(a[t][kk]));
  // bias of tiles t0 .. t1 (gathered rows in their slots) into the ring
  auto multiply = [&](int t0, int t1) __attribute__((always_inline)) {
    if (!has) return;
    for (int t = t0; t <= t1; ++t) {
      f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
      const unsigned char* eb = lds_e + (t & 3) * K32 * 1024 + lane * 16;
      // B operands read KB blocks at a time, so one LDS round trip serves
      // 2 KB matrix instructions
#pragma unroll
      for (int k0 = 0; k0 < K32; k0 += KB) {
        bf16x8_t bop[KB];
#pragma unroll
        for (int i = 0; i < KB; ++i) bop[i] = *(const bf16x8_t*)(eb + (k0 + i) * 1024);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
        for (int i = 0; i < KB; ++i) {
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][k0 + i], bop[i], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][k0 + i], bop[i], acc1, 0, 0, 0);
        }
      }
      u32x4_t w;
      w.x = pack_bf16x2(acc0[0], acc0[1]);
      w.y = pack_bf16x2(acc0[2], acc0[3]);
      w.z = pack_bf16x2(acc1[0], acc1[1]);
      w.w = pack_bf16x2(acc1[2], acc1[3]);
      *(u32x4_t*)(lds_b + (16 * (t % kBiasTiles) + n16) * BSTRIDE + (wave * 32 + 8 * g4) * 2) = w;
    }
  };

  // Prologue: the W1 rows of chunks 0 and 1 (tiles 0 .. 3 at most), then
  // chunk 0's bias.
  if (wave >= GW - 1) {
    gather(0, last_tile(1) + 1);
    wait_vmcnt<0>();
  }
  lds_barrier();
  int lt_done = last_tile(0);  // tiles whose bias is in the ring (or being written)
  multiply(0, lt_done);
  lds_barrier();

  // Chunk c: gather for chunk c + 2, bias of chunk c + 1's new tiles, then
  // stream chunk c (its bias was written a chunk ago).  One barrier.  Live
  // tiles: gathered slots lt(c)+1 .. lt(c+2) (at most four), bias tiles
  // lt(c)-2 .. lt(c+1) (at most five).
  auto chunk = [&](int c, u32x4_t pre[VPT][NV]) __attribute__((always_inline)) {
    const int l1 = last_tile(c + 1);
    if (wave >= GW - 1) gather(l1 + 1, last_tile(c + 2) - l1);
    multiply(lt_done + 1, l1);
    lt_done = l1;

    // stream the chunk; the register slot is refilled with chunk c + D
#pragma unroll
    for (int q = 0; q < VPT; ++q) {
      const int pos = RC * c + prow(q);
      const int pc = pos < rows ? pos : rows - 1;
      const uint32_t row = plan_row[pc];
      const uint32_t u = plan_uid[pc];
      const u32x4_t bs = *(const u32x4_t*)(lds_b + (16u * ((u >> 4) % kBiasTiles) + (u & 15u)) * BSTRIDE + vi * 16);
      const uint32_t ooff = (pos < rows && col_ok) ? (row * V + col) * LB : kBufferOob;
      if constexpr (LF32) {
        // fp32 logits: the bf16 bias widened exactly, one fp32 add
        const u32x4_t b0 = pre[q][0], b1 = pre[q][1];
        const float bias[8] = {bf16_lo(bs.x), bf16_hi(bs.x), bf16_lo(bs.y), bf16_hi(bs.y),
                               bf16_lo(bs.z), bf16_hi(bs.z), bf16_lo(bs.w), bf16_hi(bs.w)};
        const u32x4_t o0 = u32x4_t{__float_as_uint(__uint_as_float(b0.x) + bias[0]), __float_as_uint(__uint_as_float(b0.y) + bias[1]),
                                   __float_as_uint(__uint_as_float(b0.z) + bias[2]), __float_as_uint(__uint_as_float(b0.w) + bias[3])};
        const u32x4_t o1 = u32x4_t{__float_as_uint(__uint_as_float(b1.x) + bias[4]), __float_as_uint(__uint_as_float(b1.y) + bias[5]),
                                   __float_as_uint(__uint_as_float(b1.z) + bias[6]), __float_as_uint(__uint_as_float(b1.w) + bias[7])};
        buffer_store16(rs_out, ooff, o0);
        buffer_store16(rs_out, ooff + 16u, o1);
      } else {
        const u32x4_t bb = pre[q][0];
        u32x4_t o;
        o.x = pack_bf16x2(bf16_lo(bb.x) + bf16_lo(bs.x), bf16_hi(bb.x) + bf16_hi(bs.x));
        o.y = pack_bf16x2(bf16_lo(bb.y) + bf16_lo(bs.y), bf16_hi(bb.y) + bf16_hi(bs.y));
        o.z = pack_bf16x2(bf16_lo(bb.z) + bf16_lo(bs.z), bf16_hi(bb.z) + bf16_hi(bs.z));
        o.w = pack_bf16x2(bf16_lo(bb.w) + bf16_lo(bs.w), bf16_hi(bb.w) + bf16_hi(bs.w));
        buffer_store16(rs_out, ooff, o);
      }
      // refilled after its last use, so the new value can take its registers
      const uint32_t noff = base_off(pos + RC * D);
#pragma unroll
      for (int h = 0; h < NV; ++h) pre[q][h] = buffer_load16(rs_base, noff + 16u * h);
    }
    // the gathered rows are in LDS before the barrier (the stream's loads
    // and stores issued after them may stay in flight)
    if (wave >= GW - 1) wait_vmcnt<2 * NV * VPT>();
    lds_barrier();
  };

  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) chunk(c0 + s, ring[s]);
  }
}

// ---------------------------------------------------------------- launcher
namespace {
template <int K32, int WAVES, int RC>
hipError_t launch_wide(const KernelParams& p, hipStream_t s) {
  const int64_t S = (p.V + 31) / 32;
  const dim3 grid((unsigned)((S + WAVES - 1) / WAVES));
  hipLaunchKernelGGL((markov_apply_wide_bf16<K32, WAVES, RC>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}

template <int K32, int WAVES, int D, int KB, bool LF32>
hipError_t launch_grouped(const KernelParams& p, hipStream_t s) {
  const int64_t S = (p.V + 31) / 32;
  const dim3 grid((unsigned)((S + WAVES - 1) / WAVES));
  if (p.rows >= kGroupedMinRows && p.latent == nullptr)
    hipLaunchKernelGGL((markov_apply_grouped_bf16<K32, WAVES, D, KB, true, LF32>), grid, dim3(WAVES * 64), 0, s, p);
  else
    hipLaunchKernelGGL((markov_apply_grouped_bf16<K32, WAVES, D, KB, false, LF32>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}
}  // namespace

// Grouped teacher-forced apply (bf16 weights; bf16 or fp32 logits):
// 1 <= rows <= kGroupedMaxRows (the plan deduplicates from kGroupedMinRows
// rows), the logits and V * r * 2 at most 2^31 bytes; hipErrorNotSupported
// otherwise.
hipError_t launch_apply_grouped(const KernelParams& p, bool logits_f32, hipStream_t s) {
  static_assert(kGroupedMaxRows == kGroupedApplyMaxRows, "row limit");
  if (p.rows < 1 || p.rows > kGroupedMaxRows) return hipErrorNotSupported;
  if (p.latent != nullptr && p.latent_ld != p.r) return hipErrorNotSupported;
  if (p.rows * p.V * (logits_f32 ? 4 : 2) > ((int64_t)1 << 31) || p.V * p.r * 2 > ((int64_t)1 << 31))
    return hipErrorNotSupported;
  // fp32 logits take twice the ring registers per chunk: half the depth
  if (logits_f32) {
    switch (tile_ks_for_rank(p.r)) {
      case 1:
      case 2: return launch_grouped<1, 16, 2, 1, true>(p, s);
      case 4: return launch_grouped<2, 16, 2, 2, true>(p, s);
      case 8: return launch_grouped<4, 16, 2, 2, true>(p, s);
      case 16: return launch_grouped<8, 16, 1, 4, true>(p, s);
      case 24: return launch_grouped<12, 8, 2, 4, true>(p, s);
      case 32: return launch_grouped<16, 8, 2, 8, true>(p, s);
      default: return hipErrorNotSupported;
    }
  }
  switch (tile_ks_for_rank(p.r)) {
    case 1:
    case 2: return launch_grouped<1, 16, 4, 1, false>(p, s);
    case 4: return launch_grouped<2, 16, 4, 2, false>(p, s);
    case 8: return launch_grouped<4, 16, 4, 2, false>(p, s);
    case 16: return launch_grouped<8, 16, 2, 4, false>(p, s);
    case 24: return launch_grouped<12, 8, 4, 4, false>(p, s);
    case 32: return launch_grouped<16, 8, 4, 8, false>(p, s);
    default: return hipErrorNotSupported;
  }
}

size_t apply_sink_bytes() { return 1024 * 16; }

// Teacher-forced bf16 apply with the streaming kernel; hipErrorNotSupported
// if the rank has no instance or the element offsets need more than 31 bits.
hipError_t launch_apply_wide(const KernelParams& p, hipStream_t s) {
  if (p.latent != nullptr) return hipErrorNotSupported;  // vanilla head only
  if (p.rows * p.V >= ((int64_t)1 << 31)) return hipErrorNotSupported;
  // rank blocks of 32 (the rank is zero-padded to a multiple of 32)
  switch (tile_ks_for_rank(p.r)) {
    case 1:
    case 2: return launch_wide<1, 16, 32>(p, s);
    case 4: return launch_wide<2, 16, 32>(p, s);
    case 8: return launch_wide<4, 16, 32>(p, s);
    case 16: return launch_wide<8, 16, 32>(p, s);
    case 24: return launch_wide<12, 8, 32>(p, s);
    case 32: return launch_wide<16, 8, 32>(p, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace dspark
