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
  const int m = lane & 31;
  const int h = lane >> 5;
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

// ---------------------------------------------------------------- launcher
namespace {
template <int K32, int WAVES, int RC>
hipError_t launch_wide(const KernelParams& p, hipStream_t s) {
  const int64_t S = (p.V + 31) / 32;
  const dim3 grid((unsigned)((S + WAVES - 1) / WAVES));
  hipLaunchKernelGGL((markov_apply_wide_bf16<K32, WAVES, RC>), grid, dim3(WAVES * 64), 0, s, p);
  return hipGetLastError();
}
}  // namespace

size_t apply_sink_bytes() { return 1024 * 16; }

// Teacher-forced bf16 apply with the streaming kernel; hipErrorNotSupported
// if the rank has no instance or the element offsets need more than 31 bits.
hipError_t launch_apply_wide(const KernelParams& p, hipStream_t s) {
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
