// markov_step.hip -- one sampling step of sample_block_tokens (gfx950).
//
// A step draws the token of position k for every batch row b from the
// corrected logits c = base[b, k, :] + bias(x), x = first_prev[b] (k = 0) or
// the token drawn at k - 1 (third-party markov_head.py page, the sampling
// loop).  Greedy takes the first argmax of c; temperature sampling takes the
// first argmax of fmaf(c, log2(e) / T, g) with g base-2 Gumbel noise from
// Philox4x32-10 of (v / 4, k_abs, b_abs, 0) under the seed.  This kernel
// computes the per-(row, column block) argmax keys of one step; a second
// kernel reduces them to the tokens.
//
// Layout of the work:
//   * the vocabulary is cut into blocks of 512 columns (16 waves x 32) and
//     the rows into chunks of 32 (16 for fp32 logits, whose 8 columns per
//     lane take two 16-byte vectors); a unit is one (block, chunk).  The grid
//     has one workgroup per CU and workgroup g takes the units
//     [g U / G, (g + 1) U / G) in block-major order, so every CU gets the
//     same number of units (a grid of whole blocks would leave most CUs idle
//     in a second, short round);
//   * each wave keeps the W2w rows of its 32 columns of the current block in
//     VGPRs and reloads them when the block changes (at most a few times per
//     workgroup); the loads are issued a unit ahead of their use;
//   * unit u: the bias of unit u + 1 is multiplied on the matrix cores
//     (v_mfma_f32_16x16x32_bf16, gathered W1 rows from LDS as the B operand),
//     one 16-row tile after each of the wave's two selected vectors of unit
//     u, so matrix and vector work overlap; one barrier per unit;
//   * the selection streams the base logits of the unit (loaded a unit
//     ahead), adds the bias, keeps each thread's best score in fp32 and
//     reduces each row's 64 lanes to one key;
//   * every thread gathers 16 bytes of W1 rows for unit u + 2 with a plain
//     load issued before the unit's base loads: a wave's memory counter
//     completes in issue order, so waiting for the gather leaves the base
//     loads in flight.
// Loads and stores past the edges carry out-of-range buffer offsets, so
// every memory operation is unconditional.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {
constexpr int kStepWaves = 16;
constexpr int kStepThreads = kStepWaves * 64;
constexpr int kStepCols = 32 * kStepWaves;  // columns of a block
constexpr int kStepMaxB = 4096;             // rows of a call (tokens staged in LDS)
}  // namespace

// RD: units of base logits in flight (register ring depth; 1 where the
// selection's registers leave no room for two).  LF32: fp32 logits (the
// bias is still the bf16 Linear output, widened exactly and added in fp32).
template <int K32, int MODE, int RD, bool LF32>
__global__ __launch_bounds__(kStepThreads) void markov_step_bf16(KernelParams p) {
  constexpr int kStepRows = LF32 ? 16 : 32;               // rows of a chunk (MFMA N tiles of 16)
  constexpr int TILES = kStepRows / 16;
  constexpr int NV = LF32 ? 2 : 1;                        // 16-byte vectors per lane's 8 columns
  constexpr uint32_t LB = LF32 ? 4u : 2u;                 // bytes per logit
  constexpr int VPR = kStepCols / 8;                      // lanes of a row segment (64)
  constexpr int VPT = kStepRows * VPR / kStepThreads;     // row segments per thread and unit (2; 1 for fp32)
  constexpr int BSTRIDE = 2 * kStepCols + 16;             // LDS bytes per bias row
  constexpr int EUNIT = TILES * K32 * 1024;               // gathered W1 rows of a unit
  constexpr int GPT = EUNIT / 16 / kStepThreads > 0 ? EUNIT / 16 / kStepThreads : 1;  // gathered vectors per thread
  static_assert(VPT * NV == 2 && VPR == 64, "one wave per row segment, two vectors per thread");
  static_assert(GPT * kStepThreads * 16 >= EUNIT, "gather mapping");

  // Gathered rows of units u (slot u % 2): tile t, block kk holds at lane l's
  // 16 bytes the W1 row of row 16 t + l % 16 of the chunk, rank elements
  // 32 kk + 8 (l / 16) .. +7 (the matrix instruction's B operand).
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[2][EUNIT];
  // Bias of units (slot u % 2), row-major: [32 rows][512 columns] bf16.
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[2][kStepRows * BSTRIDE];
  __shared__ int32_t lds_tok[kStepMaxB];  // predecessor of each row (-1: zero bias)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int B = (int)p.rows;
  const uint32_t V = (uint32_t)p.V, M = (uint32_t)p.M, kstep = (uint32_t)p.k;
  const int r = (int)p.r;
  const int nch = (B + kStepRows - 1) / kStepRows;
  const int nblk = (int)((V + kStepCols - 1) / kStepCols);
  const int units = nch * nblk;
  const int u0 = (int)(((int64_t)blockIdx.x * units) / gridDim.x);
  const int u1 = (int)(((int64_t)(blockIdx.x + 1) * units) / gridDim.x);

  const uint32_t lbytes = (uint32_t)B * M * V * LB;  // <= 2^31 (host)
  const __amdgpu_buffer_rsrc_t rs_base = buffer_rsrc(p.base, lbytes);
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(p.out, p.out != nullptr ? lbytes : 0u);
  const __amdgpu_buffer_rsrc_t rs_part = buffer_rsrc(p.partials, (uint32_t)B * (uint32_t)p.nparts * 8u);
  // gated head: the gathered row of batch row b is latent row b
  const bool lat = p.latent != nullptr;
  const uint32_t eld = lat ? (uint32_t)p.latent_ld : (uint32_t)r;
  const __amdgpu_buffer_rsrc_t rs_w1 =
      lat ? buffer_rsrc(p.latent, ((uint32_t)(B - 1) * eld + (uint32_t)r) * 2u) : buffer_rsrc(p.w1, V * (uint32_t)r * 2u);
  const __amdgpu_buffer_rsrc_t rs_w2 = buffer_rsrc(p.w2, V * (uint32_t)r * 2u);

  // unit u = block * nch + chunk
  auto ublk = [&](int u) __attribute__((always_inline)) { return u / nch; };
  auto uchk = [&](int u) __attribute__((always_inline)) { return u - (u / nch) * nch; };

  // ---- predecessors of all rows (loads issued first; written to LDS once
  // the W2 loads below are in flight)
  constexpr int TPT = kStepMaxB / kStepThreads;
  int64_t tokv[TPT];
#pragma unroll
  for (int k = 0; k < TPT; ++k) {
    const uint32_t i = (uint32_t)(tid + k * kStepThreads < B ? tid + k * kStepThreads : B - 1);
    tokv[k] = kstep == 0 ? p.ids[i] : p.tokens[i * M + kstep - 1];
  }

  // ---- W2w rows of the wave's 32 columns of block j (A operands: columns
  // on M, rows on N, rank on K; col(t, m) = 8 (m / 4) + 4 t + m % 4 gives a
  // lane's 4 + 4 accumulators the 8 consecutive columns 8 g4 .. 8 g4 + 7)
  bf16x8_t a[2][K32];
  auto load_w2 = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t vrow = (uint32_t)j * kStepCols + wave * 32u + 8u * (n16 >> 2) + 4u * t + (n16 & 3);
#pragma unroll
      for (int kk = 0; kk < K32; ++kk) {
        const int kof = kk * 32 + 8 * g4;
        // default cache policy: W2 is read again by the next step's launch
        a[t][kk] = __builtin_bit_cast(
            bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                          rs_w2, (vrow < V && kof < r) ? (vrow * (uint32_t)r + kof) * 2u : kBufferOob, 0, 0));
      }
    }
  };

  // ---- gather of unit u's W1 rows into registers: 16-byte piece e = tid +
  // q * threads is tile e / (64 K32), rank block (e / 64) % K32 and B-operand
  // lane e % 64, stored at byte 16 e of the unit's slot (the layout above).
  auto gather = [&](int u, u32x4_t gv[GPT]) __attribute__((always_inline)) {
    const int c = uchk(u);
    const bool live = u < u1;
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int e = tid + q * kStepThreads;   // 16-byte piece of the unit
      const int t = e / (K32 * 64);           // tile
      const int kk = (e / 64) % K32;          // rank block
      const int l = e % 64;                   // lane of the B operand
      const int row = c * kStepRows + 16 * t + (l & 15);
      const int kof = 32 * kk + 8 * (l >> 4);
      const int x = (live && e < EUNIT / 16 && row < B) ? lds_tok[row] : -1;
      gv[q] = __builtin_amdgcn_raw_buffer_load_b128(
          rs_w1, (x >= 0 && kof < r) ? ((uint32_t)x * eld + kof) * 2u : kBufferOob, 0, 0);
    }
  };
  auto gather_to_lds = [&](int slot, const u32x4_t gv[GPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < GPT; ++q) {
      const int e = tid + q * kStepThreads;
      if (e < EUNIT / 16) *(u32x4_t*)&lds_e[slot][e * 16] = gv[q];
    }
  };

  // ---- bias of tile t of unit u (its gathered rows in slot u % 2) into
  // bias slot u % 2 (tiles past the chunk's TILES do nothing)
  auto multiply = [&](int u, int t) __attribute__((always_inline)) {
    if (u >= u1 || t >= TILES) return;
    const int slot = u & 1;
    const bool has = (uint32_t)ublk(u) * kStepCols + wave * 32u < V;
    if (!has) return;
    f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
    const unsigned char* eb = &lds_e[slot][t * K32 * 1024 + lane * 16];
#pragma unroll
    for (int kk = 0; kk < K32; ++kk) {
      const bf16x8_t bop = *(const bf16x8_t*)(eb + kk * 1024);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][kk], bop, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][kk], bop, acc1, 0, 0, 0);
    }
    u32x4_t w;  // the bias in the weight dtype (the Linear's bf16 output)
    w.x = pack_bf16x2(acc0[0], acc0[1]);
    w.y = pack_bf16x2(acc0[2], acc0[3]);
    w.z = pack_bf16x2(acc1[0], acc1[1]);
    w.w = pack_bf16x2(acc1[2], acc1[3]);
    *(u32x4_t*)&lds_b[slot][(16 * t + n16) * BSTRIDE + (wave * 32 + 8 * g4) * 2] = w;
  };

  // ---- streamed row segment q of a unit: row 16 q + wave of the chunk
  // (wave w owns rows w and w + 16), the lane's 8 columns 8 lane .. +7 of
  // the block, 16-byte vector h of them
  auto base_off = [&](int u, int q, int h) __attribute__((always_inline)) -> uint32_t {
    const uint32_t row = (uint32_t)(uchk(u) * kStepRows + 16 * q + wave);
    const uint32_t col = (uint32_t)ublk(u) * kStepCols + 8u * lane;
    return (u < u1 && row < (uint32_t)B && col < V) ? ((row * M + kstep) * V + col) * LB + 16u * (uint32_t)h
                                                      : kBufferOob;
  };

  // ---- selection of vector q of unit u from its base vectors pre[]
  // (refilled with unit u + RD after their last use): corrected values to
  // the output, the row's best key to the partials
  auto select_unit = [&](int u, u32x4_t pre[VPT][NV], int q) __attribute__((always_inline)) {
    const int slot = u & 1;
    const uint32_t colw = (uint32_t)ublk(u) * kStepCols + 8u * lane;
    {
      const int rr = 16 * q + wave;  // row within the chunk
      const uint32_t row = (uint32_t)(uchk(u) * kStepRows + rr);
      const bool ok = u < u1 && row < (uint32_t)B && colw < V;
      const u32x4_t bs = *(const u32x4_t*)&lds_b[slot][rr * BSTRIDE + lane * 16];
      const uint32_t out_off = ok ? ((row * M + kstep) * V + colw) * LB : kBufferOob;
      // corrected values of the lane's 8 columns: bf16 logits round the fp32
      // sum to bf16; fp32 logits keep it (the bias is exact in fp32)
      float cv[8];
      if constexpr (LF32) {
        const u32x4_t b0 = pre[q][0], b1 = pre[q][1];
        const uint32_t bw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
        const uint32_t sw[4] = {bs.x, bs.y, bs.z, bs.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          cv[i] = __uint_as_float(bw[i]) + ((i & 1) ? bf16_hi(sw[i >> 1]) : bf16_lo(sw[i >> 1]));
        buffer_store16(rs_out, out_off, u32x4_t{__float_as_uint(cv[0]), __float_as_uint(cv[1]),
                                                __float_as_uint(cv[2]), __float_as_uint(cv[3])});
        buffer_store16(rs_out, ok ? out_off + 16u : kBufferOob,
                       u32x4_t{__float_as_uint(cv[4]), __float_as_uint(cv[5]), __float_as_uint(cv[6]),
                               __float_as_uint(cv[7])});
      } else {
        const u32x4_t bb = pre[q][0];
        u32x4_t o;
        o.x = pack_bf16x2(bf16_lo(bb.x) + bf16_lo(bs.x), bf16_hi(bb.x) + bf16_hi(bs.x));
        o.y = pack_bf16x2(bf16_lo(bb.y) + bf16_lo(bs.y), bf16_hi(bb.y) + bf16_hi(bs.y));
        o.z = pack_bf16x2(bf16_lo(bb.z) + bf16_lo(bs.z), bf16_hi(bb.z) + bf16_hi(bs.z));
        o.w = pack_bf16x2(bf16_lo(bb.w) + bf16_lo(bs.w), bf16_hi(bb.w) + bf16_hi(bs.w));
        buffer_store16(rs_out, out_off, o);
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) cv[i] = (i & 1) ? bf16_hi(ow[i >> 1]) : bf16_lo(ow[i >> 1]);
      }
      // the thread's best score of its 8 columns (first column on ties)
      float best = 0.0f, sumc = 0.0f;
      uint32_t bi = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float sc[4] = {cv[4 * j], cv[4 * j + 1], cv[4 * j + 2], cv[4 * j + 3]};
        sumc += (sc[0] + sc[1]) + (sc[2] + sc[3]);
        if constexpr (MODE == MODE_TEMPERATURE) {
          // columns colw + 4 j .. + 3 are the words of one Philox block
          const Philox4 q4 = philox4x32_10((colw >> 2) + (uint32_t)j, p.k_abs, (uint32_t)p.batch_offset + row, 0u,
                                           p.seed_lo, p.seed_hi);
          sc[0] = __builtin_fmaf(sc[0], p.kappa, gumbel2_from_word(q4.x0));
          sc[1] = __builtin_fmaf(sc[1], p.kappa, gumbel2_from_word(q4.x1));
          sc[2] = __builtin_fmaf(sc[2], p.kappa, gumbel2_from_word(q4.x2));
          sc[3] = __builtin_fmaf(sc[3], p.kappa, gumbel2_from_word(q4.x3));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool gt = (j == 0 && i == 0) || sc[i] > best;
          best = gt ? sc[i] : best;
          bi = gt ? (uint32_t)(4 * j + i) : bi;
        }
      }
      uint64_t key = argmax_key(best, colw + bi);
      if (sumc != sumc) {
        // A score is NaN exactly when its corrected value is (the noise is
        // finite): the first NaN wins, as a NaN's key ranks above all.
        // Without one (+inf met -inf in the sum) the scan above stands.
        uint32_t first = 8;
#pragma unroll
        for (int i = 7; i >= 0; --i)
          if (cv[i] != cv[i]) first = (uint32_t)i;
        if (first < 8) key = (0xFFFFFFFFull << 32) | (uint64_t)(0xFFFFFFFFu - (colw + first));
      }
      key = ok ? key : 0ull;
      key = wave_max_u64_lane63(key);  // the row's 64 lanes, in lane 63
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      __builtin_amdgcn_raw_buffer_store_b64(
          u32x2_t{(uint32_t)key, (uint32_t)(key >> 32)}, rs_part,
          (row < (uint32_t)B && u < u1 && lane == 63) ? (row * (uint32_t)p.nparts + (uint32_t)ublk(u)) * 8u
                                                        : kBufferOob,
          0, 0);
      // refilled after its last use, so the new value can take its registers
#pragma unroll
      for (int h = 0; h < NV; ++h) pre[q][h] = buffer_load16(rs_base, base_off(u + RD, q, h));
    }
  };

  // ---- prologue: W2 of the first block and the base of units u0 .. u0 +
  // RD - 1 in flight while the predecessors go to LDS and the rows of units
  // u0 and u0 + 1 are gathered; then the bias of unit u0
  load_w2(ublk(u0));
  u32x4_t ring[RD][VPT][NV];
#pragma unroll
  for (int d = 0; d < RD; ++d)
#pragma unroll
    for (int q = 0; q < VPT; ++q)
#pragma unroll
      for (int h = 0; h < NV; ++h) ring[d][q][h] = buffer_load16(rs_base, base_off(u0 + d, q, h));
  {
    uint32_t bad = 0;  // bad ids, counted at step 0
#pragma unroll
    for (int k = 0; k < TPT; ++k) {
      const int i = tid + k * kStepThreads;
      const bool ok = tokv[k] >= 0 && tokv[k] < (int64_t)V;
      if (i < B) {
        bad += ok ? 0u : 1u;
        lds_tok[i] = ok ? (lat ? i : (int32_t)tokv[k]) : -1;
      }
    }
    if (blockIdx.x == 0 && kstep == 0 && bad) atomicAdd(p.bad_rows, bad);
  }
  lds_barrier();
  u32x4_t gv[GPT], gv1[GPT];
  gather(u0, gv);
  gather(u0 + 1, gv1);
  gather_to_lds(u0 & 1, gv);
  gather_to_lds((u0 + 1) & 1, gv1);
  lds_barrier();
  multiply(u0, 0);
  multiply(u0, 1);
  lds_barrier();

  // ---- unit u: W2 of unit u + 1's block if new (in flight during the
  // selection), the rows of unit u + 2, the selection of unit u, the bias
  // of unit u + 1, then the rows of unit u + 2 into unit u's slot
  auto step = [&](int u, u32x4_t pre[VPT][NV]) __attribute__((always_inline)) {
    if (u + 1 < u1 && ublk(u + 1) != ublk(u)) load_w2(ublk(u + 1));
    gather(u + 2, gv);
    // each bias tile of unit u + 1 follows one selected row segment of unit
    // u, so the matrix instructions run behind the wave's own vector work
    select_unit(u, pre, 0);
    multiply(u + 1, 0);
    if constexpr (VPT > 1) select_unit(u, pre, 1);
    multiply(u + 1, 1);
    gather_to_lds(u & 1, gv);
    lds_barrier();
  };
  // RD units per iteration (register slots fixed at compile time); the last
  // iteration may run units past the range, which touch no memory
  for (int u = u0; u < u1; u += RD) {
#pragma unroll
    for (int d = 0; d < RD; ++d) step(u + d, ring[d]);
  }
}

namespace {
template <int K32, int MODE, bool LF32>
hipError_t launch_step_k(const KernelParams& p, int grid, hipStream_t s) {
  constexpr int RD = (MODE == MODE_TEMPERATURE && K32 >= 8) ? 1 : 2;
  hipLaunchKernelGGL((markov_step_bf16<K32, MODE, RD, LF32>), dim3(grid), dim3(kStepThreads), 0, s, p);
  return hipGetLastError();
}

template <bool LF32>
hipError_t launch_step_l(const KernelParams& p, int grid, hipStream_t s) {
  const bool t = p.mode == MODE_TEMPERATURE;
  switch (tile_ks_for_rank(p.r)) {  // rank blocks of 16 -> blocks of 32 (zero-padded)
    case 1:
    case 2: return t ? launch_step_k<1, MODE_TEMPERATURE, LF32>(p, grid, s) : launch_step_k<1, MODE_GREEDY, LF32>(p, grid, s);
    case 4: return t ? launch_step_k<2, MODE_TEMPERATURE, LF32>(p, grid, s) : launch_step_k<2, MODE_GREEDY, LF32>(p, grid, s);
    case 8: return t ? launch_step_k<4, MODE_TEMPERATURE, LF32>(p, grid, s) : launch_step_k<4, MODE_GREEDY, LF32>(p, grid, s);
    case 16: return t ? launch_step_k<8, MODE_TEMPERATURE, LF32>(p, grid, s) : launch_step_k<8, MODE_GREEDY, LF32>(p, grid, s);
    default: return hipErrorNotSupported;
  }
}
}  // namespace

int64_t sample_step_parts(int64_t V) { return (V + kStepCols - 1) / kStepCols; }

// One sampling step with bf16 weights and bf16 (logits_f32 false) or fp32
// logits; hipErrorNotSupported when the shape does not fit (rank above 256,
// more than 4096 rows, byte offsets beyond 2^31).
hipError_t launch_sample_step(const KernelParams& p, bool logits_f32, int num_cus, hipStream_t s) {
  if (p.rows < 1 || p.rows > kStepMaxB || num_cus < 1 || p.nparts != sample_step_parts(p.V))
    return hipErrorNotSupported;
  const int64_t lb = logits_f32 ? 4 : 2;
  if (p.rows * p.M * p.V * lb > ((int64_t)1 << 31) || p.V * p.r * 2 > ((int64_t)1 << 31)) return hipErrorNotSupported;
  if (p.latent != nullptr && (p.latent_ld < p.r || p.rows * p.latent_ld * 2 > ((int64_t)1 << 31)))
    return hipErrorNotSupported;
  const int64_t rows_per_chunk = logits_f32 ? 16 : 32;
  const int64_t units = ((p.rows + rows_per_chunk - 1) / rows_per_chunk) * sample_step_parts(p.V);
  const int grid = (int)(units < num_cus ? units : num_cus);
  return logits_f32 ? launch_step_l<true>(p, grid, s) : launch_step_l<false>(p, grid, s);
}

}  // namespace dspark
