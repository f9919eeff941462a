// markov_lm_head.hip -- the vocabulary head fused with the Markov bias (gfx950).
//
// DeepSeek-V4.1's drafter computes its base logits U = h . lm_head^T in FP32
// (NeMo AutoModel "models/deepseek_v41/dspark" page, compute_logits), and the
// Markov head adds bias.to(U.dtype) to them (third-party markov_head.py page,
// apply_block_logits).  This kernel produces the corrected logits
//     out[n, v] = fp32( U[n, v] + fp32(rnd_bf16(sum_j W1[x_n, j] W2w[v, j])) )
// without U ever reaching HBM: both products run on the matrix cores
// (v_mfma_f32_16x16x32_bf16, exact bf16 products, fp32 accumulation) into
// the same output tile, and the epilogue adds them.
//
// Tiling.  A workgroup of 8 waves owns an output tile of 320 rows x 128
// vocabulary columns and walks the tiles of its row band in a persistent
// loop, so every head weight row is read from HBM once per 320 rows.  Wave
// (wr, wc) holds rows 80 wr .. +79 and columns 64 wc .. +63 as 5 x 4 blocks
// of 16 x 16 fp32 accumulators (80 VGPRs); the vocabulary columns are the
// matrix instruction's M dimension, so a lane's four accumulators of a block
// are four consecutive columns of one row (one 16-byte store).
//
// Operands.  The inner dimension is cut into chunks of 32: first the r/32
// chunks of the bias (A: the gathered W1 rows of the tile's rows, B: the
// tile's W2w rows), then the d/32 chunks of the head (A: hidden rows, B: head
// weight rows), each count padded to an even number with chunks whose
// operands are zeros (they add exact zeros).  The operands take two roads
// into LDS, both over all eight waves:
//   * B (8 KB a chunk, the HBM stream of the head weight): one buffer load
//     to LDS per wave and chunk, into one of four stages, four chunks ahead;
//   * A (20 KB a chunk, the hidden rows every tile re-reads, L2-resident):
//     two or three 16-byte register loads per thread, four chunks ahead in
//     two register sets (even chunks in one, odd in the other, so both are
//     named statically), written to one of two LDS buffers two steps
//     before use.  Loads to LDS alone for A as well measured 15-20% slower:
//     they move about 16 bytes per cycle per CU, which at 28 KB a chunk is
//     the chunk's whole time.
// One barrier a chunk.  After it a wave issues B of chunk g+4, the
// fragment reads of chunk g+1, the stores of A of chunk g+2 and the loads
// of A of chunk g+4, and the products of chunk g on the fragments it read
// a step earlier, so the next chunks' LDS and memory traffic runs beside
// this chunk's matrix work.  Every wave issues the same operations per
// chunk (the loads past the last chunk go to a junk block or read zeros),
// so one wait count serves all.  A row's four 16-byte pieces sit at
// positions q ^ ((row / 2) % 4), which keeps the fragment reads free of
// bank conflicts (the variant q ^ ((row / 4) % 4) measured 5% slower).
// After a tile's bias chunks the accumulators are rounded to bf16 (the
// Linear's output dtype) and parked in a wave-private LDS region (which
// frees their registers for the second fragment set); after its head
// chunks the epilogue adds them in fp32 and stores; the chunk stream runs
// on across tiles.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {
constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * 64;
constexpr int kLmRows = 320;                  // rows of a tile (20 blocks of 16)
constexpr int kLmCols = 128;                  // vocabulary columns of a tile (8 blocks of 16)
constexpr int kLmK = 32;                      // inner-dimension chunk (one matrix instruction)
constexpr int kLmStages = 4;                  // B stages in LDS (issued four chunks ahead)
constexpr int kLmRowBytes = kLmK * 2;         // 64 bytes per operand row and chunk
constexpr int kLmStageA = kLmRows * kLmRowBytes;   // 20 KB
constexpr int kLmStageB = kLmCols * kLmRowBytes;   // 8 KB
constexpr int kLmAPieces = kLmStageA / 16;         // 16-byte pieces of an A chunk: 1280
constexpr int kLmAPer = 3;                         // A loads per thread and chunk (the last for threads < 256)
constexpr int kLmOps = kLmAPer + 1;                // memory operations of a wave per chunk (A loads, one B load)
constexpr int kLmEpiStores = 20;                   // 16-byte stores of a wave's tile epilogue
constexpr int kLmBiasBytes = 20 * 64 * 8;          // a wave's rounded bias of a tile: 20 blocks x 64 lanes x 4 bf16
static_assert(kLmStageB / 1024 == kLmWaves, "one B load per wave and chunk");
static_assert(kLmAPer * kLmThreads >= kLmAPieces && (kLmAPer - 1) * kLmThreads < kLmAPieces, "A pieces");
}  // namespace

__device__ __forceinline__ uint32_t lm_swz(int row, int q) { return (uint32_t)(row * kLmRowBytes + 16 * (q ^ ((row >> 1) & 3))); }

__global__ __launch_bounds__(kLmThreads) void markov_lm_head_bf16(LmHeadParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[kLmStages * kLmStageB];
  __shared__ __attribute__((aligned(16))) unsigned char lds_a[2 * kLmStageA];
  __shared__ __attribute__((aligned(16))) unsigned char lds_junk[1024];
  __shared__ int32_t lds_e[kLmRows];  // gathered W1 row of each tile row (element offset), -1: zero
  // each wave's rounded bias of its current tile (wave-private)
  __shared__ __attribute__((aligned(16))) unsigned char lds_bias[kLmWaves * kLmBiasBytes];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  const int R = (int)p.rows, V = (int)p.V, r = (int)p.r, d = (int)p.d;
  const int row0 = blockIdx.y * kLmRows;
  const int ntiles = (V + kLmCols - 1) / kLmCols;
  // chunks per tile: the bias's, then the head's, each padded to an even
  // count (a padded chunk's operands are zeros and add nothing), so the
  // two register sets of the A stream alternate in a fixed order
  const int nb = ((r + kLmK - 1) / kLmK + 1) & ~1;
  const int C = nb + (((d + kLmK - 1) / kLmK + 1) & ~1);
  const int my_tiles = blockIdx.x < (unsigned)ntiles ? (ntiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int G = my_tiles * C;                   // chunks of this workgroup

  // predecessors of the band's rows (bad ids counted once, by column group 0)
  for (int i = tid; i < kLmRows; i += kLmThreads) {
    const int n = row0 + i;
    int32_t e = -1;
    if (n < R) {
      const int64_t x = p.ids[n];
      if (x >= 0 && x < V) e = (int32_t)x * r;
      else if (blockIdx.x == 0) atomicAdd(p.bad_rows, 1u);
    }
    lds_e[i] = e;
  }
  lds_barrier();

  const BufferWords bw_w2 = buffer_words(p.w2, (uint32_t)V * (uint32_t)r * 2u);
  const BufferWords bw_lm = buffer_words(p.lm, (uint32_t)V * (uint32_t)d * 2u);
  const __amdgpu_buffer_rsrc_t rs_out = buffer_rsrc(p.out, (uint32_t)R * (uint32_t)V * 4u);
  const __amdgpu_buffer_rsrc_t rs_w1 = buffer_rsrc(p.w1, (uint32_t)V * (uint32_t)r * 2u);
  const __amdgpu_buffer_rsrc_t rs_h = buffer_rsrc(p.hidden, (uint32_t)R * (uint32_t)d * 2u);

  auto chunk_of = [&](int g, int* tile, bool* bias, int* k0, int* K) __attribute__((always_inline)) {
    const int t = g / C, c = g - t * C;
    *tile = (int)blockIdx.x + t * (int)gridDim.x;
    *bias = c < nb;
    *k0 = (*bias ? c : c - nb) * kLmK;
    *K = *bias ? r : d;
  };
  // B of chunk g into its stage: wave w moves B rows 16 w .. +15; lane l
  // moves piece position l % 4 of row l / 4 (logical piece q = position ^
  // ((row / 2) % 4)).  Past the last chunk a load to a junk block keeps the
  // memory counts uniform.
  auto issue_b = [&](int g) __attribute__((always_inline)) {
    if (g >= G) {
      load_lds16(bw_lm, kBufferOob, lds_address(&lds_junk[0]));
      return;
    }
    int tile, k0, K;
    bool bias;
    chunk_of(g, &tile, &bias, &k0, &K);
    const uint32_t stage = (uint32_t)(g % kLmStages) * kLmStageB;
    const int row = 16 * wave + (lane >> 2);
    const int q = (lane & 3) ^ ((row >> 1) & 3);
    const int k = k0 + 8 * q;
    const int v = tile * kLmCols + row;
    const uint32_t off = (v < V && k < K) ? 2u * ((uint32_t)v * (uint32_t)K + (uint32_t)k) : kBufferOob;
    const uint32_t dst = lds_address(&lds_b[stage + (uint32_t)(16 * wave) * kLmRowBytes]);
    if (bias) load_lds16(bw_w2, off, dst);
    else load_lds16(bw_lm, off, dst);
  };
  // A of chunk g into registers: thread t loads pieces t + 512 j (row
  // piece / 4, logical piece piece % 4); zeros past the last chunk, past
  // the 1280 pieces, for bad ids and past the rows
  // the rows of the thread's A pieces t + 512 j are fixed for the launch:
  // their W1 element offsets (or -1) and whether the hidden row exists
  int32_t a_e[kLmAPer];
  bool a_n[kLmAPer];
#pragma unroll
  for (int j = 0; j < kLmAPer; ++j) {
    const int pc = tid + kLmThreads * j;
    const int row = (pc >> 2) < kLmRows ? (pc >> 2) : 0;
    a_e[j] = pc < kLmAPieces ? lds_e[row] : -1;
    a_n[j] = pc < kLmAPieces && row0 + row < R;
  }
  auto load_a = [&](int g, u32x4_t (&areg)[kLmAPer]) __attribute__((always_inline)) {
    int tile, k0, K;
    bool bias;
    chunk_of(g < G ? g : 0, &tile, &bias, &k0, &K);
#pragma unroll
    for (int j = 0; j < kLmAPer; ++j) {
      const int pc = tid + kLmThreads * j;
      const int k = k0 + 8 * (pc & 3);
      const uint32_t n = (uint32_t)(row0 + (pc >> 2));
      const bool ok = g < G && k < K && (bias ? a_e[j] >= 0 : a_n[j]);
      const uint32_t off = !ok ? kBufferOob : bias ? 2u * (uint32_t)(a_e[j] + k) : 2u * (n * (uint32_t)d + (uint32_t)k);
      areg[j] = __builtin_amdgcn_raw_buffer_load_b128(bias ? rs_w1 : rs_h, off, 0, 0);
    }
  };
  auto store_a = [&](int g, const u32x4_t (&areg)[kLmAPer]) __attribute__((always_inline)) {
    const uint32_t buf = (uint32_t)(g & 1) * kLmStageA;
#pragma unroll
    for (int j = 0; j < kLmAPer; ++j) {
      const int pc = tid + kLmThreads * j;
      if (j < kLmAPer - 1 || pc < kLmAPieces) *(u32x4_t*)&lds_a[buf + lm_swz(pc >> 2, pc & 3)] = areg[j];
    }
  };

  f32x4_t acc[5][4];
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Operand fragments of one chunk: fa the four 16-column blocks of B, fb
  // the five 16-row blocks of A of the wave's 80 x 64 part of the tile.
  struct Frags {
    bf16x8_t fa[4], fb[5];
  };
  auto read_frags = [&](int g, Frags& f) __attribute__((always_inline)) {
    const uint32_t stage = (uint32_t)(g % kLmStages) * kLmStageB;
    const uint32_t abuf = (uint32_t)(g & 1) * kLmStageA;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 64 * wc + 16 * j + (lane & 15);
      f.fa[j] = *(const bf16x8_t*)&lds_b[stage + lm_swz(col, lane >> 4)];
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int row = 80 * wr + 16 * i + (lane & 15);
      f.fb[i] = *(const bf16x8_t*)&lds_a[abuf + lm_swz(row, lane >> 4)];
    }
  };

  // Pipeline.  After the barrier of step g a wave issues, all independent
  // of one another: B of chunk g+4 into the stage chunk g used, the
  // fragment reads of chunk g+1, the LDS stores of A of chunk g+2 (into the
  // buffer chunk g used) and the register loads of A of chunk g+4, and the
  // products of chunk g on the fragments read a step earlier; so the LDS
  // and memory traffic of the next chunks runs under the matrix work of
  // this one, one barrier a chunk.  A of chunk c sits in register set c % 2
  // from its load (four steps ahead) to its store (two steps ahead).
  u32x4_t a0[kLmAPer], a1[kLmAPer];
  issue_b(0);
  load_a(0, a0);
  load_a(1, a1);
#pragma unroll
  for (int j = 1; j < kLmStages; ++j) issue_b(j);
  wait_vmcnt<0>();  // once: B of chunks 0..3, A of chunks 0 and 1
  store_a(0, a0);
  store_a(1, a1);
  load_a(2, a0);
  load_a(3, a1);
  lds_barrier();
  Frags f0, f1;
  read_frags(0, f0);
  int epi_left = 0;  // steps whose waits still see an epilogue's 20 stores

  // step g: `aset` holds A of chunk g+2 (set g % 2), `cur` the fragments of
  // chunk g; `nxt` receives those of chunk g+1
  auto step = [&](int g, u32x4_t (&aset)[kLmAPer], Frags& cur, Frags& nxt) __attribute__((always_inline)) {
    // B of chunk g+1 (issued three steps ago) has landed; two steps of
    // operations and A of the step before (and an epilogue's stores) may
    // stay in flight
    if (epi_left > 0) {
      wait_vmcnt<2 * kLmOps + kLmAPer + kLmEpiStores>();
      --epi_left;
    } else {
      wait_vmcnt<2 * kLmOps + kLmAPer>();
    }
    lds_barrier();
    issue_b(g + kLmStages);
    read_frags(g + 1, nxt);
    store_a(g + 2, aset);
    load_a(g + 4, aset);
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.fa[j], cur.fb[i], acc[i][j], 0, 0, 0);
  };
  // chunks g0 .. g0 + n - 1 (g0 and n even)
  auto span = [&](int g0, int n) __attribute__((always_inline)) {
    for (int g = g0; g < g0 + n; g += 2) {
      step(g, a0, f0, f1);
      step(g + 1, a1, f1, f0);
    }
  };

  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  unsigned char* const my_bias = &lds_bias[wave * kLmBiasBytes + lane * 8];
  for (int t = 0; t < my_tiles; ++t) {
    const int gt = t * C;
    span(gt, nb);
    // the bias of the tile: the Linear's bf16 output, into the wave's LDS
    // region; the head starts at zero
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *(u32x2_t*)(my_bias + (i * 4 + j) * 512) =
            u32x2_t{pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3])};
        acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    span(gt + nb, C - nb);
    // epilogue: lane l holds columns 4 (l / 16) .. +3 of row l % 16 of each
    // block; U + bias in fp32, one 16-byte store per block
    const int tile = (int)blockIdx.x + t * (int)gridDim.x;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int n = row0 + 80 * wr + 16 * i + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2_t bp = *(const u32x2_t*)(my_bias + (i * 4 + j) * 512);
        const int v = tile * kLmCols + 64 * wc + 16 * j + 4 * (lane >> 4);
        const u32x4_t o = u32x4_t{__float_as_uint(acc[i][j][0] + bf16_lo(bp.x)), __float_as_uint(acc[i][j][1] + bf16_hi(bp.x)),
                                  __float_as_uint(acc[i][j][2] + bf16_lo(bp.y)), __float_as_uint(acc[i][j][3] + bf16_hi(bp.y))};
        buffer_store16(rs_out, (n < R && v < V) ? ((uint32_t)n * (uint32_t)V + (uint32_t)v) * 4u : kBufferOob, o);
        acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
    epi_left = kLmStages - 1;
  }
  wait_vmcnt<0>();
}

// One workgroup per CU (LDS holds one), the row bands spread over the grid's
// y dimension.  Needs bf16 operands, d, r and V multiples of 8, 16-byte
// aligned buffers and every buffer within 2^31 bytes (host checks).
hipError_t launch_lm_head(const LmHeadParams& p, int num_cus, hipStream_t s) {
  if (p.rows < 1 || p.V < 8 || p.r < 8 || p.d < 8 || p.r % 8 || p.d % 8 || p.V % 8) return hipErrorNotSupported;
  const int64_t lim = (int64_t)1 << 31;
  if (p.V * p.d * 2 >= lim || p.rows * p.d * 2 >= lim || p.V * p.r * 2 >= lim || p.rows * p.V * 4 >= lim)
    return hipErrorNotSupported;
  const int64_t bands = (p.rows + kLmRows - 1) / kLmRows;
  if (bands > 65535 || num_cus < 1) return hipErrorNotSupported;
  const int64_t ntiles = (p.V + kLmCols - 1) / kLmCols;
  int64_t gx = (num_cus + bands - 1) / bands;
  if (gx > ntiles) gx = ntiles;
  if (gx < 1) gx = 1;
  hipLaunchKernelGGL(markov_lm_head_bf16, dim3((unsigned)gx, (unsigned)bands), dim3(kLmThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
