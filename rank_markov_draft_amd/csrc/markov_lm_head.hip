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
// weight rows).  Both reach LDS by buffer loads to LDS (1 KB of 16 operand
// rows per instruction), into one of five stages, four chunks ahead of use:
// a chunk is 20 such loads for A (the hidden rows every tile re-reads,
// L2-resident) and 8 for B (the HBM stream of the head weight), dealt over
// all eight waves four each (the last four to a junk block, so that every
// wave's memory counter holds the same count per chunk and one wait before
// each barrier serves all).  Staging A through registers instead (a chunk
// ahead, the register file being nearly full) measured 6% slower.  The
// chunk stream runs on across tiles, so the pipeline never drains at a tile
// edge.  A row's four 16-byte pieces sit at positions q ^ ((row / 2) % 4),
// which keeps the 16-lane fragment reads free of bank conflicts.  After the bias chunks the
// accumulators are rounded to bf16 (the Linear's output dtype), packed and
// kept; after the head chunks the epilogue adds them in fp32 and stores.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {
constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * 64;
constexpr int kLmRows = 320;                  // rows of a tile (20 blocks of 16)
constexpr int kLmCols = 128;                  // vocabulary columns of a tile (8 blocks of 16)
constexpr int kLmK = 32;                      // inner-dimension chunk (one matrix instruction)
constexpr int kLmStages = 5;
constexpr int kLmRowBytes = kLmK * 2;         // 64 bytes per operand row and chunk
constexpr int kLmStageA = kLmRows * kLmRowBytes;   // 20 KB
constexpr int kLmStageB = kLmCols * kLmRowBytes;   // 8 KB
constexpr int kLmDmaA = kLmStageA / 1024;          // 1 KB loads to LDS per chunk for A: 20
constexpr int kLmDmaB = kLmStageB / 1024;          // for B: 8
constexpr int kLmDmaPer = 4;                       // per wave and chunk (28 real, 4 to a junk block)
constexpr int kLmEpiStores = 20;                   // 16-byte stores of a wave's tile epilogue
static_assert(kLmDmaPer * kLmWaves >= kLmDmaA + kLmDmaB, "loads per chunk");
}  // namespace

__device__ __forceinline__ uint32_t lm_swz(int row, int q) { return (uint32_t)(row * kLmRowBytes + 16 * (q ^ ((row >> 1) & 3))); }

__global__ __launch_bounds__(kLmThreads) void markov_lm_head_bf16(LmHeadParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[kLmStages * kLmStageB];
  __shared__ __attribute__((aligned(16))) unsigned char lds_a[kLmStages * kLmStageA];
  __shared__ __attribute__((aligned(16))) unsigned char lds_junk[1024];
  __shared__ int32_t lds_e[kLmRows];  // gathered W1 row of each tile row (element offset), -1: zero

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wr = wave >> 1, wc = wave & 1;
  const int R = (int)p.rows, V = (int)p.V, r = (int)p.r, d = (int)p.d;
  const int row0 = blockIdx.y * kLmRows;
  const int ntiles = (V + kLmCols - 1) / kLmCols;
  const int nb = (r + kLmK - 1) / kLmK;         // bias chunks per tile
  const int C = nb + (d + kLmK - 1) / kLmK;     // chunks per tile
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

  auto chunk_of = [&](int g, int* tile, bool* bias, int* k0, int* K) __attribute__((always_inline)) {
    const int t = g / C, c = g - t * C;
    *tile = (int)blockIdx.x + t * (int)gridDim.x;
    *bias = c < nb;
    *k0 = (*bias ? c : c - nb) * kLmK;
    *K = *bias ? r : d;
  };
  const BufferWords bw_w1 = buffer_words(p.w1, (uint32_t)V * (uint32_t)r * 2u);
  const BufferWords bw_h = buffer_words(p.hidden, (uint32_t)R * (uint32_t)d * 2u);
  // Chunk g's operands into stage g % kLmStages: load d = wave + 8 j moves
  // 16 operand rows (1 KB): d < 20 the A rows 16 d .., d < 28 the B rows
  // 16 (d - 20) .., the rest a junk block (every wave issues the same count,
  // so the waits are uniform).  Lane l moves piece position l % 4 of row
  // l / 4 (logical piece q = position ^ ((row / 2) % 4)).
  auto issue = [&](int g) __attribute__((always_inline)) {
    int tile, k0, K;
    bool bias;
    chunk_of(g, &tile, &bias, &k0, &K);
    const uint32_t st = (uint32_t)(g % kLmStages);
#pragma unroll
    for (int j = 0; j < kLmDmaPer; ++j) {
      const int dd = wave + kLmWaves * j;
      if (dd < kLmDmaA) {
        const int row = 16 * dd + (lane >> 2);
        const int q = (lane & 3) ^ ((row >> 1) & 3);
        const int k = k0 + 8 * q;
        const int n = row0 + row;
        uint32_t off = kBufferOob;
        if (bias) {
          const int32_t e = lds_e[row];
          if (e >= 0 && k < K) off = 2u * (uint32_t)(e + k);
        } else if (n < R && k < K) {
          off = 2u * ((uint32_t)n * (uint32_t)d + (uint32_t)k);
        }
        const uint32_t dst = lds_address(&lds_a[st * kLmStageA + (uint32_t)(16 * dd) * kLmRowBytes]);
        if (bias) load_lds16(bw_w1, off, dst);
        else load_lds16(bw_h, off, dst);
      } else if (dd < kLmDmaA + kLmDmaB) {
        const int i = dd - kLmDmaA;
        const int row = 16 * i + (lane >> 2);
        const int q = (lane & 3) ^ ((row >> 1) & 3);
        const int k = k0 + 8 * q;
        const int v = tile * kLmCols + row;
        const uint32_t off = (v < V && k < K) ? 2u * ((uint32_t)v * (uint32_t)K + (uint32_t)k) : kBufferOob;
        const uint32_t dst = lds_address(&lds_b[st * kLmStageB + (uint32_t)(16 * i) * kLmRowBytes]);
        if (bias) load_lds16(bw_w2, off, dst);
        else load_lds16(bw_lm, off, dst);
      } else {
        load_lds16(bw_lm, kBufferOob, lds_address(&lds_junk[0]));
      }
    }
  };

  f32x4_t acc[5][4];
  uint32_t bias_pk[5][4][2];  // the rounded bias of each block, two bf16 per word
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      bias_pk[i][j][0] = bias_pk[i][j][1] = 0u;
    }

  for (int g = 0; g < kLmStages - 1 && g < G; ++g) issue(g);
  int last_epi = -kLmStages;  // iteration of the last epilogue (its stores count in the waits)

  for (int g = 0; g < G; ++g) {
    {
      // chunk g's loads are in LDS: later chunks' loads (and epilogue
      // stores issued after them) may stay in flight
      const bool tail = g + kLmStages - 2 >= G;
      const bool epi = g > last_epi && g <= last_epi + kLmStages - 1;
      if (tail) wait_vmcnt<0>();
      else if (epi) wait_vmcnt<kLmDmaPer * (kLmStages - 2) + kLmEpiStores>();
      else wait_vmcnt<kLmDmaPer * (kLmStages - 2)>();
    }
    lds_barrier();
    if (g + kLmStages - 1 < G) issue(g + kLmStages - 1);

    // chunk g: 5 row blocks x 4 column blocks of this wave
    const uint32_t stage = (uint32_t)(g % kLmStages) * kLmStageB;
    const uint32_t abuf = (uint32_t)(g % kLmStages) * kLmStageA;
    bf16x8_t fa[4], fb[5];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = 64 * wc + 16 * j + (lane & 15);
      fa[j] = *(const bf16x8_t*)&lds_b[stage + lm_swz(col, lane >> 4)];
    }
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const int row = 80 * wr + 16 * i + (lane & 15);
      fb[i] = *(const bf16x8_t*)&lds_a[abuf + lm_swz(row, lane >> 4)];
    }
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[j], fb[i], acc[i][j], 0, 0, 0);

    const int c = g % C;
    if (c == nb - 1) {
      // the bias of the tile: the Linear's bf16 output; the head starts at zero
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bias_pk[i][j][0] = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
          bias_pk[i][j][1] = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
          acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
    } else if (c == C - 1) {
      // epilogue: lane l holds columns 4 (l / 16) .. +3 of row l % 16 of
      // each block; U + bias in fp32, one 16-byte store per block
      const int tile = (int)blockIdx.x + (g / C) * (int)gridDim.x;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int n = row0 + 80 * wr + 16 * i + (lane & 15);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = tile * kLmCols + 64 * wc + 16 * j + 4 * (lane >> 4);
          const uint32_t b0 = bias_pk[i][j][0], b1 = bias_pk[i][j][1];
          const u32x4_t o = u32x4_t{__float_as_uint(acc[i][j][0] + bf16_lo(b0)), __float_as_uint(acc[i][j][1] + bf16_hi(b0)),
                                    __float_as_uint(acc[i][j][2] + bf16_lo(b1)), __float_as_uint(acc[i][j][3] + bf16_hi(b1))};
          buffer_store16(rs_out, (n < R && v < V) ? ((uint32_t)n * (uint32_t)V + (uint32_t)v) * 4u : kBufferOob, o);
          acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
      last_epi = g;
    }
  }
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
