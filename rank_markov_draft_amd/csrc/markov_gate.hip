// markov_gate.hip -- the gate of the gated Markov head (GatedMarkovHead on
// the markov_head pages: compute_gate and compute_step_bias).  For every row
// the vector the W2 projection consumes is
//   u = sigmoid(gate_proj([h; W1[x]])) * W1[x],
// gate_proj = Linear(d + r, r) with its bias, both concatenated operands in
// the weight dtype W.  Rounding: the Linear's fp32 accumulator (bias added)
// is rounded to W, the fp32 logistic of that to W, the fp32 product to W.
//
// The gate GEMM [rows, d + r] x [d + r, r] runs on 64 x 64 output tiles
// staged through LDS, with the inner dimension split over workgroups when
// there are too few tiles to cover the chip; the splits' fp32 sums are then
// added in split order by a second launch.  The GEMM is small next to the
// projection that follows (0.9 GFLOP and 6 MB at 320 rows, d = 5120,
// r = 256).
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {

__device__ __forceinline__ int64_t gate_pred(const GateParams& g, int64_t n) {
  if (g.mode == MODE_APPLY || g.k == 0) return g.ids[n];
  return g.tokens[n * g.M + g.k - 1];
}

__device__ __forceinline__ int64_t gate_hrow(const GateParams& g, int64_t n) {
  return g.mode == MODE_APPLY ? n : n * g.M + g.k;
}

__device__ __forceinline__ float round_bf16(float x) { return (float)(__bf16)x; }

__device__ __forceinline__ u32x4_t load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 8 fp32 values (two 16-byte pieces) rounded to bf16 and packed.
__device__ __forceinline__ u32x4_t pack8_bf16(u32x4_t lo, u32x4_t hi) {
  return u32x4_t{pack_bf16x2(__uint_as_float(lo.x), __uint_as_float(lo.y)),
                 pack_bf16x2(__uint_as_float(lo.z), __uint_as_float(lo.w)),
                 pack_bf16x2(__uint_as_float(hi.x), __uint_as_float(hi.y)),
                 pack_bf16x2(__uint_as_float(hi.z), __uint_as_float(hi.w))};
}

}  // namespace


// ---------------------------------------------------------------- finish
// Latent element (n, j) from the gate product z (bias not yet added): the
// roundings of the Linear output, the logistic and the product with e.
template <bool W_BF16>
__device__ __forceinline__ void gate_finish_one(const GateParams& g, int64_t n, int64_t j, float z) {
  const int64_t r = g.r;
  float gate = 1.0f;
  if (g.gated) {
    const float bj = W_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)g.gb)[j] << 16) : ((const float*)g.gb)[j];
    z = z + bj;
    if (W_BF16) z = round_bf16(z);
    gate = 1.0f / (1.0f + expf(-z));
    if (W_BF16) gate = round_bf16(gate);
  }
  const int64_t x = gate_pred(g, n);
  const bool xok = x >= 0 && x < g.V;
  float e = 0.0f;
  if (xok) e = W_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)g.w1)[x * r + j] << 16) : ((const float*)g.w1)[x * r + j];
  const float u = gate * e;
  if (W_BF16) {
    ((uint16_t*)g.latent)[n * g.latent_ld + j] = (uint16_t)(__float_as_uint(round_bf16(u)) >> 16);
  } else {
    ((float*)g.latent)[n * g.latent_ld + j] = u;
  }
}

// ---------------------------------------------------------------- GEMM (bf16)
// Workgroup (tile, split): rows 64 bx .. +63 and gate units 64 by .. +63
// over the inner columns [s kc, (s + 1) kc) of [h; e] (d + r columns).  The
// columns go through LDS in chunks of 256: every thread loads 16-byte
// pieces of the input rows and of the gate weight rows (consecutive
// threads, consecutive pieces of a row), rounds fp32 hidden values to
// bf16, and stores them in a padded layout; then each of the 16 waves
// multiplies one 16 x 16 block (v_mfma_f32_16x16x32_bf16, input rows on M,
// units on N).  One split: the tile's latent elements are finished in
// place; several: fp32 partial sums [S][rows][r] for markov_gate_finish.
constexpr int kGateTile = 64;
constexpr int kGateChunk = 256;                      // columns per LDS chunk
constexpr int kGateStride = kGateChunk * 2 + 16;     // LDS bytes per tile row

template <bool HF32>
__global__ __launch_bounds__(1024) void markov_gate_bf16(GateParams g) {
  constexpr int PIECES = kGateTile * kGateChunk / 8;  // 16-byte pieces per operand and chunk
  __shared__ __attribute__((aligned(16))) unsigned char lds_a[kGateTile * kGateStride];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[kGateTile * kGateStride];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int rows = (int)g.rows;
  const int r = (int)g.r;
  const int d = (int)g.d;
  const int K = d + r;
  const int rt = (rows + kGateTile - 1) / kGateTile;
  const int split = (int)(blockIdx.x % (unsigned)g.S);
  const int tile = (int)(blockIdx.x / (unsigned)g.S);
  const int bx = tile % rt, by = tile / rt;
  const int k0 = split * (int)g.kchunk;
  const int k1 = (k0 + (int)g.kchunk < K) ? k0 + (int)g.kchunk : K;
  const uint16_t* const w1 = (const uint16_t*)g.w1;
  const uint16_t* const gw = (const uint16_t*)g.gw;

  // the rows this thread loads pieces of (fixed over the chunks)
  constexpr int PPT = PIECES / 1024;                  // pieces per thread and operand
  int64_t hrow[PPT], xr[PPT];
  bool rok[PPT], xok[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int row = bx * kGateTile + (tid + i * 1024) / (kGateChunk / 8);
    rok[i] = row < rows;
    const int64_t x = rok[i] ? gate_pred(g, row) : -1;
    xok[i] = x >= 0 && x < g.V;
    xr[i] = xok[i] ? x * r : 0;
    hrow[i] = rok[i] ? gate_hrow(g, row) * d : 0;
  }

  // Pieces of chunk c0 into registers: one unconditional load per piece
  // (two for fp32 hidden values) from the selected tensor, or from a safe
  // address with the value then zeroed, so that all loads of a chunk are in
  // flight together.
  const void* const safe = g.gw;
  auto load_chunk = [&](int c0, u32x4_t av[PPT], u32x4_t bv[PPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pc = tid + i * 1024;
      const int k = c0 + 8 * (pc % (kGateChunk / 8));
      const bool in = rok[i] && k < k1;
      const bool hid = in && k < d;
      const bool emb = in && !hid && xok[i];
      const void* pa = safe;
      if (hid) pa = HF32 ? (const void*)((const float*)g.hidden + hrow[i] + k)
                         : (const void*)((const uint16_t*)g.hidden + hrow[i] + k);
      if (emb) pa = w1 + xr[i] + (k - d);
      u32x4_t v = *(const u32x4_t*)pa;
      if constexpr (HF32) {
        const u32x4_t hi = *(const u32x4_t*)(hid ? (const void*)((const float*)pa + 4) : safe);
        if (hid) v = pack8_bf16(v, hi);
      }
      av[i] = (hid || emb) ? v : u32x4_t{0u, 0u, 0u, 0u};
      const int j = by * kGateTile + pc / (kGateChunk / 8);
      const bool bin = j < r && k < k1;
      const u32x4_t w = *(const u32x4_t*)(bin ? (const void*)(gw + (int64_t)j * K + k) : safe);
      bv[i] = bin ? w : u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  f32x4_t acc = f32x4_t{};
  const int ib = wave >> 2, jb = wave & 3;            // the wave's 16 x 16 block
  u32x4_t av[PPT], bv[PPT];
  load_chunk(k0, av, bv);
  for (int c0 = k0; c0 < k1; c0 += kGateChunk) {
    __syncthreads();   // the previous chunk's products are done with LDS
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int pc = tid + i * 1024;
      const int off = (pc / (kGateChunk / 8)) * kGateStride + (pc % (kGateChunk / 8)) * 16;
      *(u32x4_t*)(lds_a + off) = av[i];
      *(u32x4_t*)(lds_b + off) = bv[i];
    }
    __syncthreads();
    if (c0 + kGateChunk < k1) load_chunk(c0 + kGateChunk, av, bv);   // next chunk in flight
    const unsigned char* pa = lds_a + (ib * 16 + n16) * kGateStride + g4 * 16;
    const unsigned char* pb = lds_b + (jb * 16 + n16) * kGateStride + g4 * 16;
#pragma unroll
    for (int t = 0; t < kGateChunk / 32; ++t) {
      const bf16x8_t a = *(const bf16x8_t*)(pa + t * 64);
      const bf16x8_t b = *(const bf16x8_t*)(pb + t * 64);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
  }
  // lane: unit 64 by + 16 jb + n16, rows 64 bx + 16 ib + 4 g4 + i
  const int unit = by * kGateTile + jb * 16 + n16;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = bx * kGateTile + ib * 16 + 4 * g4 + i;
    if (row < rows && unit < r) {
      if (g.S == 1)
        gate_finish_one<true>(g, row, unit, acc[i]);
      else
        g.partials[((int64_t)split * rows + row) * r + unit] = acc[i];
    }
  }
}

// Latent elements from the split partial sums, added in split order.
template <bool W_BF16>
__global__ __launch_bounds__(256) void markov_gate_finish(GateParams g) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = g.rows, r = g.r;
  if (t >= rows * r) return;
  float part[16];
  float z = 0.0f;
  for (int s0 = 0; s0 < g.S; s0 += 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) part[i] = s0 + i < g.S ? g.partials[(s0 + i) * rows * r + t] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i < g.S) z += part[i];
  }
  gate_finish_one<W_BF16>(g, t / r, t % r, z);
}

// ---------------------------------------------------------------- scalar
// Any dtypes and shapes: thread (row n, unit j) sums its inputs in order,
// the hidden values rounded to W first; without hidden states u = e.
template <bool W_BF16, bool HF32>
__global__ __launch_bounds__(256) void markov_gate_scalar(GateParams g) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = g.r, d = g.d, K = d + r;
  if (t >= g.rows * r) return;
  const int64_t n = t / r, j = t % r;
  float acc = 0.0f;
  if (g.gated) {
    const int64_t x = gate_pred(g, n);
    const bool xok = x >= 0 && x < g.V;
    const int64_t hrow = gate_hrow(g, n);
    for (int64_t k = 0; k < K; ++k) {
      float in;
      if (k < d) {
        in = HF32 ? ((const float*)g.hidden)[hrow * d + k]
                  : __uint_as_float((uint32_t)((const uint16_t*)g.hidden)[hrow * d + k] << 16);
        if (W_BF16) in = round_bf16(in);
      } else {
        const int64_t i = x * r + (k - d);
        in = !xok ? 0.0f
                  : (W_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)g.w1)[i] << 16) : ((const float*)g.w1)[i]);
      }
      const float w = W_BF16 ? __uint_as_float((uint32_t)((const uint16_t*)g.gw)[j * K + k] << 16)
                             : ((const float*)g.gw)[j * K + k];
      acc = __builtin_fmaf(in, w, acc);
    }
  }
  gate_finish_one<W_BF16>(g, n, j, acc);
}

// ---------------------------------------------------------------- launcher
// Splits of the inner dimension: as many as keep the grid within two
// workgroups per CU (512), so that a small call's workgroups each load one
// or two LDS chunks in a single round; at most 32 splits and at least 32
// columns per split.
int gate_splits(int64_t rows, int64_t r, int64_t d, int64_t* kchunk) {
  const int64_t K = d + r;
  const int64_t tiles = ((rows + kGateTile - 1) / kGateTile) * ((r + kGateTile - 1) / kGateTile);
  int64_t want = 512 / tiles;
  if (want > 32) want = 32;
  const int64_t steps = (K + 31) / 32;
  if (want > steps) want = steps;
  if (want < 1) want = 1;
  *kchunk = (steps + want - 1) / want * 32;
  return (int)((K + *kchunk - 1) / *kchunk);
}

hipError_t launch_gate(const GateParams& g, bool weights_bf16, bool hidden_f32, hipStream_t s) {
  if (g.rows <= 0) return hipSuccess;
  const int64_t K = g.d + g.r;
  const int64_t tiles = ((g.rows + kGateTile - 1) / kGateTile) * ((g.r + kGateTile - 1) / kGateTile);
  const bool mfma = g.gated && weights_bf16 && g.d % 8 == 0 && g.r % 8 == 0 && tiles <= ((int64_t)1 << 24) &&
                    g.rows <= ((int64_t)1 << 30) &&
                    g.hidden_bytes <= ((int64_t)1 << 31) && g.V * g.r * 2 <= ((int64_t)1 << 31) &&
                    g.r * K * 2 <= ((int64_t)1 << 31) && ((uintptr_t)g.hidden & 15u) == 0 &&
                    ((uintptr_t)g.w1 & 15u) == 0 && ((uintptr_t)g.gw & 15u) == 0;
  if (mfma) {
    GateParams q = g;
    q.S = gate_splits(g.rows, g.r, g.d, &q.kchunk);
    if (q.S > 1 && q.partials == nullptr) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(tiles * q.S));
    if (hidden_f32)
      hipLaunchKernelGGL((markov_gate_bf16<true>), grid, dim3(1024), 0, s, q);
    else
      hipLaunchKernelGGL((markov_gate_bf16<false>), grid, dim3(1024), 0, s, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || q.S == 1) return e;
    hipLaunchKernelGGL((markov_gate_finish<true>), dim3((unsigned)((g.rows * g.r + 255) / 256)), dim3(256), 0, s, q);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((g.rows * g.r + 255) / 256));
  if (weights_bf16 && hidden_f32)
    hipLaunchKernelGGL((markov_gate_scalar<true, true>), grid, dim3(256), 0, s, g);
  else if (weights_bf16)
    hipLaunchKernelGGL((markov_gate_scalar<true, false>), grid, dim3(256), 0, s, g);
  else if (hidden_f32)
    hipLaunchKernelGGL((markov_gate_scalar<false, true>), grid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((markov_gate_scalar<false, false>), grid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace dspark
