// markov_gate.hip -- the gate of the gated Markov head (GatedMarkovHead on
// the markov_head pages: compute_gate and compute_step_bias).  For every row
// the vector the W2 projection consumes is
//   u = sigmoid(gate_proj([h; W1[x]])) * W1[x],
// gate_proj = Linear(d + r, r) with its bias, both concatenated operands in
// the weight dtype W.  Rounding: the Linear's fp32 accumulator (bias added)
// is rounded to W, the fp32 logistic of that to W, the fp32 product to W.
//
// Two launches: the gate GEMM [rows, d + r] x [d + r, r] split along its
// inner dimension into fp32 partial sums, then one thread per (row, output)
// adds the splits in order and finishes u.  The GEMM is small next to the
// projection that follows (0.9 GFLOP and 6 MB at 320 rows, d = 5120,
// r = 256), so the split only has to fill the chip.
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

// ---------------------------------------------------------------- GEMM (bf16)
// Workgroup (bx, by, s): rows 32 bx .. +31, outputs 64 by .. +63, gate-input
// columns [s kchunk, (s + 1) kchunk).  Wave w: rows 16 (w & 1) .. +15,
// outputs 32 (w >> 1) .. +31, as two 16x16 blocks of v_mfma_f32_16x16x32_bf16
// with the input rows on M and the gate outputs on N.  Each lane loads its
// 16-byte pieces straight from memory (an input row's 8 columns, a gate
// weight row's 8 columns); columns past d + r, rows past `rows` and invalid
// ids read zeros through out-of-range buffer offsets.  The columns of a
// split go in blocks of 8 steps of 32, all loads of a block issued before
// its products.
template <bool HF32>
__global__ __launch_bounds__(256) void markov_gate_partial_bf16(GateParams g) {
  constexpr int STEPS = 8;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int rows = (int)g.rows;
  const int r = (int)g.r;
  const int d = (int)g.d;
  const int K = d + r;
  const int n = blockIdx.x * 32 + 16 * (wave & 1) + n16;
  const int jb = blockIdx.y * 64 + 32 * (wave >> 1);
  const int k0 = blockIdx.z * (int)g.kchunk;
  const int k1 = (k0 + (int)g.kchunk < K) ? k0 + (int)g.kchunk : K;

  const bool nrow = n < rows;
  const int64_t x = nrow ? gate_pred(g, n) : -1;
  const bool xok = x >= 0 && x < g.V;
  const uint32_t hbase = nrow ? (uint32_t)gate_hrow(g, n) * (uint32_t)d : 0u;
  const __amdgpu_buffer_rsrc_t rs_h = buffer_rsrc(g.hidden, (uint32_t)g.hidden_bytes);
  const __amdgpu_buffer_rsrc_t rs_w1 = buffer_rsrc(g.w1, (uint32_t)(g.V * r * 2));
  const __amdgpu_buffer_rsrc_t rs_gw = buffer_rsrc(g.gw, (uint32_t)(r * K * 2));
  const uint32_t xrow = xok ? (uint32_t)x * (uint32_t)r : 0u;
  const int j0 = jb + n16, j1 = jb + 16 + n16;

  // A piece: input row n, columns k .. k + 7 (k % 8 == 0, d % 8 == 0, so a
  // piece lies wholly in h or wholly in W1[x])
  auto load_a = [&](int k) __attribute__((always_inline)) -> u32x4_t {
    if constexpr (HF32) {
      const uint32_t off = (nrow && k < d && k < k1) ? (hbase + (uint32_t)k) * 4u : kBufferOob;
      const u32x4_t lo = load16_cached(rs_h, off);
      const u32x4_t hi = load16_cached(rs_h, off + 16u);
      const u32x4_t hv = pack8_bf16(lo, hi);
      const u32x4_t ev = load16_cached(rs_w1, (xok && k >= d && k < k1) ? (xrow + (uint32_t)(k - d)) * 2u : kBufferOob);
      return k < d ? hv : ev;
    } else {
      const u32x4_t hv = load16_cached(rs_h, (nrow && k < d && k < k1) ? (hbase + (uint32_t)k) * 2u : kBufferOob);
      const u32x4_t ev = load16_cached(rs_w1, (xok && k >= d && k < k1) ? (xrow + (uint32_t)(k - d)) * 2u : kBufferOob);
      return k < d ? hv : ev;
    }
  };
  auto load_b = [&](int j, int k) __attribute__((always_inline)) -> u32x4_t {
    return load16_cached(rs_gw, (j < r && k < k1) ? ((uint32_t)j * (uint32_t)K + (uint32_t)k) * 2u : kBufferOob);
  };

  f32x4_t acc0 = f32x4_t{}, acc1 = f32x4_t{};
  for (int kb = k0; kb < k1; kb += 32 * STEPS) {
    u32x4_t av[STEPS], bv0[STEPS], bv1[STEPS];
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const int k = kb + 32 * t + 8 * g4;
      av[t] = load_a(k);
      bv0[t] = load_b(j0, k);
      bv1[t] = load_b(j1, k);
    }
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av[t]);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv0[t]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, bv1[t]), acc1, 0, 0, 0);
    }
  }
  // lane: output jb + n16 (+16), rows 4 g4 .. 4 g4 + 3 of the wave's 16
  float* const part = g.partials + (size_t)blockIdx.z * (size_t)rows * (size_t)r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = blockIdx.x * 32 + 16 * (wave & 1) + 4 * g4 + i;
    if (row < rows) {
      if (j0 < r) part[(size_t)row * r + j0] = acc0[i];
      if (j1 < r) part[(size_t)row * r + j1] = acc1[i];
    }
  }
}

// ---------------------------------------------------------------- GEMM (scalar)
// Any dtypes and shapes: thread (row n, output j) of split s sums its
// columns in order, the hidden values rounded to W first.
template <bool W_BF16, bool HF32>
__global__ __launch_bounds__(256) void markov_gate_partial_scalar(GateParams g) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = g.r, d = g.d, K = d + r;
  if (t >= g.rows * r) return;
  const int64_t n = t / r, j = t % r;
  const int64_t k0 = (int64_t)blockIdx.y * g.kchunk;
  const int64_t k1 = (k0 + g.kchunk < K) ? k0 + g.kchunk : K;
  const int64_t x = gate_pred(g, n);
  const bool xok = x >= 0 && x < g.V;
  const int64_t hrow = gate_hrow(g, n);
  float acc = 0.0f;
  for (int64_t k = k0; k < k1; ++k) {
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
  g.partials[((int64_t)blockIdx.y * g.rows + n) * r + j] = acc;
}

// ---------------------------------------------------------------- finish
template <bool W_BF16>
__global__ __launch_bounds__(256) void markov_gate_finish(GateParams g) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = g.r;
  if (t >= g.rows * r) return;
  const int64_t n = t / r, j = t % r;
  float gate = 1.0f;
  if (g.gated) {
    float z = 0.0f;
    for (int s = 0; s < g.S; ++s) z += g.partials[((int64_t)s * g.rows + n) * r + j];
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
  float u = gate * e;
  if (W_BF16) {
    ((uint16_t*)g.latent)[n * g.latent_ld + j] = (uint16_t)(__float_as_uint(round_bf16(u)) >> 16);
  } else {
    ((float*)g.latent)[n * g.latent_ld + j] = u;
  }
}

// ---------------------------------------------------------------- launchers
int gate_splits(int64_t rows, int64_t r, int64_t d, int64_t* kchunk) {
  const int64_t K = d + r;
  const int64_t tiles = ((rows + 31) / 32) * ((r + 63) / 64);
  const int64_t blocks = (K + 255) / 256;                 // 256-column blocks
  int64_t want = (512 + tiles - 1) / tiles;               // splits to reach ~512 workgroups
  if (want > blocks) want = blocks;
  if (want < 1) want = 1;
  const int64_t per = (blocks + want - 1) / want;         // blocks per split
  *kchunk = per * 256;
  return (int)((K + *kchunk - 1) / *kchunk);
}

hipError_t launch_gate_embeddings(const GateParams& g, bool weights_bf16, hipStream_t s) {
  if (g.rows <= 0) return hipSuccess;
  GateParams e = g;
  e.gated = 0;
  const dim3 fgrid((unsigned)((g.rows * g.r + 255) / 256));
  if (weights_bf16)
    hipLaunchKernelGGL((markov_gate_finish<true>), fgrid, dim3(256), 0, s, e);
  else
    hipLaunchKernelGGL((markov_gate_finish<false>), fgrid, dim3(256), 0, s, e);
  return hipGetLastError();
}

hipError_t launch_gate(const GateParams& g, bool weights_bf16, bool hidden_f32, hipStream_t s) {
  if (g.rows <= 0) return hipSuccess;
  if (!g.gated) return launch_gate_embeddings(g, weights_bf16, s);
  const int64_t K = g.d + g.r;
  const bool mfma = weights_bf16 && g.d % 8 == 0 && g.r % 8 == 0 && g.hidden_bytes <= ((int64_t)1 << 31) &&
                    g.V * g.r * 2 <= ((int64_t)1 << 31) && g.r * K * 2 <= ((int64_t)1 << 31) &&
                    ((uintptr_t)g.hidden & 15u) == 0 && ((uintptr_t)g.w1 & 15u) == 0 &&
                    ((uintptr_t)g.gw & 15u) == 0;
  if (mfma) {
    const dim3 grid((unsigned)((g.rows + 31) / 32), (unsigned)((g.r + 63) / 64), (unsigned)g.S);
    if (hidden_f32)
      hipLaunchKernelGGL((markov_gate_partial_bf16<true>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((markov_gate_partial_bf16<false>), grid, dim3(256), 0, s, g);
  } else {
    const dim3 grid((unsigned)((g.rows * g.r + 255) / 256), (unsigned)g.S);
    if (weights_bf16 && hidden_f32)
      hipLaunchKernelGGL((markov_gate_partial_scalar<true, true>), grid, dim3(256), 0, s, g);
    else if (weights_bf16)
      hipLaunchKernelGGL((markov_gate_partial_scalar<true, false>), grid, dim3(256), 0, s, g);
    else if (hidden_f32)
      hipLaunchKernelGGL((markov_gate_partial_scalar<false, true>), grid, dim3(256), 0, s, g);
    else
      hipLaunchKernelGGL((markov_gate_partial_scalar<false, false>), grid, dim3(256), 0, s, g);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 fgrid((unsigned)((g.rows * g.r + 255) / 256));
  if (weights_bf16)
    hipLaunchKernelGGL((markov_gate_finish<true>), fgrid, dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((markov_gate_finish<false>), fgrid, dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace dspark
