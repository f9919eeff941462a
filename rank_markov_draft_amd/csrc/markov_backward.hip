// markov_backward.hip -- backward of the teacher-forced apply (training): the
// head is trained teacher-forced (the markov_head.py page's module
// docstring), so its gradients are those of apply_block_logits,
//   corrected = base + (W2w . W1[x]).to(L).
// Given G = dloss/dcorrected [rows, V]:
//   g          = G cast to the weight dtype W (backward of the cast)
//   dW2w[v, :] = sum_n g[n, v] W1[x_n]           (rounded once to W)
//   de[n, :]   = sum_v g[n, v] W2w[v, :]         (rounded once to W)
//   dW1[x, :]  = sum over rows n with x_n = x of de[n, :], in row order
// and the base logits' gradient is G itself (nothing to compute).
//
// Four launches on the bf16-weight path:
//   markov_bwd_dw2_bf16   V-sliced: each workgroup streams its 256 columns of
//                         g for all rows, with g and the gathered W1 rows
//                         staged transposed through LDS, and keeps its
//                         [256 x r] gradient block in registers;
//   markov_bwd_de_bf16    g . W2w split along V: each workgroup multiplies its
//                         rows by one 1024-column slice of W2w (staged
//                         transposed through LDS) into fp32 partial sums;
//   markov_bwd_de_finish  the slices' partial sums added in slice order;
//   markov_bwd_dw1        the de rows of each id added in row order (after a
//                         pass that links the rows of equal ids).
// Scalar forms cover fp32 weights and other shapes.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

namespace {

__device__ __forceinline__ float bf16_value(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float round_to_bf16(float x) { return (float)(__bf16)x; }
__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)(__float_as_uint(round_to_bf16(x)) >> 16); }

__device__ __forceinline__ u32x4_t load16_default(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 8 values of g at element offset off of G through a buffer resource
// (offset kBufferOob: zeros), as bf16.  Default cache policy: a 128-byte
// line of g is read by several instructions (16 to 64 bytes of it each),
// which the streaming policy would refetch from HBM.
template <bool LF32>
__device__ __forceinline__ u32x4_t buffer_g8(__amdgpu_buffer_rsrc_t rs, uint32_t eoff, bool in) {
  if constexpr (LF32) {
    const uint32_t off = in ? eoff * 4u : kBufferOob;
    const u32x4_t lo = load16_default(rs, off);
    const u32x4_t hi = load16_default(rs, in ? off + 16u : kBufferOob);
    return u32x4_t{pack_bf16x2(__uint_as_float(lo.x), __uint_as_float(lo.y)),
                   pack_bf16x2(__uint_as_float(lo.z), __uint_as_float(lo.w)),
                   pack_bf16x2(__uint_as_float(hi.x), __uint_as_float(hi.y)),
                   pack_bf16x2(__uint_as_float(hi.z), __uint_as_float(hi.w))};
  } else {
    return load16_default(rs, in ? eoff * 2u : kBufferOob);
  }
}

// Store two source rows' 8 bf16 values (a: row 2 np, b: row 2 np + 1) as the
// 32-bit column pair np of 8 consecutive rows of a transposed LDS tile (row
// stride `stride` bytes).  Lanes of a wave take the 32 column pairs of two
// pieces: with a 144-byte stride one 32-bit store per lane is free of bank
// conflicts.
__device__ __forceinline__ void store_t8x2(unsigned char* base, int stride, int np, u32x4_t a, u32x4_t b) {
  const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
  const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t lo = (c & 1) ? wa[c >> 1] >> 16 : wa[c >> 1] & 0xFFFFu;
    const uint32_t hi = (c & 1) ? wb[c >> 1] >> 16 : wb[c >> 1] & 0xFFFFu;
    *(uint32_t*)(base + c * stride + np * 4) = lo | (hi << 16);
  }
}

}  // namespace

// ---------------------------------------------------------------- dW2 (bf16)
// Workgroup: columns v0 .. v0 + 255 (8 waves x 32).  Chunks of 64 rows: the
// g tile [64 x 256] and the gathered rows E = W1[x_n] [64 x r] go to LDS as
// gT [256][64] and eT [r][64] (rows of 128 bytes plus 16 of padding), then
// wave w multiplies D[j][v] += eT[j][n] gT[v][n] over the chunk's 64 rows
// for its v blocks 2w, 2w + 1 and every 16-unit block of r
// (v_mfma_f32_16x16x32_bf16: rank units on M, columns on N, rows on K).
constexpr int kBwdChunk = 64;                    // columns per LDS chunk of the de product
constexpr int kBwdStride = kBwdChunk * 2 + 16;   // LDS bytes per transposed row (+ pad)
constexpr int kDw2Chunk = 64;                    // rows per LDS chunk of the dW2 product
constexpr int kDw2Stride = kDw2Chunk * 2 + 16;

constexpr int kBwdRowBlock = 4096;  // rows whose W1 offsets sit in LDS at a time

template <int JB, bool LF32>
__global__ __launch_bounds__(512) void markov_bwd_dw2_bf16(BwdParams p) {
  constexpr int CH = kDw2Chunk;
  __shared__ __attribute__((aligned(16))) unsigned char lds_g[256 * kDw2Stride];
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[JB * 16 * kDw2Stride];
  __shared__ int32_t lds_xr[kBwdRowBlock];  // W1 element offset x r of each row, -1: invalid id
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int64_t V = p.V;
  const int r = (int)p.r;
  const int rows = (int)p.rows;
  const int64_t v0 = (int64_t)blockIdx.x * 256;
  constexpr int EP = JB * 2;          // 16-byte pieces per gathered row (JB*16 units), <= 32

  f32x4_t acc[JB][2];
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) acc[jb][0] = acc[jb][1] = f32x4_t{};

  // The W1 offsets of a block of rows go to LDS once; every load is
  // unconditional (buffer offsets past the end read zeros), so one wait per
  // chunk suffices.
  const __amdgpu_buffer_rsrc_t rs_g = buffer_rsrc(p.grad, (uint32_t)(p.rows * V * (LF32 ? 4 : 2)));
  const __amdgpu_buffer_rsrc_t rs_w1 = buffer_rsrc(p.w1, (uint32_t)(V * r * 2));
  // unit u = t + 512 i: row pair np = u % 64 (rows n0 + 2 np, + 1) and piece
  // pq = u / 64 (8 columns of g: 32 pieces; 8 units of W1: EP pieces)
  constexpr int NP = CH / 2;           // row pairs per chunk
  constexpr int UPT = NP * 32 / 512;          // units per thread
  int rb0 = 0;   // first row of the block in LDS
  auto load_chunk = [&](int n0, u32x4_t gv[UPT][2], u32x4_t ev[UPT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 512 * i;
      const int np = u % NP, pq = u / NP;
      const int64_t c = v0 + 8 * pq;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + 2 * np + h;
        gv[i][h] = buffer_g8<LF32>(rs_g, (uint32_t)(n * V + c), n < rows && c < V);
      }
    }
#pragma unroll
    for (int i = 0; i < UPT; ++i) {
      const int u = tid + 512 * i;
      const int np = u % NP, pq = u / NP;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int n = n0 + 2 * np + h;
        const int32_t xr = n < rows ? lds_xr[n - rb0] : -1;
        const bool ein = pq < EP && xr >= 0 && 8 * pq < r;
        ev[i][h] = load16_default(rs_w1, ein ? (uint32_t)(xr + 8 * pq) * 2u : kBufferOob);
      }
    }
  };
  u32x4_t gv[UPT][2], ev[UPT][2];
  for (; rb0 < rows; rb0 += kBwdRowBlock) {
    const int rb1 = (rb0 + kBwdRowBlock < rows) ? rb0 + kBwdRowBlock : rows;
    __syncthreads();   // the previous block's last chunk is done with the table
    for (int n = rb0 + tid; n < rb1; n += 512) {
      const int64_t x = p.ids[n];
      lds_xr[n - rb0] = (x >= 0 && x < V) ? (int32_t)(x * r) : -1;
    }
    __syncthreads();
    load_chunk(rb0, gv, ev);
    for (int n0 = rb0; n0 < rb1; n0 += CH) {
      __syncthreads();   // the previous chunk's products are done with LDS
#pragma unroll
      for (int i = 0; i < UPT; ++i) {
        const int u = tid + 512 * i;
        const int np = u % NP, pq = u / NP;
        store_t8x2(lds_g + (8 * pq) * kDw2Stride, kDw2Stride, np, gv[i][0], gv[i][1]);
        if (pq < EP) store_t8x2(lds_e + (8 * pq) * kDw2Stride, kDw2Stride, np, ev[i][0], ev[i][1]);
      }
      __syncthreads();
      if (n0 + CH < rb1) load_chunk(n0 + CH, gv, ev);   // next chunk in flight
#pragma unroll
      for (int t = 0; t < CH / 32; ++t) {
        bf16x8_t b[2];
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
          b[vb] = *(const bf16x8_t*)(lds_g + ((2 * wave + vb) * 16 + n16) * kDw2Stride + t * 64 + g4 * 16);
#pragma unroll
        for (int jb = 0; jb < JB; ++jb) {
          const bf16x8_t a = *(const bf16x8_t*)(lds_e + (jb * 16 + n16) * kDw2Stride + t * 64 + g4 * 16);
          acc[jb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[0], acc[jb][0], 0, 0, 0);
          acc[jb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[1], acc[jb][1], 0, 0, 0);
        }
      }
    }
  }
  // lane: column v = v0 + 32 wave + 16 vb + n16, units 16 jb + 4 g4 .. + 3
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    const int64_t v = v0 + 32 * wave + 16 * vb + n16;
    if (v >= V) continue;
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) {
      const int j = 16 * jb + 4 * g4;
      if (j >= r) continue;
      const f32x4_t a = acc[jb][vb];
      uint2 w;
      w.x = pack_bf16x2(a[0], a[1]);
      w.y = pack_bf16x2(a[2], a[3]);
      *(uint2*)((uint16_t*)p.dw2 + v * r + j) = w;   // r % 8 == 0: 4 units stay in the row
    }
  }
}

// ---------------------------------------------------------------- de (bf16)
// Workgroup (slice s, row group): rows 256 rg .. + 255, 8 waves of 32 rows
// (2 row blocks each, so that every W2w operand read from LDS serves two
// products), columns [s SL, (s + 1) SL).  Chunks of 64 columns: W2w[64 x r]
// goes to LDS transposed as w2T[r][64]; wave w multiplies
// D[n][j] += g[n][c] w2T[j][c] (rows on M, rank units on N, columns on K),
// its g pieces loaded straight from memory one chunk ahead.  Partial sums
// [S][rows][r] fp32.
template <int JB, bool LF32>
__global__ __launch_bounds__(512) void markov_bwd_de_bf16(BwdParams p) {
  constexpr int NB = 2;                       // row blocks of 16 per wave
  __shared__ __attribute__((aligned(16))) unsigned char lds_w[JB * 16 * kBwdStride];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n16 = lane & 15;
  const int g4 = lane >> 4;
  const int64_t V = p.V;
  const int r = (int)p.r;
  const int rows = (int)p.rows;
  const int s = (int)(blockIdx.x % (unsigned)p.S);
  const int rg = (int)(blockIdx.x / (unsigned)p.S);
  const int64_t c0 = (int64_t)s * p.SL;
  const int64_t c1 = (c0 + p.SL < V) ? c0 + p.SL : V;
  const int nbase = rg * 256 + 32 * wave;     // first row of the wave
  constexpr int WP = JB * 2;                  // 16-byte pieces per W2w row (<= 32)
  constexpr int WU = 32 * WP;                 // (row pair, piece) units of a chunk
  constexpr int WPT = (WU + 511) / 512;

  f32x4_t acc[NB][JB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int jb = 0; jb < JB; ++jb) acc[b][jb] = f32x4_t{};

  // unconditional loads: buffer offsets past the end read zeros
  const __amdgpu_buffer_rsrc_t rs_g = buffer_rsrc(p.grad, (uint32_t)(p.rows * V * (LF32 ? 4 : 2)));
  const __amdgpu_buffer_rsrc_t rs_w2 = buffer_rsrc(p.w2, (uint32_t)(V * r * 2));
  auto load_a = [&](int64_t c, u32x4_t av[NB][kBwdChunk / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < kBwdChunk / 32; ++t) {
        const int n = nbase + 16 * b + n16;
        const int64_t col = c + 32 * t + 8 * g4;
        av[b][t] = buffer_g8<LF32>(rs_g, (uint32_t)((int64_t)n * V + col), n < rows && col < c1);
      }
  };
  // W2w staging: unit u = t + 512 i: row pair u % 32 of the chunk's 64 rows,
  // piece u / 32
  auto load_w = [&](int64_t c, u32x4_t wv[WPT][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int u = tid + 512 * i;
      const int np = u & 31, pq = u >> 5;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t v = c + 2 * np + h;
        const bool in = u < WU && v < c1 && 8 * pq < r;
        wv[i][h] = load16_default(rs_w2, in ? (uint32_t)(v * r + 8 * pq) * 2u : kBufferOob);
      }
    }
  };
  u32x4_t av[NB][kBwdChunk / 32];
  u32x4_t wv[WPT][2];
  load_a(c0, av);
  load_w(c0, wv);
  for (int64_t c = c0; c < c1; c += kBwdChunk) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < WPT; ++i) {
      const int u = tid + 512 * i;
      if (u < WU) store_t8x2(lds_w + (8 * (u >> 5)) * kBwdStride, kBwdStride, u & 31, wv[i][0], wv[i][1]);
    }
    __syncthreads();
    u32x4_t a[NB][kBwdChunk / 32];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int t = 0; t < kBwdChunk / 32; ++t) a[b][t] = av[b][t];
    if (c + kBwdChunk < c1) {   // next chunk in flight during the products
      load_a(c + kBwdChunk, av);
      load_w(c + kBwdChunk, wv);
    }
#pragma unroll
    for (int t = 0; t < kBwdChunk / 32; ++t)
#pragma unroll
      for (int jb = 0; jb < JB; ++jb) {
        const bf16x8_t w = *(const bf16x8_t*)(lds_w + (jb * 16 + n16) * kBwdStride + t * 64 + g4 * 16);
#pragma unroll
        for (int b = 0; b < NB; ++b)
          acc[b][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[b][t]), w,
                                                              acc[b][jb], 0, 0, 0);
      }
  }
  // lane: unit j = 16 jb + n16, rows nbase + 16 b + 4 g4 .. + 3
  float* const part = p.partials + (int64_t)s * rows * r;
#pragma unroll
  for (int jb = 0; jb < JB; ++jb) {
    const int j = 16 * jb + n16;
    if (j >= r) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = nbase + 16 * b + 4 * g4 + i;
        if (row < rows) part[(int64_t)row * r + j] = acc[b][jb][i];
      }
  }
}

// de[n][j] = rnd_W(sum of the S slices' partial sums, in slice order).
template <bool W_BF16>
__global__ __launch_bounds__(256) void markov_bwd_de_finish(BwdParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = p.rows * p.r;
  if (t >= total) return;
  float part[16];
  float z = 0.0f;
  for (int64_t s0 = 0; s0 < p.S; s0 += 16) {
#pragma unroll
    for (int i = 0; i < 16; ++i) part[i] = s0 + i < p.S ? p.partials[(s0 + i) * total + t] : 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (s0 + i < p.S) z += part[i];
  }
  if (W_BF16)
    ((uint16_t*)p.de)[t] = bf16_bits(z);
  else
    ((float*)p.de)[t] = z;
}

// ---------------------------------------------------------------- scalar forms
template <bool L_BF16, bool W_BF16>
__device__ __forceinline__ float g_value(const BwdParams& p, int64_t i) {
  const float x = L_BF16 ? bf16_value(((const uint16_t*)p.grad)[i]) : ((const float*)p.grad)[i];
  return W_BF16 ? round_to_bf16(x) : x;
}
template <bool W_BF16>
__device__ __forceinline__ float w_value(const void* w, int64_t i) {
  return W_BF16 ? bf16_value(((const uint16_t*)w)[i]) : ((const float*)w)[i];
}

// Compensated fp32 sum (Kahan): the scalar forms reduce over up to V
// products, and fp32 weights keep their result to fp32 accuracy.
struct KahanSum {
  float s = 0.0f, c = 0.0f;
  __device__ __forceinline__ void add(float x) {
    const float y = x - c;
    const float t = s + y;
    c = (t - s) - y;
    s = t;
  }
};

// dW2w[v][j], one thread each, rows in order.
template <bool L_BF16, bool W_BF16>
__global__ __launch_bounds__(256) void markov_bwd_dw2_scalar(BwdParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.V * p.r) return;
  const int64_t v = t / p.r, j = t % p.r;
  KahanSum k;
  for (int64_t n = 0; n < p.rows; ++n) {
    const int64_t x = p.ids[n];
    if (x < 0 || x >= p.V) continue;
    k.add(g_value<L_BF16, W_BF16>(p, n * p.V + v) * w_value<W_BF16>(p.w1, x * p.r + j));
  }
  const float a = k.s;
  if (W_BF16)
    ((uint16_t*)p.dw2)[t] = bf16_bits(a);
  else
    ((float*)p.dw2)[t] = a;
}

// de[n][j], one thread each, columns in order.
template <bool L_BF16, bool W_BF16>
__global__ __launch_bounds__(256) void markov_bwd_de_scalar(BwdParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.rows * p.r) return;
  const int64_t n = t / p.r, j = t % p.r;
  KahanSum k;
  for (int64_t v = 0; v < p.V; ++v) k.add(g_value<L_BF16, W_BF16>(p, n * p.V + v) * w_value<W_BF16>(p.w2, v * p.r + j));
  const float a = k.s;
  if (W_BF16)
    ((uint16_t*)p.de)[t] = bf16_bits(a);
  else
    ((float*)p.de)[t] = a;
}

// ---------------------------------------------------------------- dW1
// Row links: link[n] = -2 unless n is the first row of its (valid) id;
// link[rows + n] = the next row with the same valid id (-1: none).  Invalid
// ids are counted in the device error word.  One wave per row n: the lanes
// compare the ids 64 at a time; a ballot finds an earlier equal id and a
// wave minimum the next one.
__global__ __launch_bounds__(256) void markov_bwd_link(BwdParams p) {
  const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (n >= p.rows) return;
  const int64_t x = p.ids[n];
  const bool ok = x >= 0 && x < p.V;
  bool earlier = false;
  int64_t next = INT64_MAX;
  if (ok) {
    for (int64_t m0 = 0; m0 < p.rows; m0 += 64) {
      const int64_t m = m0 + lane;
      const bool same = m < p.rows && m != n && p.ids[m] == x;
      earlier = earlier || __ballot(same && m < n) != 0ull;
      if (same && m > n && m < next) next = m;
    }
    // wave minimum of next
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const int64_t o = __shfl_xor(next, off, 64);
      next = o < next ? o : next;
    }
  }
  if (lane != 0) return;
  if (!ok) atomicAdd(p.bad_rows, 1u);
  p.link[n] = (ok && !earlier) ? 0 : -2;
  p.link[p.rows + n] = (ok && next != INT64_MAX) ? (int32_t)next : -1;
}

// dW1[x_n][j] for the first row n of each id: its rows' de summed in row
// order (fp32), rounded to W.  dW1 is zero-filled before.
template <bool W_BF16>
__global__ __launch_bounds__(256) void markov_bwd_dw1(BwdParams p) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= p.rows * p.r) return;
  const int64_t n = t / p.r, j = t % p.r;
  if (p.link[n] == -2) return;
  KahanSum k;
  for (int64_t m = n; m >= 0; m = p.link[p.rows + m]) k.add(w_value<W_BF16>(p.de, m * p.r + j));
  const float a = k.s;
  const int64_t x = p.ids[n];
  if (W_BF16)
    ((uint16_t*)p.dw1)[x * p.r + j] = bf16_bits(a);
  else
    ((float*)p.dw1)[x * p.r + j] = a;
}

// ---------------------------------------------------------------- launcher
namespace {
template <int JB, bool LF32>
hipError_t launch_bwd_fast(const BwdParams& p, hipStream_t s) {
  hipLaunchKernelGGL((markov_bwd_dw2_bf16<JB, LF32>), dim3((unsigned)((p.V + 255) / 256)), dim3(512), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned groups = (unsigned)((p.rows + 255) / 256);
  hipLaunchKernelGGL((markov_bwd_de_bf16<JB, LF32>), dim3((unsigned)p.S * groups), dim3(512), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((markov_bwd_de_finish<true>), dim3((unsigned)((p.rows * p.r + 255) / 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}
}  // namespace

int64_t backward_slices(int64_t V, int64_t* slice_cols) {
  *slice_cols = 1024;
  return (V + 1023) / 1024;
}

hipError_t launch_backward(const BwdParams& p, bool logits_bf16, bool weights_bf16, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  const int64_t blocks = (p.r + 15) / 16;
  const bool fast = weights_bf16 && p.r % 8 == 0 && p.r <= 256 && p.S == (p.V + p.SL - 1) / p.SL &&
                    p.rows * p.V * (logits_bf16 ? 2 : 4) <= ((int64_t)1 << 31) && p.V * p.r * 2 <= ((int64_t)1 << 31) &&
                    p.partials != nullptr && ((uintptr_t)p.grad & 15u) == 0 && ((uintptr_t)p.w1 & 15u) == 0 &&
                    ((uintptr_t)p.w2 & 15u) == 0 && ((uintptr_t)p.dw2 & 7u) == 0 && p.V % 8 == 0 &&
                    p.rows <= ((int64_t)1 << 24);
  hipError_t e = hipSuccess;
  if (fast) {
    const bool f = !logits_bf16;
    switch (blocks) {
      case 1: e = f ? launch_bwd_fast<1, true>(p, s) : launch_bwd_fast<1, false>(p, s); break;
      case 2: e = f ? launch_bwd_fast<2, true>(p, s) : launch_bwd_fast<2, false>(p, s); break;
      case 3:
      case 4: e = f ? launch_bwd_fast<4, true>(p, s) : launch_bwd_fast<4, false>(p, s); break;
      case 5: case 6: case 7:
      case 8: e = f ? launch_bwd_fast<8, true>(p, s) : launch_bwd_fast<8, false>(p, s); break;
      default: e = f ? launch_bwd_fast<16, true>(p, s) : launch_bwd_fast<16, false>(p, s); break;
    }
  } else {
    const dim3 g2((unsigned)((p.V * p.r + 255) / 256)), ge((unsigned)((p.rows * p.r + 255) / 256));
    if (logits_bf16 && weights_bf16) {
      hipLaunchKernelGGL((markov_bwd_dw2_scalar<true, true>), g2, dim3(256), 0, s, p);
      hipLaunchKernelGGL((markov_bwd_de_scalar<true, true>), ge, dim3(256), 0, s, p);
    } else if (logits_bf16) {
      hipLaunchKernelGGL((markov_bwd_dw2_scalar<true, false>), g2, dim3(256), 0, s, p);
      hipLaunchKernelGGL((markov_bwd_de_scalar<true, false>), ge, dim3(256), 0, s, p);
    } else if (weights_bf16) {
      hipLaunchKernelGGL((markov_bwd_dw2_scalar<false, true>), g2, dim3(256), 0, s, p);
      hipLaunchKernelGGL((markov_bwd_de_scalar<false, true>), ge, dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL((markov_bwd_dw2_scalar<false, false>), g2, dim3(256), 0, s, p);
      hipLaunchKernelGGL((markov_bwd_de_scalar<false, false>), ge, dim3(256), 0, s, p);
    }
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(markov_bwd_link, dim3((unsigned)((p.rows + 3) / 4)), dim3(256), 0, s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_fill_zero(p.dw1, (size_t)(p.V * p.r) * (weights_bf16 ? 2 : 4), s);
  if (e != hipSuccess) return e;
  const dim3 ge((unsigned)((p.rows * p.r + 255) / 256));
  if (weights_bf16)
    hipLaunchKernelGGL((markov_bwd_dw1<true>), ge, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((markov_bwd_dw1<false>), ge, dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dspark
