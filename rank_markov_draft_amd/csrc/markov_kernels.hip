// markov_kernels.hip -- gfx950 kernels of the DSpark low-rank Markov head.
//
// The head (third-party markov_head.py page, module docstring) corrects a
// drafter's base logits U_k by B(x_{k-1}, :) = W2 . W1[x_{k-1}]:
//   A2  gather  e = W1[x]                         (get_prev_embeddings)
//   A3  project acc_v = sum_j e_j W2w[v, j]        (project_bias, fp32 accumulate)
//   A4  add     c_v = round_L(base_v + round_L(round_W(acc_v)))  (apply_*_logits)
//   A5  select  argmax or Gumbel-max over v       (_sample_tokens)
//   A6  chain   the drawn token feeds the next position's gather
//                                                  (sample_block_tokens)
//
// markov_tile_bf16 is the bf16 hot path.  A workgroup owns a 128-column slice
// of the vocabulary and walks every row of the call through it:
//   * each of its four waves keeps the W2w rows of 32 columns in VGPRs for the
//     whole launch, so W2 is read from HBM once per call;
//   * per 32-row tile the W1 rows of the predecessors are gathered into LDS and
//     multiplied on the matrix cores (v_mfma_f32_32x32x16_bf16: vocabulary on
//     the M side, rows on the N side, rank on K);
//   * the rounded bias goes back through LDS in row-major order, so the stream
//     of base logits in and corrected logits out is read and written with
//     coalesced 16-byte accesses, 256 contiguous bytes per row and tile;
//   * in sampling steps the same pass folds the corrected values (or their
//     Gumbel scores) into one argmax key per row and slice.
// markov_generic handles fp32 and shapes the tile kernel does not take.
// reduce_row_keys finishes a sampling step: one token per row.
#include "device_common.h"
#include "markov_kernels.h"

namespace dspark {

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ int64_t predecessor(const KernelParams& p, int64_t n) {
  if (p.mode == MODE_APPLY || p.k == 0) return p.ids[n];
  return p.tokens[n * p.M + p.k - 1];
}

__device__ __forceinline__ int64_t base_row_offset(const KernelParams& p, int64_t n) {
  return (p.mode == MODE_APPLY ? n : n * p.M + p.k) * p.V;
}

// ---------------------------------------------------------------- tile kernel
// KS = rank / 16 rounded up to an instantiated value; rank entries past r are
// zero on both operands.
template <int KS, int MODE>
__global__ __launch_bounds__(256) void markov_tile_bf16(KernelParams p) {
  constexpr int RT = 32;                 // rows per tile (MFMA N)
  constexpr int VT = 128;                // vocabulary columns per workgroup
  constexpr int CPR = 2 * KS;            // 16-byte chunks per gathered W1 row
  constexpr int ESTRIDE = 32 * KS + 16;  // LDS bytes per gathered row (+16 against bank conflicts)
  constexpr int BSTRIDE = 2 * VT + 16;   // LDS bytes per bias row
  __shared__ __attribute__((aligned(16))) unsigned char lds_e[RT * ESTRIDE];
  __shared__ __attribute__((aligned(16))) unsigned char lds_b[RT * BSTRIDE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 31;
  const int h = lane >> 5;
  const int64_t V = p.V;
  const int64_t r = p.r;
  const int64_t rows = p.rows;
  const int64_t v0 = (int64_t)blockIdx.x * VT;
  const uint16_t* __restrict__ w1 = (const uint16_t*)p.w1;
  const uint16_t* __restrict__ w2 = (const uint16_t*)p.w2;
  const uint16_t* __restrict__ base = (const uint16_t*)p.base;
  uint16_t* __restrict__ out = (uint16_t*)p.out;

  // A operand: lane (m, h) holds W2w[col(m)][16 kk + 8 h .. + 7] for every kk.
  // col(m) permutes the wave's 32 columns so that the 16 accumulators a lane
  // receives (MFMA rows 8i + 4h + j) are the 16 consecutive columns 16h + 4i + j.
  const int perm = 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
  const int64_t vrow = v0 + wave * 32 + perm;
  bf16x8_t a[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int64_t kof = kk * 16 + 8 * h;
    if (vrow < V && kof < r)
      a[kk] = *(const bf16x8_t*)(w2 + vrow * r + kof);
    else
      a[kk] = bf16x8_t{};
  }

  const int er = tid >> 4;         // epilogue: row within a 16-row half tile
  const int ec = (tid & 15) * 8;   // epilogue: first of 8 columns
  const bool col_ok = (v0 + ec) < V;
  const bool count_bad = (blockIdx.x == 0) && (MODE == MODE_APPLY || p.k == 0);

  for (int64_t row0 = 0; row0 < rows; row0 += RT) {
    // Base logits of this tile's epilogue, requested before the gather so the
    // loads are in flight during the matrix work.
    u32x4_t bl[2];
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int64_t n = row0 + ps * 16 + er;
      if (n < rows && col_ok)
        bl[ps] = __builtin_nontemporal_load((const u32x4_t*)(base + base_row_offset(p, n) + v0 + ec));
      else
        bl[ps] = u32x4_t{0u, 0u, 0u, 0u};
    }

    // A2: gather W1 rows of the tile's predecessors into LDS.
    for (int c = tid; c < RT * CPR; c += 256) {
      const int rr = c / CPR;
      const int part = c - rr * CPR;
      const int64_t n = row0 + rr;
      u32x4_t d = u32x4_t{0u, 0u, 0u, 0u};
      if (n < rows) {
        const int64_t x = predecessor(p, n);
        const bool ok = (x >= 0) && (x < V);
        if (ok && part * 8 < r) d = *(const u32x4_t*)(w1 + x * r + part * 8);
        if (!ok && part == 0 && count_bad) atomicAdd(p.bad_rows, 1u);
      }
      *(u32x4_t*)(lds_e + rr * ESTRIDE + part * 16) = d;
    }
    __syncthreads();

    // A3: acc[col][row] over the rank on the matrix cores.
    f32x16_t acc = f32x16_t{};
    const unsigned char* eb = lds_e + m * ESTRIDE + h * 16;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const bf16x8_t b = *(const bf16x8_t*)(eb + kk * 32);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk], b, acc, 0, 0, 0);
    }
    // The bias in the weight dtype (the Linear's bf16 output), row-major in LDS.
    {
      u32x4_t lo, hi;
      lo.x = pack_bf16x2(acc[0], acc[1]);
      lo.y = pack_bf16x2(acc[2], acc[3]);
      lo.z = pack_bf16x2(acc[4], acc[5]);
      lo.w = pack_bf16x2(acc[6], acc[7]);
      hi.x = pack_bf16x2(acc[8], acc[9]);
      hi.y = pack_bf16x2(acc[10], acc[11]);
      hi.z = pack_bf16x2(acc[12], acc[13]);
      hi.w = pack_bf16x2(acc[14], acc[15]);
      unsigned char* bp = lds_b + m * BSTRIDE + (wave * 32 + 16 * h) * 2;
      *(u32x4_t*)bp = lo;
      *(u32x4_t*)(bp + 16) = hi;
    }
    __syncthreads();

    // A4 (+A5 partials): stream the tile.
#pragma unroll
    for (int ps = 0; ps < 2; ++ps) {
      const int rr = ps * 16 + er;
      const int64_t n = row0 + rr;
      const bool ok = (n < rows) && col_ok;
      const u32x4_t bs = *(const u32x4_t*)(lds_b + rr * BSTRIDE + ec * 2);
      const u32x4_t bb = bl[ps];
      float c[8];
      c[0] = bf16_lo(bb.x) + bf16_lo(bs.x);
      c[1] = bf16_hi(bb.x) + bf16_hi(bs.x);
      c[2] = bf16_lo(bb.y) + bf16_lo(bs.y);
      c[3] = bf16_hi(bb.y) + bf16_hi(bs.y);
      c[4] = bf16_lo(bb.z) + bf16_lo(bs.z);
      c[5] = bf16_hi(bb.z) + bf16_hi(bs.z);
      c[6] = bf16_lo(bb.w) + bf16_lo(bs.w);
      c[7] = bf16_hi(bb.w) + bf16_hi(bs.w);
      u32x4_t o;
      o.x = pack_bf16x2(c[0], c[1]);
      o.y = pack_bf16x2(c[2], c[3]);
      o.z = pack_bf16x2(c[4], c[5]);
      o.w = pack_bf16x2(c[6], c[7]);
      if (ok && out != nullptr)
        __builtin_nontemporal_store(o, (u32x4_t*)(out + base_row_offset(p, n) + v0 + ec));
      if constexpr (MODE != MODE_APPLY) {
        // Selection runs on the L-typed corrected values: the thread's best
        // score (first column on ties) in fp32, one key per thread.
        const uint32_t ow[4] = {o.x, o.y, o.z, o.w};
        const uint32_t vv = (uint32_t)(v0 + ec);
        float best = 0.0f, sumc = 0.0f;
        uint32_t bi = 0;
        // four columns per Philox block (words 0..3 = columns vv + 4 j ..)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float sc[4] = {bf16_lo(ow[2 * j]), bf16_hi(ow[2 * j]), bf16_lo(ow[2 * j + 1]), bf16_hi(ow[2 * j + 1])};
          sumc += (sc[0] + sc[1]) + (sc[2] + sc[3]);
          if constexpr (MODE == MODE_TEMPERATURE) {
            const Philox4 q4 = philox4x32_10((vv >> 2) + (uint32_t)j, p.k_abs, (uint32_t)(p.batch_offset + n), 0u,
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
        uint64_t key = argmax_key(best, vv + bi);
        if (sumc != sumc) {
          // A score is NaN exactly when its corrected value is (the noise is
          // finite): the first NaN wins, as a NaN's key ranks above all.
          // Without one (+inf met -inf in the sum) the scan above stands.
          uint32_t first = 8;
#pragma unroll
          for (int i = 7; i >= 0; --i) {
            const uint32_t hb = (i & 1) ? (ow[i >> 1] >> 16) : (ow[i >> 1] & 0xFFFFu);
            if ((hb & 0x7FFFu) > 0x7F80u) first = (uint32_t)i;
          }
          if (first < 8) key = (0xFFFFFFFFull << 32) | (uint64_t)(0xFFFFFFFFu - (vv + first));
        }
        key = ok ? key : 0ull;
        key = group_max_u64<16>(key);
        if ((tid & 15) == 0 && n < rows) p.partials[n * p.nparts + blockIdx.x] = key;
      }
    }
  }
}

// ---------------------------------------------------------------- generic kernel
// One workgroup per (row, 256-column slice); plain fp32 FMA dot products.
__device__ __forceinline__ float load_f32(const void* p, int64_t i) { return ((const float*)p)[i]; }
__device__ __forceinline__ float load_bf16(const void* p, int64_t i) {
  return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
}
__device__ __forceinline__ float round_bf16_value(float x) {
  return __uint_as_float(pack_bf16x2(x, 0.0f) << 16);
}

template <int MODE, bool L_BF16, bool W_BF16>
__global__ __launch_bounds__(256) void markov_generic(KernelParams p) {
  extern __shared__ float lds_row[];
  __shared__ uint64_t lds_key[4];
  const int64_t n = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t V = p.V, r = p.r;
  const int64_t v = (int64_t)blockIdx.y * 256 + tid;
  const bool count_bad = (blockIdx.y == 0) && (MODE == MODE_APPLY || p.k == 0);

  const int64_t x = predecessor(p, n);
  const bool ok = (x >= 0) && (x < V);
  if (!ok && tid == 0 && count_bad) atomicAdd(p.bad_rows, 1u);
  // gated head: latent row n instead of W1[x]
  const void* const erow = p.latent != nullptr ? p.latent : p.w1;
  const int64_t ebase = p.latent != nullptr ? n * p.latent_ld : x * r;
  for (int64_t j = tid; j < r; j += 256)
    lds_row[j] = ok ? (W_BF16 ? load_bf16(erow, ebase + j) : load_f32(erow, ebase + j)) : 0.0f;
  __syncthreads();

  uint64_t key = 0;
  if (v < V) {
    float acc = 0.0f;
    for (int64_t j = 0; j < r; ++j) {
      const float w = W_BF16 ? load_bf16(p.w2, v * r + j) : load_f32(p.w2, v * r + j);
      acc = __builtin_fmaf(lds_row[j], w, acc);
    }
    float bias = W_BF16 ? round_bf16_value(acc) : acc;
    if (L_BF16) bias = round_bf16_value(bias);
    const int64_t off = base_row_offset(p, n) + v;
    const float b = L_BF16 ? load_bf16(p.base, off) : load_f32(p.base, off);
    float c = b + bias;
    if (L_BF16) c = round_bf16_value(c);
    if (p.out != nullptr) {
      if (L_BF16)
        ((uint16_t*)p.out)[off] = (uint16_t)(__float_as_uint(c) >> 16);
      else
        ((float*)p.out)[off] = c;
    }
    if constexpr (MODE == MODE_GREEDY) key = argmax_key(c, (uint32_t)v);
    if constexpr (MODE == MODE_TEMPERATURE) {
      const Philox4 q = philox4x32_10((uint32_t)((uint64_t)v >> 2), p.k_abs,
                                      (uint32_t)(p.batch_offset + n), 0u, p.seed_lo, p.seed_hi);
      const uint32_t words[4] = {q.x0, q.x1, q.x2, q.x3};
      key = argmax_key(__builtin_fmaf(c, p.kappa, gumbel2_from_word(words[v & 3])), (uint32_t)v);
    }
  }
  if constexpr (MODE != MODE_APPLY) {
    key = group_max_u64<64>(key);
    if ((tid & 63) == 0) lds_key[tid >> 6] = key;
    __syncthreads();
    if (tid == 0) {
      const uint64_t k01 = max_u64(lds_key[0], lds_key[1]);
      const uint64_t k23 = max_u64(lds_key[2], lds_key[3]);
      p.partials[n * p.nparts + blockIdx.y] = max_u64(k01, k23);
    }
  }
}

// ---------------------------------------------------------------- reduction
// One workgroup per batch row: the token of step k is the index in the
// largest of the row's slice keys.
__global__ __launch_bounds__(256) void reduce_row_keys(const uint64_t* __restrict__ partials,
                                                       int64_t nparts, int64_t M, int64_t k,
                                                       int64_t* __restrict__ tokens) {
  __shared__ uint64_t lds_key[4];
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  uint64_t key = 0;
  for (int64_t i = tid; i < nparts; i += 256) key = max_u64(key, partials[b * nparts + i]);
  key = group_max_u64<64>(key);
  if ((tid & 63) == 0) lds_key[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    const uint64_t best = max_u64(max_u64(lds_key[0], lds_key[1]), max_u64(lds_key[2], lds_key[3]));
    tokens[b * M + k] = key_index(best);
  }
}

__global__ void fill_zero_kernel(u32x4_t* __restrict__ p, int64_t n16, unsigned char* __restrict__ tail,
                                 int64_t ntail) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = i; j < n16; j += stride) p[j] = u32x4_t{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0;
}

// Device copy with the streaming (non-temporal) cache policy that the
// kernels above use for logits: each thread has four 16-byte vectors in
// flight per pass, all loaded before any is stored.  A bandwidth reference
// for the measurements, not a step of the head.
__global__ __launch_bounds__(256) void copy_stream_kernel(const u32x4_t* __restrict__ src,
                                                          u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n; base += stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + 256 * u;
      v[u] = i < n ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + 256 * u;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

// ---------------------------------------------------------------- launchers
template <int MODE>
static hipError_t launch_tile_mode(const KernelParams& p, int ks, hipStream_t s) {
  const dim3 grid((unsigned)((p.V + 127) / 128));
  const dim3 block(256);
  switch (ks) {
#define DSPARK_TILE_CASE(K) \
  case K:                   \
    hipLaunchKernelGGL((markov_tile_bf16<K, MODE>), grid, block, 0, s, p); break;
    DSPARK_TILE_CASE(1)
    DSPARK_TILE_CASE(2)
    DSPARK_TILE_CASE(4)
    DSPARK_TILE_CASE(8)
    DSPARK_TILE_CASE(16)
    DSPARK_TILE_CASE(24)
    DSPARK_TILE_CASE(32)
#undef DSPARK_TILE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int tile_ks_for_rank(int64_t r) {
  const int64_t ks = (r + 15) / 16;
  static const int table[] = {1, 2, 4, 8, 16, 24, 32};
  for (int t : table)
    if (ks <= t) return t;
  return 0;
}

hipError_t launch_tile(const KernelParams& p, hipStream_t s) {
  if (p.latent != nullptr) return hipErrorNotSupported;  // vanilla head only
  const int ks = tile_ks_for_rank(p.r);
  if (p.mode == MODE_APPLY) return launch_tile_mode<MODE_APPLY>(p, ks, s);
  if (p.mode == MODE_GREEDY) return launch_tile_mode<MODE_GREEDY>(p, ks, s);
  return launch_tile_mode<MODE_TEMPERATURE>(p, ks, s);
}

template <int MODE>
static hipError_t launch_generic_mode(const KernelParams& p, bool lbf, bool wbf, hipStream_t s) {
  const dim3 grid((unsigned)p.rows, (unsigned)((p.V + 255) / 256));
  const dim3 block(256);
  const size_t lds = (size_t)p.r * sizeof(float);
  if (lbf && wbf)
    hipLaunchKernelGGL((markov_generic<MODE, true, true>), grid, block, lds, s, p);
  else if (!lbf && !wbf)
    hipLaunchKernelGGL((markov_generic<MODE, false, false>), grid, block, lds, s, p);
  else if (lbf)
    hipLaunchKernelGGL((markov_generic<MODE, true, false>), grid, block, lds, s, p);
  else
    hipLaunchKernelGGL((markov_generic<MODE, false, true>), grid, block, lds, s, p);
  return hipGetLastError();
}

hipError_t launch_generic(const KernelParams& p, bool logits_bf16, bool weights_bf16, hipStream_t s) {
  if (p.mode == MODE_APPLY) return launch_generic_mode<MODE_APPLY>(p, logits_bf16, weights_bf16, s);
  if (p.mode == MODE_GREEDY) return launch_generic_mode<MODE_GREEDY>(p, logits_bf16, weights_bf16, s);
  return launch_generic_mode<MODE_TEMPERATURE>(p, logits_bf16, weights_bf16, s);
}

hipError_t launch_reduce(const uint64_t* partials, int64_t nparts, int64_t B, int64_t M, int64_t k,
                         int64_t* tokens, hipStream_t s) {
  hipLaunchKernelGGL(reduce_row_keys, dim3((unsigned)B), dim3(256), 0, s, partials, nparts, M, k,
                     tokens);
  return hipGetLastError();
}

hipError_t launch_copy_stream(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 1023) / 1024;
  if (blocks > 8192) blocks = 8192;   // measured best: 4096 - 8192 workgroups of 256
  hipLaunchKernelGGL(copy_stream_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4_t*)src,
                     (u32x4_t*)dst, n);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t ntail = (int64_t)(bytes % 16);
  int64_t blocks = (n16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (u32x4_t*)p, n16,
                     (unsigned char*)p + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace dspark
