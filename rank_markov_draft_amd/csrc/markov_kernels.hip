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
// fp32 weights go to markov_rows_mfma_f32w (fp32 products on the matrix
// cores, 64 rows x 128 columns per workgroup) when r and V are multiples of
// 4; markov_rows_fma (scalar FMA, 32 rows x 128 columns, any dtype pair and
// rank) takes every other shape that no faster kernel takes.
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

// ---------------------------------------------------------------- row-tile FMA kernel
// Any dtype pair and rank (fp32 weights, bf16 logits with fp32 weights,
// shapes the matrix-core kernels do not take).  A workgroup of 256 threads
// owns a tile of 32 rows x 128 vocabulary columns.  The rank is walked in
// chunks of 64: the chunk of the tile's 128 W2w rows and of the 32 rows'
// gathered W1 rows (or latent rows) is loaded into LDS with coalesced
// 16-byte loads (the 64 rank elements of a row are contiguous), then thread
// (ty, tx) accumulates rows 2 ty, 2 ty + 1 and columns 8 tx .. 8 tx + 7 with
// fp32 FMAs in rank order.  W2w is thus read once per 32 rows, not once per
// row.  Sampling writes one argmax key per (row, 128-column tile).
__device__ __forceinline__ float load_f32(const void* p, int64_t i) { return ((const float*)p)[i]; }
__device__ __forceinline__ float load_bf16(const void* p, int64_t i) {
  return __uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
}
__device__ __forceinline__ float round_bf16_value(float x) {
  return __uint_as_float(pack_bf16x2(x, 0.0f) << 16);
}

namespace {
constexpr int kFmaRows = 32;
constexpr int kFmaCols = 128;
constexpr int kFmaK = 64;
constexpr int kFmaPitch = kFmaK + 1;  // floats per LDS row (odd: conflict-free column walks)
}  // namespace

// Eight consecutive elements [i, i + 8) of a W-typed array, as floats; the
// caller guarantees the range is in bounds or passes ok = false (zeros).
template <bool W_BF16>
__device__ __forceinline__ void load8(const void* p, int64_t i, bool ok, float out[8]) {
  if (!ok) {
#pragma unroll
    for (int q = 0; q < 8; ++q) out[q] = 0.0f;
    return;
  }
  if constexpr (W_BF16) {
    const u32x4_t v = *(const u32x4_t*)((const uint16_t*)p + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      out[2 * q] = bf16_lo(w[q]);
      out[2 * q + 1] = bf16_hi(w[q]);
    }
  } else {
    const f32x4_t a = *(const f32x4_t*)((const float*)p + i);
    const f32x4_t b = *(const f32x4_t*)((const float*)p + i + 4);
    out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
    out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
  }
}

template <int MODE, bool L_BF16, bool W_BF16>
__global__ __launch_bounds__(256) void markov_rows_fma(KernelParams p, int64_t chunk0) {
  __shared__ float lds_w[kFmaCols * kFmaPitch];  // W2w chunk [128 columns][64 rank]
  __shared__ float lds_e[kFmaRows * kFmaPitch];  // gathered rows [32][64 rank]
  __shared__ int64_t lds_src[kFmaRows];          // source row of each tile row's E (-1: zero)
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t V = p.V, r = p.r;
  const int64_t v0 = (int64_t)blockIdx.x * kFmaCols;
  const int64_t n0 = (chunk0 + blockIdx.y) * kFmaRows;
  const bool count_bad = blockIdx.x == 0 && (MODE == MODE_APPLY || p.k == 0);
  // 16-byte loads of 8-element pieces: rows of a multiple of 8 elements and
  // 16-byte aligned arrays (else element loads)
  const void* const erow = p.latent != nullptr ? p.latent : p.w1;
  const int64_t eld = p.latent != nullptr ? p.latent_ld : r;
  const bool vec_ok = r % 8 == 0 && ((uintptr_t)p.w2 & 15) == 0;
  const bool evec_ok = r % 8 == 0 && eld % 8 == 0 && ((uintptr_t)erow & 15) == 0;

  if (tid < kFmaRows) {
    const int64_t n = n0 + tid;
    int64_t src = -1;
    if (n < p.rows) {
      const int64_t x = predecessor(p, n);
      const bool ok = x >= 0 && x < V;
      if (!ok && count_bad) atomicAdd(p.bad_rows, 1u);
      if (ok) src = p.latent != nullptr ? n * p.latent_ld : x * r;
    }
    lds_src[tid] = src;
  }

  float acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[i][c] = 0.0f;

  for (int64_t k0 = 0; k0 < r; k0 += kFmaK) {
    __syncthreads();  // the previous chunk's reads are done (and lds_src is written)
    // W2w chunk: 128 rows x 64 rank = 1024 pieces of 8; thread t takes pieces t + 256 q
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int piece = tid + 256 * q;
      const int row = piece >> 3, kp = (piece & 7) * 8;
      const int64_t v = v0 + row, k = k0 + kp;
      float w[8];
      if (vec_ok) {
        load8<W_BF16>(p.w2, v * r + k, v < V && k < r, w);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          w[c] = (v < V && k + c < r) ? (W_BF16 ? load_bf16(p.w2, v * r + k + c) : load_f32(p.w2, v * r + k + c))
                                      : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) lds_w[row * kFmaPitch + kp + c] = w[c];
    }
    // E chunk: 32 rows x 64 rank = 256 pieces of 8, one per thread
    {
      const int row = tid >> 3, kp = (tid & 7) * 8;
      const int64_t src = lds_src[row], k = k0 + kp;
      float e[8];
      if (evec_ok) {
        load8<W_BF16>(erow, src + k, src >= 0 && k < r, e);
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c)
          e[c] = (src >= 0 && k + c < r) ? (W_BF16 ? load_bf16(erow, src + k + c) : load_f32(erow, src + k + c))
                                         : 0.0f;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) lds_e[row * kFmaPitch + kp + c] = e[c];
    }
    __syncthreads();
    const int kn = (int)(r - k0 < kFmaK ? r - k0 : kFmaK);
    for (int k = 0; k < kn; ++k) {
      const float e0 = lds_e[(2 * ty) * kFmaPitch + k];
      const float e1 = lds_e[(2 * ty + 1) * kFmaPitch + k];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float w = lds_w[(8 * tx + c) * kFmaPitch + k];
        acc[0][c] = __builtin_fmaf(e0, w, acc[0][c]);
        acc[1][c] = __builtin_fmaf(e1, w, acc[1][c]);
      }
    }
  }

  // epilogue: thread (ty, tx) finishes rows n0 + 2 ty + i, columns v0 + 8 tx + c
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 2 * ty + i;
    const bool row_ok = n < p.rows;
    const int64_t rowoff = row_ok ? base_row_offset(p, n) : 0;
    uint64_t key = 0;
    uint32_t words[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};  // noise words of the 8 columns
    if constexpr (MODE == MODE_TEMPERATURE) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // columns 8 tx + 4 h .. + 3 share one Philox block
        const Philox4 q = philox4x32_10((uint32_t)((uint64_t)(v0 + 8 * tx + 4 * h) >> 2), p.k_abs,
                                        (uint32_t)(p.batch_offset + n), 0u, p.seed_lo, p.seed_hi);
        words[4 * h] = q.x0;
        words[4 * h + 1] = q.x1;
        words[4 * h + 2] = q.x2;
        words[4 * h + 3] = q.x3;
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int64_t v = v0 + 8 * tx + c;
      if (!row_ok || v >= V) continue;
      float bias = W_BF16 ? round_bf16_value(acc[i][c]) : acc[i][c];
      if (L_BF16) bias = round_bf16_value(bias);
      const int64_t off = rowoff + v;
      const float b = L_BF16 ? load_bf16(p.base, off) : load_f32(p.base, off);
      float cval = b + bias;
      if (L_BF16) cval = round_bf16_value(cval);
      if (p.out != nullptr) {
        if (L_BF16)
          ((uint16_t*)p.out)[off] = (uint16_t)(__float_as_uint(cval) >> 16);
        else
          ((float*)p.out)[off] = cval;
      }
      if constexpr (MODE == MODE_GREEDY) key = max_u64(key, argmax_key(cval, (uint32_t)v));
      if constexpr (MODE == MODE_TEMPERATURE)
        key = max_u64(key, argmax_key(__builtin_fmaf(cval, p.kappa, gumbel2_from_word(words[c])), (uint32_t)v));
    }
    if constexpr (MODE != MODE_APPLY) {
      key = group_max_u64<16>(key);  // the 16 threads (tx) of row n
      if (tx == 0 && row_ok) p.partials[n * p.nparts + blockIdx.x] = key;
    }
  }
}

// ---------------------------------------------------------------- fp32 weights on the matrix cores
// The projection of fp32 weights with v_mfma_f32_16x16x4_f32 (fp32 in, fp32
// accumulate), for r and V multiples of 4 and 16-byte aligned operands.  A
// workgroup of eight waves owns 64 rows x 128 columns (one key tile per row,
// as markov_rows_fma); wave w the columns v0 + 16 w .. + 15 for all 64 rows
// (four 16-row tiles, 16 accumulators per lane).
//
// The rank is walked in chunks of 64.  Lane (i, g) = (lane % 16, lane / 16)
// loads W2w[v0 + 16 w + i][16 b + 4 g .. + 3] (one 16-byte load per block b
// of 16 ranks, straight from HBM, one chunk ahead in registers) and feeds
// element q of it to step q of block b: step (b, q) contracts ranks
// {16 b + 4 g + q : g = 0..3}, a partition of the block.  The B operand of
// row j uses the same ranks, read from the 64 rows staged in LDS per chunk
// (two buffers; each chunk's rows are loaded into registers while the
// previous chunk multiplies), or, at ranks up to 256 (WHOLE), all of the 64
// rows staged once before the products, which then run without barriers.  The sum over the rank thus runs in another
// order than the FMA kernel's, inside the admissible interval of an fp32
// sum.  The epilogue is the FMA kernel's: lane (j, g) of row tile t holds
// rows n0 + 16 t + j, columns v0 + 16 w + 4 g .. + 3 (one Philox block).
namespace {
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kFwWaves = 8;
constexpr int kFwThreads = 64 * kFwWaves;
constexpr int kFwCols = 16 * kFwWaves;  // = kFmaCols: the same key tiles
constexpr int kFwRows = 64;
constexpr int kFwK = 64;
constexpr int kFwPitch = kFwK + 4;      // floats per staged row (16-byte aligned, offset banks)
constexpr int kFwWholeK = 256;           // ranks up to which all of a row is staged at once
constexpr int kFwWholePitch = kFwWholeK + 4;
static_assert(kFwCols == kFmaCols, "key tiles");
}  // namespace

template <int MODE, bool L_BF16, bool WHOLE>
__global__ __launch_bounds__(kFwThreads) void markov_rows_mfma_f32w(KernelParams p, int64_t chunk0) {
  constexpr int kBuf = WHOLE ? kFwRows * kFwWholePitch : kFwRows * kFwPitch;  // floats of a staging buffer
  __shared__ __attribute__((aligned(16))) float lds_e[WHOLE ? 1 : 2][kBuf];
  __shared__ int64_t lds_src[kFwRows];
  __shared__ uint64_t lds_key[kFwRows];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15, g = lane >> 4;
  const int64_t V = p.V, r = p.r;
  const int64_t v0 = (int64_t)blockIdx.x * kFwCols;
  const int64_t n0 = (chunk0 + blockIdx.y) * kFwRows;
  const bool count_bad = blockIdx.x == 0 && (MODE == MODE_APPLY || p.k == 0);
  const float* const erow = (const float*)(p.latent != nullptr ? p.latent : p.w1);
  const float* const w2 = (const float*)p.w2;

  if (tid < kFwRows) {
    const int64_t n = n0 + tid;
    int64_t src = -1;
    if (n < p.rows) {
      const int64_t x = predecessor(p, n);
      const bool ok = x >= 0 && x < V;
      if (!ok && count_bad) atomicAdd(p.bad_rows, 1u);
      if (ok) src = p.latent != nullptr ? n * p.latent_ld : x * r;
    }
    lds_src[tid] = src;
    lds_key[tid] = 0ull;
  }
  __syncthreads();

  // staged rows: a chunk of 64 rows x 64 ranks = 1024 vectors of 4, two
  // per thread; row j, rank k of a chunk at lds_e[buf][j * pitch + kofs + k]
  constexpr int kPitch = WHOLE ? kFwWholePitch : kFwPitch;
  f32x4_t ev[WHOLE ? kFwWholeK / kFwK : 1][2];
  auto load_e = [&](int64_t k0, f32x4_t (&e)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int piece = tid + kFwThreads * q;
      const int row = piece >> 4, kp = (piece & 15) * 4;
      const int64_t src = lds_src[row], k = k0 + kp;
      e[q] = (src >= 0 && k < r) ? *(const f32x4_t*)(erow + src + k) : f32x4_t{};
    }
  };
  auto store_e = [&](int buf, int kofs, const f32x4_t (&e)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int piece = tid + kFwThreads * q;
      *(f32x4_t*)&lds_e[buf][(piece >> 4) * kPitch + kofs + (piece & 15) * 4] = e[q];
    }
  };
  const int64_t vrow = v0 + 16 * wave + j16;
  const bool vok = vrow < V;
  f32x4_t a_cur[4], a_nxt[4];
  auto load_a = [&](int64_t k0, f32x4_t (&a)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t k = k0 + 16 * b + 4 * g;
      a[b] = (vok && k < r) ? __builtin_nontemporal_load((const f32x4_t*)(w2 + vrow * r + k)) : f32x4_t{};
    }
  };

  f32x4_t acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4_t{};
  load_a(0, a_cur);
  if constexpr (WHOLE) {
    // every chunk's rows in flight at once, then into LDS
#pragma unroll
    for (int c = 0; c < kFwWholeK / kFwK; ++c) load_e(c * kFwK, ev[c]);
#pragma unroll
    for (int c = 0; c < kFwWholeK / kFwK; ++c) store_e(0, c * kFwK, ev[c]);
  } else {
    load_e(0, ev[0]);
    store_e(0, 0, ev[0]);
  }
  __syncthreads();
  for (int64_t k0 = 0, c = 0; k0 < r; k0 += kFwK, ++c) {
    const int buf = WHOLE ? 0 : (int)(c & 1);
    const int kofs = WHOLE ? (int)k0 : 0;
    const bool more = k0 + kFwK < r;
    if (more) {
      load_a(k0 + kFwK, a_nxt);
      if constexpr (!WHOLE) load_e(k0 + kFwK, ev[0]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f32x4_t bv = *(const f32x4_t*)&lds_e[buf][(16 * t + j16) * kPitch + kofs + 16 * b + 4 * g];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a_cur[b][q], bv[q], acc[t], 0, 0, 0);
      }
    }
    if constexpr (!WHOLE) {
      if (more) store_e(buf ^ 1, 0, ev[0]);  // the other buffer's last reads ended at the previous barrier
      __syncthreads();
    }
    if (more) {
#pragma unroll
      for (int b = 0; b < 4; ++b) a_cur[b] = a_nxt[b];
    }
  }

  // epilogue: lane (j16, g), row tile t: row n0 + 16 t + j16, columns
  // v0 + 16 wave + 4 g .. + 3 (accumulator element e = column + e)
  const int64_t vc = v0 + 16 * wave + 4 * g;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t n = n0 + 16 * t + j16;
    const bool row_ok = n < p.rows;
    uint64_t key = 0;
    if (row_ok && vc < V) {
      const int64_t off = base_row_offset(p, n) + vc;
      float b4[4];
      if constexpr (L_BF16) {
        const u32x2_t w = *(const u32x2_t*)((const uint16_t*)p.base + off);
        b4[0] = bf16_lo(w.x); b4[1] = bf16_hi(w.x); b4[2] = bf16_lo(w.y); b4[3] = bf16_hi(w.y);
      } else {
        const f32x4_t w = *(const f32x4_t*)((const float*)p.base + off);
        b4[0] = w[0]; b4[1] = w[1]; b4[2] = w[2]; b4[3] = w[3];
      }
      float cv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float bias = acc[t][e];
        if (L_BF16) bias = round_bf16_value(bias);
        cv[e] = b4[e] + bias;
        if (L_BF16) cv[e] = round_bf16_value(cv[e]);
      }
      if (p.out != nullptr) {
        if constexpr (L_BF16)
          *(u32x2_t*)((uint16_t*)p.out + off) =
              u32x2_t{(__float_as_uint(cv[0]) >> 16) | (__float_as_uint(cv[1]) & 0xFFFF0000u),
                      (__float_as_uint(cv[2]) >> 16) | (__float_as_uint(cv[3]) & 0xFFFF0000u)};
        else
          *(f32x4_t*)((float*)p.out + off) = f32x4_t{cv[0], cv[1], cv[2], cv[3]};
      }
      if constexpr (MODE == MODE_GREEDY) {
#pragma unroll
        for (int e = 0; e < 4; ++e) key = max_u64(key, argmax_key(cv[e], (uint32_t)(vc + e)));
      }
      if constexpr (MODE == MODE_TEMPERATURE) {
        const Philox4 q4 = philox4x32_10((uint32_t)((uint64_t)vc >> 2), p.k_abs, (uint32_t)(p.batch_offset + n), 0u,
                                         p.seed_lo, p.seed_hi);
        const uint32_t words[4] = {q4.x0, q4.x1, q4.x2, q4.x3};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          key = max_u64(key, argmax_key(__builtin_fmaf(cv[e], p.kappa, gumbel2_from_word(words[e])),
                                        (uint32_t)(vc + e)));
      }
    }
    if constexpr (MODE != MODE_APPLY) {
      key = max_row_lanes(key);  // the row's four lanes (g) in this wave
      if (g == 0 && key != 0ull) atomicMax((unsigned long long*)&lds_key[16 * t + j16], (unsigned long long)key);
    }
  }
  if constexpr (MODE != MODE_APPLY) {
    __syncthreads();
    if (tid < kFwRows && n0 + tid < p.rows) p.partials[(n0 + tid) * p.nparts + blockIdx.x] = lds_key[tid];
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

template <int MODE, bool LBF, bool WBF>
static hipError_t launch_rows_fma(const KernelParams& p, hipStream_t s) {
  const int64_t chunks = (p.rows + kFmaRows - 1) / kFmaRows;
  const unsigned tiles = (unsigned)((p.V + kFmaCols - 1) / kFmaCols);
  for (int64_t c0 = 0; c0 < chunks; c0 += 65535) {  // grid.y holds at most 65535 row chunks
    const int64_t nc = chunks - c0 < 65535 ? chunks - c0 : 65535;
    hipLaunchKernelGGL((markov_rows_fma<MODE, LBF, WBF>), dim3(tiles, (unsigned)nc), dim3(256), 0, s, p, c0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The matrix-core kernel for fp32 weights when the shapes allow 16-byte
// vectors: r, V (and the latent row pitch) multiples of 4, operands 16-byte
// aligned; hipErrorNotSupported otherwise (the FMA kernel takes the call).
template <int MODE, bool LBF>
static hipError_t launch_rows_mfma_f32w(const KernelParams& p, hipStream_t s) {
  const void* erow = p.latent != nullptr ? p.latent : p.w1;
  auto a16 = [](const void* q) { return ((uintptr_t)q & 15u) == 0; };
  if (p.r % 4 != 0 || p.V % 4 != 0 || (p.latent != nullptr && p.latent_ld % 4 != 0)) return hipErrorNotSupported;
  if (!a16(p.w2) || !a16(erow) || !a16(p.base) || (p.out != nullptr && !a16(p.out))) return hipErrorNotSupported;
  const int64_t chunks = (p.rows + kFwRows - 1) / kFwRows;
  const unsigned tiles = (unsigned)((p.V + kFwCols - 1) / kFwCols);
  for (int64_t c0 = 0; c0 < chunks; c0 += 65535) {  // grid.y holds at most 65535 row chunks
    const int64_t nc = chunks - c0 < 65535 ? chunks - c0 : 65535;
    if (p.r <= kFwWholeK)
      hipLaunchKernelGGL((markov_rows_mfma_f32w<MODE, LBF, true>), dim3(tiles, (unsigned)nc), dim3(kFwThreads), 0, s, p, c0);
    else
      hipLaunchKernelGGL((markov_rows_mfma_f32w<MODE, LBF, false>), dim3(tiles, (unsigned)nc), dim3(kFwThreads), 0, s, p,
                         c0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int MODE>
static hipError_t launch_generic_mode(const KernelParams& p, bool lbf, bool wbf, hipStream_t s) {
  if (p.mode != MODE_APPLY && p.nparts != generic_parts(p.V)) return hipErrorInvalidValue;
  if (!wbf) {
    const hipError_t e = lbf ? launch_rows_mfma_f32w<MODE, true>(p, s) : launch_rows_mfma_f32w<MODE, false>(p, s);
    if (e != hipErrorNotSupported) return e;
  }
  if (lbf && wbf) return launch_rows_fma<MODE, true, true>(p, s);
  if (!lbf && !wbf) return launch_rows_fma<MODE, false, false>(p, s);
  if (lbf) return launch_rows_fma<MODE, true, false>(p, s);
  return launch_rows_fma<MODE, false, true>(p, s);
}

int64_t generic_parts(int64_t V) { return (V + kFmaCols - 1) / kFmaCols; }

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
