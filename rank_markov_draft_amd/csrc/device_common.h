// device_common.h -- small device helpers shared by the gfx950 kernels of the
// DSpark low-rank Markov head: bf16 packing, argmax keys and the Philox4x32-10
// Gumbel noise.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- buffers
// Raw buffer loads and stores: a 128-bit resource in scalar registers plus a
// 32-bit byte offset per lane.  The hardware drops a store and returns zeros
// for a load whose offset lies beyond the resource's size, and an offset of
// kBufferOob always does when the size is at most 2^31 bytes.  Kernels use
// that for masked-off lanes instead of branches, so every memory operation
// is unconditional and the compiler keeps exact counts of the ones in
// flight.  kNonTemporal is the streaming cache policy.
constexpr uint32_t kBufferOob = 0x80000000u;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  // word 3: 32-bit data format, as the gfx9 family expects for raw access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNonTemporal);
}
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kNonTemporal);
}
// A device-coherent 8-byte load (the sc1 policy, as a relaxed device-scope
// atomic load uses).  Unlike atomic loads, several of these are issued
// back to back before the first is waited for.
constexpr int kDeviceCoherent = 16;
__device__ __forceinline__ uint64_t buffer_load8_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kDeviceCoherent);
  return ((uint64_t)v.y << 32) | v.x;
}

// ---------------------------------------------------------------- waits and loads to LDS
// s_waitcnt on the vector memory counter only (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data only.  __syncthreads() also orders global
// memory at workgroup scope, which would wait for every load in flight.
// Here each wave finishes its own LDS accesses (lgkmcnt); the buffer loads
// to LDS are waited for explicitly, by count, where their data is needed.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes land at
// LDS address lds + 16 l (lds must be uniform over the wave).  Written as
// inline assembly so that the compiler does not track these loads: it would
// otherwise make later LDS reads of every wave wait for all of them.  Their
// completion is waited for explicitly (wait_vmcnt) before the data is used.
// M0 is saved and restored around the load.
struct BufferWords {
  u32x4_t w;  // V# of a raw buffer: base, stride 0, size in bytes, 32-bit data format
};
__device__ __forceinline__ BufferWords buffer_words(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  return BufferWords{u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, 0x00020000u}};
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)p;
}
// lds must be the same in every lane; it is read through readfirstlane so a
// uniform value the compiler keeps in a vector register still reaches m0.
__device__ __forceinline__ void load_lds16(const BufferWords& r, uint32_t off, uint32_t lds) {
  uint32_t saved;
  __asm__ volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
                   : "=&s"(saved) : "v"(off), "s"(r.w), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
__device__ __forceinline__ void load_lds16_coherent(const BufferWords& r, uint32_t off, uint32_t lds) {
  uint32_t saved;
  __asm__ volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds\n\ts_mov_b32 m0, %0"
                   : "=&s"(saved) : "v"(off), "s"(r.w), "s"(lds) : "memory");
}

// ---------------------------------------------------------------- bf16
// A bf16 value is the upper half of a binary32 value.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round two floats to bf16 (nearest, ties to even: v_cvt_pk_bf16_f32) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t t;
  t[0] = (__bf16)lo;
  t[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, t);
}

// x rounded to bf16 (nearest, ties to even), as a float: one
// v_cvt_pk_bf16_f32 with the rounded value in the upper half and +0 in the
// lower, which is that float's bit pattern.  (The packing helper above makes
// the compiler convert into the lower half and then move it up.)
__device__ __forceinline__ float bf16_rne(float x) {
  float y;
  __asm__("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(y) : "v"(x));
  return y;
}
// Two bf16-valued floats (lower halves zero) packed into one word, lo first.
__device__ __forceinline__ uint32_t join_bf16(float lo, float hi) {
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// corrected = round(fp32(base) + fp32(bias)) for a pair of bf16 logits, with
// the bias first rounded to bf16 (the Linear's output dtype).
__device__ __forceinline__ uint32_t add_bias_pair(uint32_t base2, float acc_lo, float acc_hi) {
  const uint32_t bias2 = pack_bf16x2(acc_lo, acc_hi);
  return pack_bf16x2(bf16_lo(base2) + bf16_lo(bias2), bf16_hi(base2) + bf16_hi(bias2));
}

// ---------------------------------------------------------------- argmax keys
// A 64-bit key whose unsigned order is the argmax order of the pages'
// torch.argmax: larger score first, then the smaller vocabulary index.
// Scores map to an order-preserving 32-bit code (-0 is folded onto +0 and
// every NaN ranks above +inf, as torch.argmax returns a NaN's index); the
// low word holds the complement of the index.
__device__ __forceinline__ uint32_t ordered_code(float s) {
  s = s + 0.0f;  // -0 -> +0
  if (s != s) return 0xFFFFFFFFu;
  uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint64_t argmax_key(float s, uint32_t v) {
  return ((uint64_t)ordered_code(s) << 32) | (uint64_t)(0xFFFFFFFFu - v);
}

__device__ __forceinline__ int64_t key_index(uint64_t key) {
  return (int64_t)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFu));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes of one row of
// a 16 x 16 matrix-instruction result), every lane getting the result: two
// lane-swap instructions (v_permlane16_swap_b32, v_permlane32_swap_b32)
// pair each lane's value with its partner's without a trip through LDS.
// Each swap leaves a lane holding its own word and its partner's, in one
// order or the other; the max does not care which.
__device__ __forceinline__ uint64_t max_row_lanes(uint64_t k) {
  uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  auto l16 = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  auto h16 = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  k = max_u64(((uint64_t)h16[0] << 32) | l16[0], ((uint64_t)h16[1] << 32) | l16[1]);
  lo = (uint32_t)k;
  hi = (uint32_t)(k >> 32);
  auto l32 = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  auto h32 = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  return max_u64(((uint64_t)h32[0] << 32) | l32[0], ((uint64_t)h32[1] << 32) | l32[1]);
}

// Max over the lanes of groups of `width` consecutive lanes (width a power
// of two <= 64); every lane of the group gets the result.
template <int width>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t k) {
#pragma unroll
  for (int off = width / 2; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)k, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(k >> 32), off, 64);
    k = max_u64(k, ((uint64_t)hi << 32) | lo);
  }
  return k;
}

// Order-preserving 16-bit code of a bf16 value (-0 folded onto +0, every
// NaN above +inf), for reductions that only ever compare bf16 values.
__device__ __forceinline__ uint32_t ordered_code_bf16(uint32_t bits16) {
  if (bits16 == 0x8000u) bits16 = 0u;                                  // -0 -> +0
  if ((bits16 & 0x7F80u) == 0x7F80u && (bits16 & 0x007Fu)) return 0xFFFFu;  // NaN
  return (bits16 & 0x8000u) ? (~bits16 & 0xFFFFu) : (bits16 | 0x8000u);
}

// Unsigned max over the 64 lanes of a wave with DPP moves (no LDS traffic);
// the result is valid in lane 63.
__device__ __forceinline__ uint32_t wave_max_u32_to_lane63(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));  // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));  // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));  // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));  // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));  // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

// Float max over the 64 lanes of a wave with DPP moves; valid in lane 63.
// Lanes without a source take -inf.  NaN operands are ignored (v_max_f32).
__device__ __forceinline__ float wave_max_f32_to_lane63(float v) {
  const int ninf = (int)0xFF800000u;
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x111, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x112, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x114, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x118, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x142, 0xA, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(ninf, __float_as_int(v), 0x143, 0xC, 0xF, false)));
  return v;
}

// Unsigned min over the 64 lanes of a wave with DPP moves; valid in lane 63.
__device__ __forceinline__ uint32_t wave_min_u32_to_lane63(uint32_t v) {
  const int big = -1;
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x111, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x112, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x114, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x118, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(big, (int)v, 0x143, 0xC, 0xF, false));
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: row shifts by
// 1, 2, 4 and 8 within each row of 16 lanes, then the broadcasts of lane 15
// (into rows 1 and 3) and lane 31 (into rows 2 and 3).
__device__ __forceinline__ uint32_t wave_inclusive_sum_u32(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Unsigned 64-bit max over the 64 lanes of a wave with DPP moves of both
// halves (row shifts, then the row broadcasts); the result is valid in
// lane 63.  Lanes without a source see 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_u64_step(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, ROW_MASK, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}
__device__ __forceinline__ uint64_t wave_max_u64_lane63(uint64_t k) {
  k = dpp_max_u64_step<0x111, 0xF>(k);  // row_shr:1
  k = dpp_max_u64_step<0x112, 0xF>(k);  // row_shr:2
  k = dpp_max_u64_step<0x114, 0xF>(k);  // row_shr:4
  k = dpp_max_u64_step<0x118, 0xF>(k);  // row_shr:8
  k = dpp_max_u64_step<0x142, 0xA>(k);  // row_bcast:15
  k = dpp_max_u64_step<0x143, 0xC>(k);  // row_bcast:31
  return k;
}

// Order codes of the two bf16 values of a word, one per half: sign set ->
// all bits flipped, else the sign bit set (packed 16-bit shift, then one
// and-or and one xor for both halves).  -0 sorts just below +0 and NaNs sit
// at the ends; callers treat both cases separately.
__device__ __forceinline__ uint32_t pair_order_codes(uint32_t w) {
  typedef short s16x2_t __attribute__((ext_vector_type(2)));
  const s16x2_t sh = __builtin_bit_cast(s16x2_t, w) >> (short)15;
  const uint32_t t = __builtin_bit_cast(uint32_t, sh);
  return w ^ ((t & 0x7FFF7FFFu) | 0x80008000u);
}

// Max over the 64 lanes of a wave with DPP (v_max_u32_dpp); valid in lane 63.
__device__ __forceinline__ uint32_t wave_max_u32_lane63(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return v;
}

// Min over the 64 lanes of a wave with DPP (v_min_u32_dpp); valid in lane 63.
__device__ __forceinline__ uint32_t wave_min_u32_lane63(uint32_t v) {
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x111, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x112, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x114, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x118, 0xF, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x142, 0xA, 0xF, false));
  v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, 0x143, 0xC, 0xF, false));
  return v;
}

// First argmax of a row of bf16 values spread over a wave: lane l holds the
// 8 columns 8l .. 8l+7 as the 4 words o (column 2q in the low half of word
// q), valid when ok; maybe_nan is the lane's hint that one of its values
// may be NaN (from its fp32 sums).  Returns the winning column (< 512, or
// 0xFFFF if no lane is valid) and the 16-bit order code of its value.  NaN
// ranks above everything (torch.argmax returns a NaN's index); -0 and +0 tie
// (the first of them wins).
//
// Fast path: per value a 32-bit key (order code << 16 | 0xFFFF - column),
// the lane's max of 8 keys, one DPP max over the wave.  A row holding a NaN,
// or whose maximum is a zero, takes an exact second pass.
__device__ __forceinline__ void wave_row_argmax_bf16(const u32x4_t o, bool ok, bool maybe_nan,
                                                     uint32_t lane, uint32_t* col, uint32_t* code) {
  const uint32_t w[4] = {o.x, o.y, o.z, o.w};
  const uint32_t c0 = 8u * lane;
  const bool nan_hint = __ballot(ok && maybe_nan) != 0;
  uint32_t kmax = 0;
  if (ok) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t c2 = pair_order_codes(w[q]);
      const uint32_t klo = (c2 << 16) | (0xFFFFu - (c0 + 2u * q));
      const uint32_t khi = (c2 & 0xFFFF0000u) | (0xFFFFu - (c0 + 2u * q + 1u));
      kmax = max(kmax, max(klo, khi));
    }
  }
  const uint32_t K = (uint32_t)__builtin_amdgcn_readlane((int)wave_max_u32_lane63(kmax), 63);
  uint32_t best_code = K >> 16;
  uint32_t best_col = 0xFFFFu - (K & 0xFFFFu);
  const bool zero_max = (best_code == 0x8000u || best_code == 0x7FFFu);
  if (nan_hint || zero_max) {
    // exact pass: first NaN column if any, else first column equal to +-0
    uint32_t nan_idx = 0xFFFFFFFFu, zero_idx = 0xFFFFFFFFu;
    if (ok) {
#pragma unroll
      for (int i = 7; i >= 0; --i) {
        const uint32_t hb = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        const uint32_t mag = hb & 0x7FFFu;
        if (mag > 0x7F80u) nan_idx = c0 + (uint32_t)i;
        if (mag == 0u) zero_idx = c0 + (uint32_t)i;
      }
    }
    const uint32_t first_nan = (uint32_t)__builtin_amdgcn_readlane((int)wave_min_u32_lane63(nan_idx), 63);
    if (first_nan != 0xFFFFFFFFu) {
      best_col = first_nan;
      best_code = 0xFFFFu;
    } else if (zero_max) {
      best_col = (uint32_t)__builtin_amdgcn_readlane((int)wave_min_u32_lane63(zero_idx), 63);
      best_code = 0x8000u;  // the code of +0
    }
  }
  *col = best_col;
  *code = best_code;
}

// ---------------------------------------------------------------- noise
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies by the
// Philox multipliers, a swap of the high halves xored with the neighbour
// words and the round key; the key advances by the Weyl constants.
struct Philox4 {
  uint32_t x0, x1, x2, x3;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p2 = (uint64_t)0xCD9E8D57u * c2;
    // three-way xors in one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p2 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p2;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return Philox4{c0, c1, c2, c3};
}

// Two Philox4x32-10 blocks whose counters differ only in the first word,
// with their rounds interleaved (two independent dependency chains).
__device__ __forceinline__ void philox4x32_10_pair(uint32_t c0a, uint32_t c0b, uint32_t c1, uint32_t c2,
                                                   uint32_t c3, uint32_t k0, uint32_t k1, Philox4& ra,
                                                   Philox4& rb) {
  uint32_t a1 = c1, a2 = c2, a3 = c3, b1 = c1, b2 = c2, b3 = c3;
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t pa0 = (uint64_t)0xD2511F53u * c0a, pa2 = (uint64_t)0xCD9E8D57u * a2;
    const uint64_t pb0 = (uint64_t)0xD2511F53u * c0b, pb2 = (uint64_t)0xCD9E8D57u * b2;
    const uint32_t na0 = __builtin_amdgcn_bitop3_b32((uint32_t)(pa2 >> 32), a1, k0, 0x96);
    const uint32_t na2 = __builtin_amdgcn_bitop3_b32((uint32_t)(pa0 >> 32), a3, k1, 0x96);
    const uint32_t nb0 = __builtin_amdgcn_bitop3_b32((uint32_t)(pb2 >> 32), b1, k0, 0x96);
    const uint32_t nb2 = __builtin_amdgcn_bitop3_b32((uint32_t)(pb0 >> 32), b3, k1, 0x96);
    a1 = (uint32_t)pa2;
    a3 = (uint32_t)pa0;
    b1 = (uint32_t)pb2;
    b3 = (uint32_t)pb0;
    c0a = na0;
    a2 = na2;
    c0b = nb0;
    b2 = nb2;
  }
  ra = Philox4{c0a, a1, a2, a3};
  rb = Philox4{c0b, b1, b2, b3};
}

// Base-2 Gumbel noise from one Philox word: u = (2*(w >> 9) + 1) * 2^-24 lies
// in [2^-24, 1 - 2^-24] (exact in fp32), g = -log2(-log2(u)) with the
// hardware log2 (v_log_f32).  u is formed in two instructions: the 23 bits
// w >> 9 as the mantissa of x = 1 + (w >> 9) 2^-23 (one v_alignbit_b32),
// then u = x - (1 - 2^-24), exact since x and 1 - 2^-24 lie within a factor
// of two of each other.
__device__ __forceinline__ float gumbel2_from_word(uint32_t w) {
  const float x = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  const float u = x - 0x1.fffffep-1f;
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

}  // namespace dspark
