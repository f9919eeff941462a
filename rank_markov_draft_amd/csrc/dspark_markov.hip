// dspark_markov.hip -- host side of the C ABI declared in include/dspark_markov.h:
// argument validation, workspace layout, kernel selection and launch.
#include "dspark_markov.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstring>
#include <string>

#include "markov_kernels.h"

namespace {

thread_local std::string g_last_error;

// Workspace layout (the same for every call, so calls of different shapes
// may share a workspace):
//   [0, 256)      control block: the device error word, the
//                 synchronisation-failure count of the persistent chain and
//                 its test hook, each on its own 64-byte line;
//   chain area    arrival counters (kChainSyncBytes), then the device-wide
//                 argmax keys per (step, key group, row): 64-byte slots for
//                 up to kChainMaxSteps steps of 64 rows (greedy chain), or
//                 16-byte slots for up to 4096 step-rows (temperature
//                 chain).  Only the persistent chains write here, and they
//                 leave the area zeroed: their keys and counters must start
//                 at zero, so no other path may put data in it;
//   data          from kDataOffset: the apply kernels' store sink, or the
//                 sampling steps' per-(row, vocabulary slice) argmax keys
//                 (B * ceil(V/128) words), or the backward's and the gated
//                 head's scratch.
constexpr size_t kControlBytes = 256;
constexpr int64_t kChainMaxSteps = 16;
constexpr size_t kChainAreaBytes =
    dspark::kChainSyncBytes + (size_t)kChainMaxSteps * 8 * 64 * dspark::kKeyPad * sizeof(uint64_t);
constexpr size_t kDataOffset = kControlBytes + kChainAreaBytes;
static_assert(kDataOffset % 256 == 0, "data region alignment");

struct Control {
  uint32_t bad_rows;       // byte 0: rows with out-of-range ids
  uint32_t pad0[15];
  uint32_t sync_failures;  // byte 64: failed device-wide waits of the persistent chain
  uint32_t pad1[15];
  uint32_t chain_test_hook;  // byte 128: nonzero makes the chain's waits give up at once
  uint32_t pad2[15];
};
static_assert(sizeof(Control) <= kControlBytes, "control block");

// Size arithmetic of the workspace queries saturates at SIZE_MAX, the
// answer for sizes that cannot be represented.
size_t add_sz(size_t a, size_t b) {
  size_t o;
  return __builtin_add_overflow(a, b, &o) ? SIZE_MAX : o;
}
size_t mul_sz(size_t a, size_t b) {
  size_t o;
  return __builtin_mul_overflow(a, b, &o) ? SIZE_MAX : o;
}
size_t align256(size_t x) { return x > SIZE_MAX - 255 ? SIZE_MAX : (x + 255) & ~(size_t)255; }

size_t partials_bytes(int64_t B, int64_t V) {
  return align256(mul_sz(mul_sz((size_t)B, (size_t)(V / 128 + (V % 128 != 0))), sizeof(uint64_t)));
}

// Compute units of the current device, cached per device.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    cache[dev] = prop.multiProcessorCount;
  }
  return cache[dev];
}

dspark_status_t device_failure(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return DSPARK_ERR_DEVICE;
}

bool known_dtype(int d) { return d == DSPARK_F32 || d == DSPARK_BF16; }

size_t dtype_bytes(dspark_dtype_t d) { return d == DSPARK_F32 ? 4 : 2; }

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int64_t vocab_slices(int64_t V) { return (V + 127) / 128; }

// Largest rank the row-tile kernels take (they walk the rank in chunks; the
// limit is the documented one of the C ABI).
constexpr int64_t kGenericMaxRank = 16384;

// The bf16 tile kernel takes the call when both dtypes are bf16, the rank is
// a multiple of 8 no larger than 512, rows of logits are whole 16-byte
// vectors and every streamed pointer is 16-byte aligned.
bool tile_path(dspark_dtype_t ldt, dspark_dtype_t wdt, int64_t V, int64_t r, const void* base,
               const void* out, const void* w1, const void* w2) {
  return ldt == DSPARK_BF16 && wdt == DSPARK_BF16 && r % 8 == 0 &&
         dspark::tile_ks_for_rank(r) != 0 && V % 8 == 0 && aligned16(base) &&
         (out == nullptr || aligned16(out)) && aligned16(w1) && aligned16(w2);
}

// Shared checks of both operations.  Returns DSPARK_OK to proceed, or the
// status to return; *empty is set when there is no work.
dspark_status_t check_common(int ldt, int wdt, int64_t B, int64_t M, int64_t V, int64_t r,
                             int64_t* elems) {
  if (!known_dtype(ldt) || !known_dtype(wdt)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (B < 0 || M < 0 || V < 0 || r <= 0) return DSPARK_ERR_INVALID_ARGUMENT;
  int64_t rows = 0, e = 0, wv = 0;
  if (!mul_ok(B, M, &rows) || !mul_ok(rows, V, &e) || !mul_ok(V, r, &wv))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (V > (int64_t)0x7FFFFFFF) return DSPARK_ERR_UNSUPPORTED;
  *elems = e;
  return DSPARK_OK;
}

// ---- gated head
// Gated-call workspace past the vanilla layout: the latent rows of the call
// ([rows, r], at most 4 bytes per element), then the gate GEMM's split sums
// ([S][rows][r] fp32) when it splits its inner dimension.
size_t gated_region_bytes(int64_t rows, int64_t r, int64_t d) {
  int64_t rr = 0, t = 0;
  if (!mul_ok(rows, r, &rr) || !mul_ok(rows, d, &t) || d > (int64_t)0x7FFFFFFF) return SIZE_MAX;
  int64_t kchunk = 0;
  const int S = d > 0 ? dspark::gate_splits(rows, r, d, &kchunk) : 1;
  const size_t lat = align256(mul_sz((size_t)rr, 4));
  return S > 1 ? add_sz(lat, align256(mul_sz(mul_sz((size_t)S, (size_t)rr), 4))) : lat;
}

dspark_status_t check_gate_args(bool gated, int hdt, int64_t d, const void* gw, const void* gb, int64_t rows,
                                int64_t r) {
  if (!gated) return DSPARK_OK;
  if (!known_dtype(hdt) || d <= 0) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!gw || !gb) return DSPARK_ERR_INVALID_ARGUMENT;
  int64_t t = 0, k = 0;
  if (!mul_ok(rows, d, &t) || !mul_ok(t, 4, &t) || !mul_ok(d + r, r, &k)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (d > (int64_t)0x7FFFFFFF || k > (int64_t)0x3FFFFFFF) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

// The gate of `rows` rows: apply (ids = token_ids, hidden row n) or
// sampling step k (ids = first_prev, tokens, hidden row b * M + k); latent
// rows go to `latent` (row stride latent_ld elements).  `region` is the
// gated workspace region (latent scratch, then the split sums).
hipError_t run_gate(char* region, const void* hidden, dspark_dtype_t hdt, int64_t d, const int64_t* ids,
                    const int64_t* tokens, const void* w1, const void* gw, const void* gb, dspark_dtype_t wdt,
                    int64_t rows, int64_t V, int64_t r, int64_t M, int64_t k, void* latent, int64_t latent_ld,
                    int mode, bool gated, hipStream_t s) {
  dspark::GateParams g{};
  g.partials = (float*)(region + align256((size_t)(rows * r) * 4));
  g.hidden = gated ? hidden : nullptr;
  g.ids = ids;
  g.tokens = tokens;
  g.w1 = w1;
  g.gw = gw;
  g.gb = gb;
  g.latent = latent;
  g.rows = rows;
  g.V = V;
  g.r = r;
  g.d = gated ? d : 0;
  g.M = M;
  g.k = k;
  g.latent_ld = latent_ld;
  g.mode = mode;
  g.gated = gated ? 1 : 0;
  g.hidden_bytes = gated ? rows * (mode == dspark::MODE_APPLY ? 1 : M) * d * (int64_t)dtype_bytes(hdt) : 0;
  return dspark::launch_gate(g, wdt == DSPARK_BF16, hdt == DSPARK_F32, s);
}

}  // namespace

extern "C" {

size_t dspark_markov_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r, int sample_mode) {
  (void)r;
  if (B < 0 || V < 0 || M < 0) return kDataOffset;
  // a sampling workspace also serves the apply of the same sizes
  const size_t sink = dspark::apply_sink_bytes();
  if (sample_mode) {
    const size_t parts = partials_bytes(B, V);
    return add_sz(kDataOffset, parts > sink ? parts : sink);
  }
  return kDataOffset + sink;
}

dspark_status_t dspark_markov_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (!workspace || bytes == 0) return DSPARK_ERR_INVALID_ARGUMENT;
  const hipError_t e = dspark::launch_fill_zero(workspace, bytes, (hipStream_t)stream);
  if (e != hipSuccess) return device_failure(e, "workspace fill");
  return DSPARK_OK;
}

dspark_status_t dspark_markov_apply_block(const void* base_logits, dspark_dtype_t logits_dtype,
                                          const int64_t* token_ids, const void* w1,
                                          const void* w2, dspark_dtype_t weight_dtype,
                                          int64_t B, int64_t M, int64_t V, int64_t r,
                                          void* corrected_logits, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  int64_t elems = 0;
  dspark_status_t st = check_common(logits_dtype, weight_dtype, B, M, V, r, &elems);
  if (st != DSPARK_OK) return st;
  if (elems == 0) return DSPARK_OK;  // numel() == 0: the input is the result
  if (!base_logits || !token_ids || !w1 || !w2 || !corrected_logits) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_workspace_bytes(B, M, V, r, 0))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const size_t lbytes = (size_t)elems * dtype_bytes(logits_dtype);
  const size_t wbytes = (size_t)(V * r) * dtype_bytes(weight_dtype);
  const size_t ibytes = (size_t)(B * M) * sizeof(int64_t);
  if (corrected_logits != base_logits && overlaps(corrected_logits, lbytes, base_logits, lbytes))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (overlaps(corrected_logits, lbytes, w1, wbytes) || overlaps(corrected_logits, lbytes, w2, wbytes) ||
      overlaps(corrected_logits, lbytes, token_ids, ibytes))
    return DSPARK_ERR_INVALID_ARGUMENT;

  dspark::KernelParams p{};
  p.base = base_logits;
  p.out = corrected_logits;
  p.ids = token_ids;
  p.w1 = w1;
  p.w2 = w2;
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.rows = B * M;
  p.V = V;
  p.r = r;
  p.M = M;
  p.mode = dspark::MODE_APPLY;
  hipError_t e;
  const bool tile = tile_path(logits_dtype, weight_dtype, V, r, base_logits, corrected_logits, w1, w2);
  // fp32 logits with bf16 weights stream through the grouped kernel too
  const bool f32_tile = tile_path(DSPARK_BF16, weight_dtype, V, r, base_logits, corrected_logits, w1, w2) &&
                        logits_dtype == DSPARK_F32;
  if (!tile && !f32_tile && r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
  p.sink = (char*)workspace + kDataOffset;
  e = hipErrorNotSupported;
  if (f32_tile) {
    e = dspark::launch_apply_grouped(p, true, (hipStream_t)stream);
    if (e == hipErrorNotSupported) {
      (void)hipGetLastError();
      e = dspark::launch_generic(p, false, true, (hipStream_t)stream);
    }
  } else if (tile) {
    // grouped form (one bias per distinct predecessor) when the plan fits
    // in LDS, else the streaming form, else the tile kernel
    e = dspark::launch_apply_grouped(p, false, (hipStream_t)stream);
    if (e == hipErrorNotSupported) {
      (void)hipGetLastError();
      e = dspark::launch_apply_wide(p, (hipStream_t)stream);
    }
    if (e == hipErrorNotSupported) {  // element offsets beyond 31 bits
      (void)hipGetLastError();
      e = dspark::launch_tile(p, (hipStream_t)stream);
    }
  } else
    e = dspark::launch_generic(p, logits_dtype == DSPARK_BF16, weight_dtype == DSPARK_BF16,
                               (hipStream_t)stream);
  if (e != hipSuccess) return device_failure(e, "apply launch");
  return DSPARK_OK;
}

}  // extern "C"

namespace dspark {

void set_last_error(const std::string& msg) { g_last_error = msg; }

// Left-to-right sampling on a given workspace.  `clear_control` zero-fills
// the workspace's control block (error words and test hook) on the stream
// once the arguments have passed validation, before the first kernel: the
// static-scratch variant starts every call from a clean record.
dspark_status_t sample_block_impl(const void* base_logits, dspark_dtype_t logits_dtype,
                                  const int64_t* first_prev_token_ids, const void* w1, const void* w2,
                                  dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V, int64_t r,
                                  double temperature, uint64_t seed, int64_t position_offset,
                                  int64_t batch_offset, int64_t* sampled_tokens, void* corrected_logits,
                                  void* workspace, size_t workspace_bytes, void* stream, bool clear_control) {
  int64_t elems = 0;
  dspark_status_t st = check_common(logits_dtype, weight_dtype, B, M, V, r, &elems);
  if (st != DSPARK_OK) return st;
  if (std::isnan(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (B == 0 || M == 0) return DSPARK_OK;
  if (V == 0) return DSPARK_ERR_INVALID_ARGUMENT;  // nothing to draw from
  if (!base_logits || !first_prev_token_ids || !w1 || !w2 || !sampled_tokens)
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_workspace_bytes(B, M, V, r, 1))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const size_t lbytes = (size_t)elems * dtype_bytes(logits_dtype);
  const size_t wbytes = (size_t)(V * r) * dtype_bytes(weight_dtype);
  const size_t tbytes = (size_t)(B * M) * sizeof(int64_t);
  const void* ins[4] = {base_logits, w1, w2, first_prev_token_ids};
  const size_t ins_bytes[4] = {lbytes, wbytes, wbytes, (size_t)B * sizeof(int64_t)};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(sampled_tokens, tbytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
    if (corrected_logits && overlaps(corrected_logits, lbytes, ins[i], ins_bytes[i]))
      return DSPARK_ERR_INVALID_ARGUMENT;
  }
  if (corrected_logits && overlaps(corrected_logits, lbytes, sampled_tokens, tbytes))
    return DSPARK_ERR_INVALID_ARGUMENT;

  if (clear_control) {
    const hipError_t e = dspark::launch_fill_zero(workspace, kControlBytes, (hipStream_t)stream);
    if (e != hipSuccess) return device_failure(e, "scratch control clear");
  }
  const bool greedy = temperature < 1e-5;
  dspark::KernelParams p{};
  p.base = base_logits;
  p.out = corrected_logits;
  p.ids = first_prev_token_ids;
  p.tokens = sampled_tokens;
  p.w1 = w1;
  p.w2 = w2;
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.partials = (uint64_t*)((char*)workspace + kDataOffset);
  p.rows = B;
  p.V = V;
  p.r = r;
  p.M = M;
  p.batch_offset = batch_offset;
  p.mode = greedy ? dspark::MODE_GREEDY : dspark::MODE_TEMPERATURE;
  p.kappa = greedy ? 0.0f : (float)(1.4426950408889634 / temperature);
  p.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(seed >> 32);
  const bool tile = tile_path(logits_dtype, weight_dtype, V, r, base_logits, corrected_logits, w1, w2);
  // fp32 logits with bf16 weights sample through the step kernel too
  const bool f32_tile = logits_dtype == DSPARK_F32 &&
                        tile_path(DSPARK_BF16, weight_dtype, V, r, base_logits, corrected_logits, w1, w2);
  if (!tile && !f32_tile && r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
  p.nparts = tile ? vocab_slices(V) : dspark::generic_parts(V);
  hipStream_t s = (hipStream_t)stream;
  Control* ctl = (Control*)workspace;

  // Greedy chains with bf16 weights (bf16 or fp32 logits) that fit the
  // persistent kernel run in one launch.
  const int cus = device_cus();
  if ((tile || f32_tile) && greedy && cus > 0 && B <= dspark::chain_max_rows() && M <= kChainMaxSteps &&
      (V + 31) / 32 <= (int64_t)cus * dspark::chain_waves_per_group()) {
    dspark::ChainParams c{};
    c.base = base_logits;
    c.out = corrected_logits;
    c.lf32 = !tile;
    c.first_prev = first_prev_token_ids;
    c.tokens = sampled_tokens;
    c.w1 = (const uint16_t*)w1;
    c.w2 = (const uint16_t*)w2;
    c.sync = (uint32_t*)((char*)workspace + kControlBytes);
    c.keys = (uint64_t*)((char*)c.sync + dspark::kChainSyncBytes);
    c.bad_rows = &ctl->bad_rows;
    c.sync_failures = &ctl->sync_failures;
    c.test_hook = &ctl->chain_test_hook;
    c.B = B;
    c.M = M;
    c.V = V;
    c.r = r;
    c.S = (V + 31) / 32;
    const hipError_t e = dspark::launch_chain_greedy(c, cus, s);
    if (e == hipSuccess) return DSPARK_OK;
    (void)hipGetLastError();  // not launchable here: take the step-by-step path
  }
  // Temperature chains with bf16 weights (bf16 or fp32 logits) that fit the
  // persistent sampling kernel, and greedy chains the greedy chain did not
  // take (more rows, or a wider vocabulary per CU): the same kernel
  // selecting without noise.
  if ((tile || f32_tile) && cus > 0 && B <= dspark::chain_sample_max_rows() &&
      M * B <= dspark::chain_sample_max_step_rows() &&
      (V + 31) / 32 <= (int64_t)cus * dspark::chain_sample_slices_per_group(!tile)) {
    dspark::ChainSampleParams c{};
    c.base = base_logits;
    c.out = corrected_logits;
    c.lf32 = !tile;
    c.first_prev = first_prev_token_ids;
    c.tokens = sampled_tokens;
    c.w1 = (const uint16_t*)w1;
    c.w2 = (const uint16_t*)w2;
    c.sync = (uint32_t*)((char*)workspace + kControlBytes);
    c.keys = (uint64_t*)((char*)c.sync + dspark::kChainSyncBytes);
    c.bad_rows = &ctl->bad_rows;
    c.sync_failures = &ctl->sync_failures;
    c.test_hook = &ctl->chain_test_hook;
    c.B = B;
    c.M = M;
    c.V = V;
    c.r = r;
    c.S = (V + 31) / 32;
    c.kappa = p.kappa;
    c.k_abs0 = (uint32_t)position_offset;
    c.batch_offset = (uint32_t)batch_offset;
    c.seed_lo = p.seed_lo;
    c.seed_hi = p.seed_hi;
    c.greedy = greedy;
    const hipError_t e = dspark::launch_chain_sample(c, cus, s);
    if (e == hipSuccess) return DSPARK_OK;
    (void)hipGetLastError();
  }
  for (int64_t k = 0; k < M; ++k) {
    p.k = k;
    p.k_abs = (uint32_t)(position_offset + k);
    hipError_t e = hipErrorNotSupported;
    if (tile || f32_tile) {
      // the persistent step kernel where the shape fits, else the tile
      // kernel (bf16 logits) or the generic one
      p.nparts = dspark::sample_step_parts(V);
      e = dspark::launch_sample_step(p, f32_tile, cus, s);
      if (e == hipErrorNotSupported && tile) {
        (void)hipGetLastError();
        p.nparts = vocab_slices(V);
        e = dspark::launch_tile(p, s);
      }
    }
    if (e == hipErrorNotSupported) {
      (void)hipGetLastError();
      if (r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
      p.nparts = dspark::generic_parts(V);
      e = dspark::launch_generic(p, logits_dtype == DSPARK_BF16, weight_dtype == DSPARK_BF16, s);
    }
    if (e != hipSuccess) return device_failure(e, "sample step launch");
    e = dspark::launch_reduce(p.partials, p.nparts, B, M, k, sampled_tokens, s);
    if (e != hipSuccess) return device_failure(e, "sample reduce launch");
  }
  return DSPARK_OK;
}

}  // namespace dspark

extern "C" {

dspark_status_t dspark_markov_sample_block(const void* base_logits, dspark_dtype_t logits_dtype,
                                           const int64_t* first_prev_token_ids, const void* w1,
                                           const void* w2, dspark_dtype_t weight_dtype,
                                           int64_t B, int64_t M, int64_t V, int64_t r,
                                           double temperature, uint64_t seed,
                                           int64_t position_offset, int64_t batch_offset,
                                           int64_t* sampled_tokens, void* corrected_logits,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  return dspark::sample_block_impl(base_logits, logits_dtype, first_prev_token_ids, w1, w2, weight_dtype, B, M,
                                   V, r, temperature, seed, position_offset, batch_offset, sampled_tokens,
                                   corrected_logits, workspace, workspace_bytes, stream, false);
}

size_t dspark_markov_gated_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r, int64_t d,
                                           int sample_mode) {
  const size_t base = align256(dspark_markov_workspace_bytes(B, M, V, r, sample_mode));
  if (B < 0 || M < 0 || V < 0 || r <= 0 || d < 0) return base;
  int64_t rows = B;
  if (!sample_mode && !mul_ok(B, M, &rows)) return SIZE_MAX;
  return add_sz(base, gated_region_bytes(rows, r, d));
}

dspark_status_t dspark_markov_apply_block_gated(
    const void* base_logits, dspark_dtype_t logits_dtype, const int64_t* token_ids,
    const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d, const void* w1,
    const void* w2, const void* gate_weight, const void* gate_bias, dspark_dtype_t weight_dtype,
    int64_t B, int64_t M, int64_t V, int64_t r, void* corrected_logits, void* latent_out,
    void* workspace, size_t workspace_bytes, void* stream) {
  int64_t elems = 0;
  dspark_status_t st = check_common(logits_dtype, weight_dtype, B, M, V, r, &elems);
  if (st != DSPARK_OK) return st;
  const bool gated = hidden_states != nullptr;
  st = check_gate_args(gated, hidden_dtype, d, gate_weight, gate_bias, B * M, r);
  if (st != DSPARK_OK) return st;
  if (elems == 0) return DSPARK_OK;
  if (!gated && !latent_out)  // the vanilla fallback
    return dspark_markov_apply_block(base_logits, logits_dtype, token_ids, w1, w2, weight_dtype, B, M, V,
                                     r, corrected_logits, workspace, workspace_bytes, stream);
  if (!base_logits || !token_ids || !w1 || !w2 || !corrected_logits) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_gated_workspace_bytes(B, M, V, r, gated ? d : 0, 0))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const int64_t rows = B * M;
  const size_t lbytes = (size_t)elems * dtype_bytes(logits_dtype);
  const size_t wbytes = (size_t)(V * r) * dtype_bytes(weight_dtype);
  const size_t ubytes = (size_t)(rows * r) * dtype_bytes(weight_dtype);
  const size_t hbytes = gated ? (size_t)(rows * d) * dtype_bytes(hidden_dtype) : 0;
  const size_t gwbytes = gated ? (size_t)(r * (d + r)) * dtype_bytes(weight_dtype) : 0;
  const size_t gbbytes = gated ? (size_t)r * dtype_bytes(weight_dtype) : 0;
  const void* ins[6] = {w1, w2, token_ids, hidden_states, gate_weight, gate_bias};
  const size_t ins_bytes[6] = {wbytes, wbytes, (size_t)rows * sizeof(int64_t), hbytes, gwbytes, gbbytes};
  if (corrected_logits != base_logits && overlaps(corrected_logits, lbytes, base_logits, lbytes))
    return DSPARK_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 6; ++i) {
    if (overlaps(corrected_logits, lbytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
    if (latent_out && overlaps(latent_out, ubytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
  }
  if (latent_out && (overlaps(latent_out, ubytes, corrected_logits, lbytes) ||
                     overlaps(latent_out, ubytes, base_logits, lbytes)))
    return DSPARK_ERR_INVALID_ARGUMENT;

  hipStream_t s = (hipStream_t)stream;
  char* const region = (char*)workspace + align256(dspark_markov_workspace_bytes(B, M, V, r, 0));
  void* const latent = latent_out ? latent_out : (void*)region;
  hipError_t e = run_gate(region, hidden_states, hidden_dtype, d, token_ids, nullptr, w1, gate_weight, gate_bias,
                          weight_dtype, rows, V, r, M, 0, latent, r, dspark::MODE_APPLY, gated, s);
  if (e != hipSuccess) return device_failure(e, "gate launch");

  dspark::KernelParams p{};
  p.base = base_logits;
  p.out = corrected_logits;
  p.ids = token_ids;
  p.w1 = w1;
  p.w2 = w2;
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.sink = (char*)workspace + kDataOffset;
  p.latent = latent;
  p.latent_ld = r;
  p.rows = rows;
  p.V = V;
  p.r = r;
  p.M = M;
  p.mode = dspark::MODE_APPLY;
  // bf16 weights: the grouped kernel (rows in their own order, one
  // launch per block of rows the kernel takes); otherwise the generic one
  const bool fast = tile_path(DSPARK_BF16, weight_dtype, V, r, base_logits, corrected_logits, w1, w2) &&
                    aligned16(latent);
  if (fast) {
    const size_t lb = dtype_bytes(logits_dtype);
    int64_t blk = dspark::kGroupedApplyMaxRows;
    const int64_t fit = ((int64_t)1 << 31) / (V * (int64_t)lb);
    if (fit < blk) blk = fit;
    for (int64_t off = 0; off < rows && blk > 0; off += blk) {
      dspark::KernelParams q = p;
      q.rows = rows - off < blk ? rows - off : blk;
      q.base = (const char*)base_logits + (size_t)(off * V) * lb;
      q.out = (char*)corrected_logits + (size_t)(off * V) * lb;
      q.ids = token_ids + off;
      q.latent = (const char*)latent + (size_t)(off * r) * 2;
      e = dspark::launch_apply_grouped(q, logits_dtype == DSPARK_F32, s);
      if (e == hipErrorNotSupported) {
        (void)hipGetLastError();
        e = dspark::launch_generic(q, logits_dtype == DSPARK_BF16, true, s);
      }
      if (e != hipSuccess) return device_failure(e, "gated apply launch");
    }
    if (blk > 0) return DSPARK_OK;
  }
  if (r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
  e = dspark::launch_generic(p, logits_dtype == DSPARK_BF16, weight_dtype == DSPARK_BF16, s);
  if (e != hipSuccess) return device_failure(e, "gated apply launch");
  return DSPARK_OK;
}

dspark_status_t dspark_markov_sample_block_gated(
    const void* base_logits, dspark_dtype_t logits_dtype, const int64_t* first_prev_token_ids,
    const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d, const void* w1,
    const void* w2, const void* gate_weight, const void* gate_bias, dspark_dtype_t weight_dtype,
    int64_t B, int64_t M, int64_t V, int64_t r, double temperature, uint64_t seed,
    int64_t position_offset, int64_t batch_offset, int64_t* sampled_tokens,
    void* corrected_logits, void* latent_out, void* workspace, size_t workspace_bytes,
    void* stream) {
  int64_t elems = 0;
  dspark_status_t st = check_common(logits_dtype, weight_dtype, B, M, V, r, &elems);
  if (st != DSPARK_OK) return st;
  if (std::isnan(temperature)) return DSPARK_ERR_INVALID_ARGUMENT;
  const bool gated = hidden_states != nullptr;
  st = check_gate_args(gated, hidden_dtype, d, gate_weight, gate_bias, B * M, r);
  if (st != DSPARK_OK) return st;
  if (B == 0 || M == 0) return DSPARK_OK;
  if (V == 0) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!gated && !latent_out)  // the vanilla fallback
    return dspark_markov_sample_block(base_logits, logits_dtype, first_prev_token_ids, w1, w2, weight_dtype,
                                      B, M, V, r, temperature, seed, position_offset, batch_offset,
                                      sampled_tokens, corrected_logits, workspace, workspace_bytes, stream);
  if (!base_logits || !first_prev_token_ids || !w1 || !w2 || !sampled_tokens)
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_gated_workspace_bytes(B, M, V, r, gated ? d : 0, 1))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const size_t lbytes = (size_t)elems * dtype_bytes(logits_dtype);
  const size_t wbytes = (size_t)(V * r) * dtype_bytes(weight_dtype);
  const size_t tbytes = (size_t)(B * M) * sizeof(int64_t);
  const size_t ubytes = (size_t)(B * M * r) * dtype_bytes(weight_dtype);
  const size_t hbytes = gated ? (size_t)(B * M * d) * dtype_bytes(hidden_dtype) : 0;
  const size_t gwbytes = gated ? (size_t)(r * (d + r)) * dtype_bytes(weight_dtype) : 0;
  const size_t gbbytes = gated ? (size_t)r * dtype_bytes(weight_dtype) : 0;
  const void* ins[7] = {base_logits, w1, w2, first_prev_token_ids, hidden_states, gate_weight, gate_bias};
  const size_t ins_bytes[7] = {lbytes, wbytes, wbytes, (size_t)B * sizeof(int64_t), hbytes, gwbytes, gbbytes};
  for (int i = 0; i < 7; ++i) {
    if (overlaps(sampled_tokens, tbytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
    if (corrected_logits && overlaps(corrected_logits, lbytes, ins[i], ins_bytes[i]))
      return DSPARK_ERR_INVALID_ARGUMENT;
    if (latent_out && overlaps(latent_out, ubytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
  }
  if (corrected_logits && overlaps(corrected_logits, lbytes, sampled_tokens, tbytes))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (latent_out && (overlaps(latent_out, ubytes, sampled_tokens, tbytes) ||
                     (corrected_logits && overlaps(latent_out, ubytes, corrected_logits, lbytes))))
    return DSPARK_ERR_INVALID_ARGUMENT;

  const bool greedy = temperature < 1e-5;
  hipStream_t s = (hipStream_t)stream;
  char* const region = (char*)workspace + align256(dspark_markov_workspace_bytes(B, M, V, r, 1));
  dspark::KernelParams p{};
  p.base = base_logits;
  p.out = corrected_logits;
  p.ids = first_prev_token_ids;
  p.tokens = sampled_tokens;
  p.w1 = w1;
  p.w2 = w2;
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.partials = (uint64_t*)((char*)workspace + kDataOffset);
  p.rows = B;
  p.V = V;
  p.r = r;
  p.M = M;
  p.batch_offset = batch_offset;
  p.mode = greedy ? dspark::MODE_GREEDY : dspark::MODE_TEMPERATURE;
  p.kappa = greedy ? 0.0f : (float)(1.4426950408889634 / temperature);
  p.seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
  p.seed_hi = (uint32_t)(seed >> 32);
  // each step's latent rows: straight into latent_out[:, k, :], else a scratch [B, r]
  const int64_t lld = latent_out ? M * r : r;
  const bool lat_ok = latent_out == nullptr || aligned16(latent_out);
  const bool tile = tile_path(logits_dtype, weight_dtype, V, r, base_logits, corrected_logits, w1, w2) && lat_ok;
  const bool f32_tile = logits_dtype == DSPARK_F32 && lat_ok &&
                        tile_path(DSPARK_BF16, weight_dtype, V, r, base_logits, corrected_logits, w1, w2);
  if (!tile && !f32_tile && r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
  const int cus = device_cus();
  for (int64_t k = 0; k < M; ++k) {
    void* const latent = latent_out ? (void*)((char*)latent_out + (size_t)(k * r) * dtype_bytes(weight_dtype))
                                    : (void*)region;
    hipError_t e = run_gate(region, hidden_states, hidden_dtype, d, first_prev_token_ids, sampled_tokens, w1, gate_weight,
                            gate_bias, weight_dtype, B, V, r, M, k, latent, lld, p.mode, gated, s);
    if (e != hipSuccess) return device_failure(e, "gate launch");
    p.k = k;
    p.k_abs = (uint32_t)(position_offset + k);
    p.latent = latent;
    p.latent_ld = lld;
    e = hipErrorNotSupported;
    if (tile || f32_tile) {
      p.nparts = dspark::sample_step_parts(V);
      e = dspark::launch_sample_step(p, f32_tile, cus, s);
      if (e == hipErrorNotSupported) (void)hipGetLastError();
    }
    if (e == hipErrorNotSupported) {
      if (r > kGenericMaxRank) return DSPARK_ERR_UNSUPPORTED;
      p.nparts = dspark::generic_parts(V);
      e = dspark::launch_generic(p, logits_dtype == DSPARK_BF16, weight_dtype == DSPARK_BF16, s);
    }
    if (e != hipSuccess) return device_failure(e, "gated sample step launch");
    e = dspark::launch_reduce(p.partials, p.nparts, B, M, k, sampled_tokens, s);
    if (e != hipSuccess) return device_failure(e, "sample reduce launch");
  }
  return DSPARK_OK;
}

size_t dspark_markov_backward_workspace_bytes(int64_t B, int64_t M, int64_t V, int64_t r) {
  if (B < 0 || M < 0 || V < 0 || r <= 0) return kDataOffset;
  int64_t rows = 0, rr = 0;
  if (!mul_ok(B, M, &rows) || !mul_ok(rows, r, &rr)) return SIZE_MAX;
  int64_t sl = 0;
  const int64_t S = V > 0 ? dspark::backward_slices(V, &sl) : 0;
  const size_t de = align256(mul_sz((size_t)rr, 4));
  const size_t parts = align256(mul_sz(mul_sz((size_t)S, (size_t)rr), 4));
  return add_sz(add_sz(add_sz(kDataOffset, de), parts), align256(mul_sz((size_t)rows, 8)));
}

dspark_status_t dspark_markov_apply_block_backward(const void* grad_corrected, dspark_dtype_t logits_dtype,
                                                   const int64_t* token_ids, const void* w1, const void* w2,
                                                   dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V,
                                                   int64_t r, void* grad_w1, void* grad_w2, void* workspace,
                                                   size_t workspace_bytes, void* stream) {
  int64_t elems = 0;
  dspark_status_t st = check_common(logits_dtype, weight_dtype, B, M, V, r, &elems);
  if (st != DSPARK_OK) return st;
  if (V == 0) return DSPARK_OK;   // no parameters
  if (!w1 || !w2 || !grad_w1 || !grad_w2) return DSPARK_ERR_INVALID_ARGUMENT;
  const int64_t rows = B * M;
  if (rows > 0 && (!grad_corrected || !token_ids)) return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_backward_workspace_bytes(B, M, V, r))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const size_t lbytes = (size_t)elems * dtype_bytes(logits_dtype);
  const size_t wbytes = (size_t)(V * r) * dtype_bytes(weight_dtype);
  const void* ins[4] = {grad_corrected, token_ids, w1, w2};
  const size_t ins_bytes[4] = {lbytes, (size_t)rows * sizeof(int64_t), wbytes, wbytes};
  for (int i = 0; i < 4; ++i)
    if (overlaps(grad_w1, wbytes, ins[i], ins_bytes[i]) || overlaps(grad_w2, wbytes, ins[i], ins_bytes[i]))
      return DSPARK_ERR_INVALID_ARGUMENT;
  if (overlaps(grad_w1, wbytes, grad_w2, wbytes)) return DSPARK_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (rows == 0) {   // no rows: both gradients are zero
    e = dspark::launch_fill_zero(grad_w1, wbytes, s);
    if (e == hipSuccess) e = dspark::launch_fill_zero(grad_w2, wbytes, s);
    if (e != hipSuccess) return device_failure(e, "backward fill");
    return DSPARK_OK;
  }
  dspark::BwdParams p{};
  p.grad = grad_corrected;
  p.ids = token_ids;
  p.w1 = w1;
  p.w2 = w2;
  p.dw1 = grad_w1;
  p.dw2 = grad_w2;
  char* const region = (char*)workspace + kDataOffset;
  p.de = region;
  p.S = dspark::backward_slices(V, &p.SL);
  p.partials = (float*)(region + align256((size_t)(rows * r) * 4));
  p.link = (int32_t*)((char*)p.partials + align256((size_t)p.S * (size_t)(rows * r) * 4));
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.rows = rows;
  p.V = V;
  p.r = r;
  e = dspark::launch_backward(p, logits_dtype == DSPARK_BF16, weight_dtype == DSPARK_BF16, s);
  if (e != hipSuccess) return device_failure(e, "backward launch");
  return DSPARK_OK;
}

dspark_status_t dspark_markov_apply_block_lm_head(const void* hidden_states, dspark_dtype_t hidden_dtype, int64_t d,
                                                  const void* lm_head_weight, dspark_dtype_t lm_head_dtype,
                                                  const int64_t* token_ids, const void* w1, const void* w2,
                                                  dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V,
                                                  int64_t r, float* corrected_logits, void* workspace,
                                                  size_t workspace_bytes, void* stream) {
  if (!known_dtype(hidden_dtype) || !known_dtype(lm_head_dtype) || !known_dtype(weight_dtype))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (B < 0 || M < 0 || V < 0 || r <= 0 || d <= 0) return DSPARK_ERR_INVALID_ARGUMENT;
  int64_t rows = 0, elems = 0, t = 0;
  if (!mul_ok(B, M, &rows) || !mul_ok(rows, V, &elems) || !mul_ok(V, r, &t) || !mul_ok(V, d, &t) ||
      !mul_ok(rows, d, &t))
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (elems == 0) return DSPARK_OK;
  if (!hidden_states || !lm_head_weight || !token_ids || !w1 || !w2 || !corrected_logits)
    return DSPARK_ERR_INVALID_ARGUMENT;
  if (!workspace || workspace_bytes < dspark_markov_workspace_bytes(B, M, V, r, 0))
    return DSPARK_ERR_WORKSPACE_TOO_SMALL;
  const size_t obytes = (size_t)elems * 4;
  const void* ins[5] = {hidden_states, lm_head_weight, token_ids, w1, w2};
  const size_t ins_bytes[5] = {(size_t)(rows * d) * dtype_bytes(hidden_dtype), (size_t)(V * d) * dtype_bytes(lm_head_dtype),
                               (size_t)rows * sizeof(int64_t), (size_t)(V * r) * dtype_bytes(weight_dtype),
                               (size_t)(V * r) * dtype_bytes(weight_dtype)};
  for (int i = 0; i < 5; ++i)
    if (overlaps(corrected_logits, obytes, ins[i], ins_bytes[i])) return DSPARK_ERR_INVALID_ARGUMENT;
  // the matrix-core kernel takes bf16 operands, sizes in multiples of 8 and
  // 16-byte aligned buffers
  if (hidden_dtype != DSPARK_BF16 || lm_head_dtype != DSPARK_BF16 || weight_dtype != DSPARK_BF16 || d % 8 ||
      r % 8 || V % 8 || !aligned16(hidden_states) || !aligned16(lm_head_weight) || !aligned16(w1) ||
      !aligned16(w2) || !aligned16(corrected_logits)) {
    g_last_error = "apply_block_lm_head: bf16 hidden states, head and Markov weights, d, r and V multiples of 8 "
                   "and 16-byte aligned buffers";
    return DSPARK_ERR_UNSUPPORTED;
  }
  dspark::LmHeadParams p{};
  p.hidden = hidden_states;
  p.lm = lm_head_weight;
  p.ids = token_ids;
  p.w1 = w1;
  p.w2 = w2;
  p.out = corrected_logits;
  p.bad_rows = &((Control*)workspace)->bad_rows;
  p.rows = rows;
  p.V = V;
  p.r = r;
  p.d = d;
  const hipError_t e = dspark::launch_lm_head(p, device_cus(), (hipStream_t)stream);
  if (e == hipErrorNotSupported) {
    (void)hipGetLastError();
    g_last_error = "apply_block_lm_head: every buffer must fit in 2^31 bytes";
    return DSPARK_ERR_UNSUPPORTED;
  }
  if (e != hipSuccess) return device_failure(e, "lm head launch");
  return DSPARK_OK;
}

dspark_status_t dspark_markov_read_device_error(void* workspace, void* stream, int64_t* bad_rows) {
  if (!workspace || !bad_rows) return DSPARK_ERR_INVALID_ARGUMENT;
  hipStream_t s = (hipStream_t)stream;
  Control c{};
  hipError_t e = hipMemcpyAsync(&c, workspace, sizeof(c), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_failure(e, "read device error");
  *bad_rows = (int64_t)c.bad_rows;
  // clear the error words; the test hook (third line) stays as the caller set it
  e = dspark::launch_fill_zero(workspace, offsetof(Control, chain_test_hook), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_failure(e, "clear device error");
  if (c.sync_failures != 0) {
    g_last_error = "the persistent chain timed out waiting for its workgroups and returned -1 tokens; "
                   "the failure count is now cleared";
    return DSPARK_ERR_DEVICE;
  }
  return DSPARK_OK;
}

const char* dspark_status_string(dspark_status_t status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_INVALID_ARGUMENT: return "invalid argument";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported dtype pair or shape";
    case DSPARK_ERR_WORKSPACE_TOO_SMALL: return "workspace missing or too small";
    case DSPARK_ERR_DEVICE: return "HIP runtime failure";
  }
  return "unknown status";
}

const char* dspark_markov_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
