// dspark_static.hip -- dspark_markov_sample_block_static, the sampling entry
// point that allocates nothing (include/dspark_markov.h): it runs
// dspark_markov_sample_block's kernels on a static device array in place of
// a caller-allocated workspace.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "dspark_markov.h"
#include "markov_kernels.h"

namespace dspark {

// Defined with the rest of the ABI in dspark_markov.hip.
void set_last_error(const std::string& msg);
dspark_status_t sample_block_impl(const void* base_logits, dspark_dtype_t logits_dtype,
                                  const int64_t* first_prev_token_ids, const void* w1, const void* w2,
                                  dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V, int64_t r,
                                  double temperature, uint64_t seed, int64_t position_offset,
                                  int64_t batch_offset, int64_t* sampled_tokens, void* corrected_logits,
                                  void* workspace, size_t workspace_bytes, void* stream, bool clear_control);

}  // namespace dspark

namespace {

// A file-scope device array, one copy per GPU, used as the sampling
// workspace.  In host code `scratch` names a host-side stand-in, not the
// device copy: its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is ever passed to
// kernels or fills.
constexpr size_t kStaticScratchBytes = (size_t)4 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

dspark_status_t fail(hipError_t e, const char* what) {
  dspark::set_last_error(std::string(what) + ": " + hipGetErrorString(e));
  return DSPARK_ERR_DEVICE;
}

// Device address of this device's scratch in *out; the first call on a
// device also zero-fills it on `stream` (a kernel, no memset).
dspark_status_t static_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(e, "static scratch: current device");
  if (dev < 0 || dev >= 64) return fail(hipErrorInvalidDevice, "static scratch: current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return fail(e, "static scratch: hipGetSymbolAddress");
    if (!ptr) return fail(hipErrorInvalidSymbol, "static scratch: hipGetSymbolAddress");
    e = dspark::launch_fill_zero(ptr, kStaticScratchBytes, stream);
    if (e != hipSuccess) return fail(e, "static scratch: zero fill");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" dspark_status_t dspark_markov_sample_block_static(
    const void* base_logits, dspark_dtype_t logits_dtype, const int64_t* first_prev_token_ids, const void* w1,
    const void* w2, dspark_dtype_t weight_dtype, int64_t B, int64_t M, int64_t V, int64_t r, double temperature,
    uint64_t seed, int64_t position_offset, int64_t batch_offset, int64_t* sampled_tokens, void* corrected_logits,
    void* stream) {
  if (B > 0 && M > 0 && V >= 0 && r > 0) {
    const size_t need = dspark_markov_workspace_bytes(B, M, V, r, 1);
    if (need > kStaticScratchBytes) {
      dspark::set_last_error("sample_block_static: these sizes need " + std::to_string(need) +
                             " bytes of workspace, beyond the static scratch of " +
                             std::to_string(kStaticScratchBytes));
      return DSPARK_ERR_WORKSPACE_TOO_SMALL;
    }
  }
  void* ws = nullptr;
  if (B > 0 && M > 0) {
    const dspark_status_t st = static_scratch((hipStream_t)stream, &ws);
    if (st != DSPARK_OK) return st;
  }
  return dspark::sample_block_impl(base_logits, logits_dtype, first_prev_token_ids, w1, w2, weight_dtype, B, M, V,
                                   r, temperature, seed, position_offset, batch_offset, sampled_tokens,
                                   corrected_logits, ws, ws ? kStaticScratchBytes : 0, stream, true);
}
