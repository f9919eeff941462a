// bandwidth_probe.hip -- streaming probes that the benchmark times beside the
// head as the practical HBM ceilings of this device.  Not part of the head:
// built as its own library (libdspark_bandwidth.so), outside the C ABI of
// include/dspark_markov.h.
//
//   dspark_bandwidth_copy(dst, src, bytes, stream)
//       reads `bytes` from src and writes them to dst (1 : 1);
//   dspark_bandwidth_read_mix(dst, dst_bytes, src, src_bytes, stream)
//       writes dst_bytes to dst while reading src_bytes >= dst_bytes from src:
//       vector i of dst is the xor of src vectors i, i + n, i + 2n, ... (n =
//       dst_bytes / 16), so every byte read is used.  A src of 1.8x dst gives
//       the head's read : write mix (base logits and W2 in, corrected out).
// Both use the streaming (non-temporal) cache policy of the head's logit
// traffic, 16-byte vectors, and keep four vectors per thread in flight.
//   dspark_bandwidth_mfma(out, out_bytes, form, waves_per_cu, iters, stream)
//       the matrix-core counterpart: every wave of waves_per_cu (4, 8 or 16)
//       per CU runs `iters` rounds of eight independent bf16 products of
//       one form (0: v_mfma_f32_16x16x32_bf16, 16384 flops; 1:
//       v_mfma_f32_32x32x16_bf16, 32768 flops) and writes one float per
//       thread to out (out_bytes >= CUs * waves_per_cu * 64 * 4), so the
//       caller can time each form's throughput.
// Buffers: device memory, 16-byte aligned, sizes multiples of 16, not
// overlapping.  Returns 0, 1 for an invalid argument, 4 for a launch failure.
// Asynchronous on `stream` (a hipStream_t).
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

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

// n output vectors from m >= n source vectors; passes = ceil(m / n).
template <int PASSES>
__global__ __launch_bounds__(256) void read_mix_kernel(const u32x4_t* __restrict__ src, int64_t m,
                                                       u32x4_t* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t base = (int64_t)blockIdx.x * 1024 + threadIdx.x; base < n; base += stride) {
    u32x4_t v[4][PASSES];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int q = 0; q < PASSES; ++q) {
        const int64_t i = base + 256 * u + (int64_t)q * n;
        v[u][q] = (base + 256 * u < n && i < m) ? __builtin_nontemporal_load(src + i) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t i = base + 256 * u;
      u32x4_t x = v[u][0];
#pragma unroll
      for (int q = 1; q < PASSES; ++q) x ^= v[u][q];
      if (i < n) __builtin_nontemporal_store(x, dst + i);
    }
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// eight independent accumulators per wave, operands fixed in registers
template <int FORM>
__global__ __launch_bounds__(256) void mfma_probe_kernel(float* out, int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (float)i);
  }
  float sum = 0.0f;
  if constexpr (FORM == 0) {
    f32x4_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c) sum += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  } else {
    f32x16_t acc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[c][e];
  }
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

unsigned grid_for(int64_t n) {
  int64_t blocks = (n + 1023) / 1024;
  if (blocks > 8192) blocks = 8192;   // measured best: 4096 - 8192 workgroups of 256
  return (unsigned)blocks;
}

}  // namespace

extern "C" {

int dspark_bandwidth_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (bytes == 0) return 0;
  if (!dst || !src || !aligned16(dst) || !aligned16(src) || bytes % 16 != 0 || overlaps(dst, bytes, src, bytes))
    return 1;
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(copy_stream_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, (u32x4_t*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int dspark_bandwidth_read_mix(void* dst, size_t dst_bytes, const void* src, size_t src_bytes, void* stream) {
  if (dst_bytes == 0) return 0;
  if (!dst || !src || !aligned16(dst) || !aligned16(src) || dst_bytes % 16 != 0 || src_bytes % 16 != 0 ||
      src_bytes < dst_bytes || overlaps(dst, dst_bytes, src, src_bytes))
    return 1;
  const int64_t n = (int64_t)(dst_bytes / 16), m = (int64_t)(src_bytes / 16);
  const int64_t passes = (m + n - 1) / n;
  const dim3 grid(grid_for(n)), block(256);
  hipStream_t s = (hipStream_t)stream;
  switch (passes) {
    case 1: hipLaunchKernelGGL(read_mix_kernel<1>, grid, block, 0, s, (const u32x4_t*)src, m, (u32x4_t*)dst, n); break;
    case 2: hipLaunchKernelGGL(read_mix_kernel<2>, grid, block, 0, s, (const u32x4_t*)src, m, (u32x4_t*)dst, n); break;
    case 3: hipLaunchKernelGGL(read_mix_kernel<3>, grid, block, 0, s, (const u32x4_t*)src, m, (u32x4_t*)dst, n); break;
    case 4: hipLaunchKernelGGL(read_mix_kernel<4>, grid, block, 0, s, (const u32x4_t*)src, m, (u32x4_t*)dst, n); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int dspark_bandwidth_mfma(float* out, size_t out_bytes, int form, int waves_per_cu, int iters, void* stream) {
  if (!out || !aligned16(out) || (form != 0 && form != 1) ||
      (waves_per_cu != 4 && waves_per_cu != 8 && waves_per_cu != 16) || iters < 1)
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return 4;
  const int blocks = cus * waves_per_cu / 4;
  if (out_bytes < (size_t)blocks * 256 * sizeof(float)) return 1;
  hipStream_t s = (hipStream_t)stream;
  if (form == 0) hipLaunchKernelGGL(mfma_probe_kernel<0>, dim3(blocks), dim3(256), 0, s, out, iters);
  else hipLaunchKernelGGL(mfma_probe_kernel<1>, dim3(blocks), dim3(256), 0, s, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
