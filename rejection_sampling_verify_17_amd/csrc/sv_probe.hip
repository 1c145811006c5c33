// Measurement aids beside the verification kernels: a plain read stream (the
// bandwidth a simple kernel reaches on this GPU, the context the verification
// kernels' rates are read against) and the device arithmetic the samplers and
// statistics rely on, evaluated on caller inputs so a test can compare it with
// an fp64 host reference.  Declared in include/specverify.h.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "specverify.h"
#include "sv_device.h"

namespace {

using sv::u32x4;

constexpr int kProbeThreads = 256;
constexpr int kProbeU = 4;  // 16-byte loads in flight per thread

// Each block reads a contiguous slab of the buffer (16-byte vectors, kProbeU
// in flight per thread) and folds it into one float, written per block so the
// loads cannot be dropped.  Vectors past the buffer are not read.  NT: loads
// with the non-temporal hint (no allocation for reuse in the caches).
template <bool NT>
__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4 *x, long long n16, float *out) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long lo = per * blockIdx.x;
  const long long hi = lo + per < n16 ? lo + per : n16;
  float s = 0.0f;
  for (long long i = lo + threadIdx.x; i < hi; i += (long long)kProbeThreads * kProbeU) {
    u32x4 a[kProbeU];
#pragma unroll
    for (int u = 0; u < kProbeU; ++u) {
      const long long k = i + (long long)u * kProbeThreads;
      if (NT) a[u] = k < hi ? __builtin_nontemporal_load(x + k) : u32x4{0u, 0u, 0u, 0u};
      else a[u] = k < hi ? x[k] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kProbeU; ++u)
      s += __uint_as_float(a[u].x) + __uint_as_float(a[u].y) + __uint_as_float(a[u].z) + __uint_as_float(a[u].w);
  }
  s = sv::wave_sum_f(s);
  __shared__ float red[kProbeThreads / sv::kWave];
  if (threadIdx.x % sv::kWave == 0) red[threadIdx.x / sv::kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.0f;
    for (int w = 0; w < kProbeThreads / sv::kWave; ++w) t += red[w];
    out[blockIdx.x] = t;
  }
}

// out[i] = the sampler's exponential variate (base 2) of Philox word
// (first + i) << 9, i.e. of U = (2 (first + i) + 1) 2^-24.
__global__ __launch_bounds__(kProbeThreads) void k_probe_variates(uint32_t first, int n, float *out) {
  const int i = blockIdx.x * kProbeThreads + threadIdx.x;
  if (i < n) out[i] = sv::exp2_variate((first + (uint32_t)i) << 9);
}

// out[i] = native exp2 (op 0) or log2 (op 1) of x[i].
__global__ __launch_bounds__(kProbeThreads) void k_probe_math(const float *x, int n, int op, float *out) {
  const int i = blockIdx.x * kProbeThreads + threadIdx.x;
  if (i < n) out[i] = op == 0 ? __builtin_amdgcn_exp2f(x[i]) : __builtin_amdgcn_logf(x[i]);
}

}  // namespace

extern "C" {

sv_status sv_probe_read(const void *x, size_t bytes, float *out, int32_t grid, int32_t nontemporal, void *stream) {
  if (!x || !out || grid < 1 || bytes < 16 || ((uintptr_t)x % 16) || ((uintptr_t)out % 4)) return SV_EINVAL;
  (void)hipGetLastError();
  if (nontemporal)
    hipLaunchKernelGGL(k_probe_read<true>, dim3((unsigned)grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (long long)(bytes / 16), out);
  else
    hipLaunchKernelGGL(k_probe_read<false>, dim3((unsigned)grid), dim3(kProbeThreads), 0, (hipStream_t)stream,
                       (const u32x4 *)x, (long long)(bytes / 16), out);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_probe_variates(uint32_t first, int32_t n, float *out, void *stream) {
  if (!out || n < 1 || (uint64_t)first + (uint64_t)n > (1ull << 23) || ((uintptr_t)out % 4)) return SV_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_probe_variates, dim3((unsigned)((n + kProbeThreads - 1) / kProbeThreads)),
                     dim3(kProbeThreads), 0, (hipStream_t)stream, first, n, out);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

sv_status sv_probe_math(const float *x, int32_t n, int32_t op, float *out, void *stream) {
  if (!x || !out || n < 1 || (op != 0 && op != 1) || ((uintptr_t)x % 4) || ((uintptr_t)out % 4)) return SV_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_probe_math, dim3((unsigned)((n + kProbeThreads - 1) / kProbeThreads)), dim3(kProbeThreads),
                     0, (hipStream_t)stream, x, n, op, out);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

}  // extern "C"
