// A plain streaming read (the read-stream ceiling the KV-read rates are
// quoted against).  Nothing of the method is computed here.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "verify_probe.h"

namespace va_probe_detail {

constexpr int kBlocks = 1024, kThreads = 256, kUnroll = 4;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const uint4 *src, size_t n16, uint32_t *sink) {
  const size_t stride = (size_t)kBlocks * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;  // keeps the loads; almost never taken
}

}  // namespace va_probe_detail

extern "C" va_status va_read_probe(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  if (!src || !sink || ((uintptr_t)src & 15u) || (bytes & 15u)) return VA_ERR_INVALID;
  if (bytes == 0) return VA_OK;
  hipLaunchKernelGGL(va_probe_detail::read_probe_kernel, dim3(va_probe_detail::kBlocks),
                     dim3(va_probe_detail::kThreads), 0, stream, (const uint4 *)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? VA_OK : VA_ERR_HIP;
}
