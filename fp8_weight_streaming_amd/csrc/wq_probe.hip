// wq_probe.hip -- measurement kernels: a streaming HBM read and a plain copy.
//
// The crit README (Eval: "Physics-based evaluation") and the NInfer README
// (a standalone memory-bandwidth probe) both price a kernel against the
// bandwidth the GPU actually attains.  wq_probe_read streams a buffer with
// 16-byte non-temporal loads, the same load the weight stream uses, so its
// rate is the attainable ceiling for the verify pass; wq_probe_copy reads
// and writes a buffer once each, a kernel of known traffic for scaling HBM
// byte counters.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

namespace wq {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4* __restrict__ p, uint64_t n,
                                                                   uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kProbeUnroll - 1) * stride < n; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per thread, so the loads cannot be dropped
  sink[(uint64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                                                   uint64_t n) {
  const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
  for (uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n; i += stride) d[i] = s[i];
}

}  // namespace
}  // namespace wq

extern "C" {

size_t wq_probe_sink_words(void) { return (size_t)4096 * wq::kProbeThreads; }

wq_status wq_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes < 16 || bytes % 16) return WQ_ERROR_INVALID_VALUE;
  if (((uintptr_t)src & 15u) || ((uintptr_t)sink & 3u)) return WQ_ERROR_MISALIGNED;
  hipLaunchKernelGGL(wq::probe_read_kernel, dim3(4096), dim3(wq::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const wq::u32x4*>(src), (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes < 16 || bytes % 16) return WQ_ERROR_INVALID_VALUE;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return WQ_ERROR_MISALIGNED;
  hipLaunchKernelGGL(wq::probe_copy_kernel, dim3(4096), dim3(wq::kProbeThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const wq::u32x4*>(src), static_cast<wq::u32x4*>(dst), (uint64_t)(bytes / 16));
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

}  // extern "C"
