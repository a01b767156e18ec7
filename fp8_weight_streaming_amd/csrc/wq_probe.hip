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

// The read probe runs as the weight stream does: one workgroup of 8 waves
// per CU, each wave streaming its own contiguous share of the buffer in
// whole 1 KB requests (16 bytes per lane), 8 requests in flight as a ring
// (each slot's next load issued as soon as its last one is consumed).  On
// MI355X: a grid of many small workgroups striding over the whole buffer
// read about 10% slower; batches of 8 loads consumed together 1.5% slower
// than the ring; rings of 12 or 16 the same as 8 (7.0 TB/s); default-policy
// loads 12% slower than non-temporal ones.
constexpr int kReadThreads = 512;
constexpr int kReadWaves = kReadThreads / 64;

// EVERY > 0: after each EVERY 1 KB steps, one 256-byte store (4 bytes per
// lane) to the wave's next 256 bytes of dst (slice of `slice` bytes per wave),
// written through to memory (device scope), like the verify pass's outputs.
template <bool WRITE>
__global__ __launch_bounds__(kReadThreads) void probe_read_kernel(const char* __restrict__ p, uint64_t n16,
                                                                  uint32_t* __restrict__ sink, char* __restrict__ dst,
                                                                  uint32_t slice, uint32_t every) {
  const int lane = threadIdx.x & 63;
  const uint64_t nw = (uint64_t)gridDim.x * kReadWaves;
  const uint64_t w = (uint64_t)blockIdx.x * kReadWaves + (threadIdx.x >> 6);
  const uint64_t v0 = n16 * w / nw, v1 = n16 * (w + 1) / nw;  // the wave's 16-byte vectors
  // range-checked buffer loads: offsets past the share read as zero
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p + 16 * v0), (short)0, (int)(16 * (v1 - v0)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(WRITE ? dst + (uint64_t)slice * w : nullptr, (short)0, WRITE ? (int)slice : 0,
                                        0x00020000);
  const uint32_t steps = (uint32_t)((v1 - v0 + 63) / 64);
  uint32_t acc = 0, cursor = 0;
  // (loads past the share read as zero, so the ring may run ahead of it)
  auto load = [&](uint32_t step) {
    return __builtin_bit_cast(u32x4,
                              __builtin_amdgcn_raw_buffer_load_b128(r, (int)((step * 64u + lane) * 16u), 0, 2 /* nt */));
  };
  u32x4 v[kProbeUnroll];
#pragma unroll
  for (int u = 0; u < kProbeUnroll; ++u) v[u] = load((uint32_t)u);
  for (uint32_t s = 0; s < steps; s += kProbeUnroll) {
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      v[u] = load(s + kProbeUnroll + (uint32_t)u);
    }
    if (WRITE && (s + kProbeUnroll) % every == 0) {
      __builtin_amdgcn_raw_buffer_store_b32(acc, rd, (int)(cursor + 4u * lane), 0, 16 /* sc1 */);
      cursor += 256u;
    }
  }
  // one word per thread, so the loads cannot be dropped
  sink[(uint64_t)blockIdx.x * kReadThreads + threadIdx.x] = acc;
}

// The read probes' grid and per-wave geometry.
struct ReadGeom {
  int grid = 0;
  uint64_t wave_steps = 0;  // 1 KB steps of the longest share, rounded up to the unroll
};
wq_status read_geom(size_t bytes, ReadGeom* g) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return WQ_ERROR_DEVICE;
  // one workgroup per CU (the sink holds wq_probe_sink_words() words)
  g->grid = cus < 2048 ? cus : 2048;
  const uint64_t nw = (uint64_t)g->grid * kReadWaves;
  const uint64_t share = (bytes / 16 + nw - 1) / nw;  // 16-byte vectors of the longest share
  // each wave's share (and the ring's loads up to 8 KB past it) is
  // addressed with 32-bit offsets
  if (share * 16 + 16 * 1024 >= (1ull << 31)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  g->wave_steps = ((share + 63) / 64 + kProbeUnroll - 1) / kProbeUnroll * kProbeUnroll;
  return WQ_SUCCESS;
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
  wq::ReadGeom g;
  const wq_status st = wq::read_geom(bytes, &g);
  if (st != WQ_SUCCESS) return st;
  hipLaunchKernelGGL(wq::probe_read_kernel<false>, dim3(g.grid), dim3(wq::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src), (uint64_t)(bytes / 16), sink,
                     nullptr, 0u, 0u);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

// Per wave: one 256-byte store after every `every_kb` steps of the longest
// share; shorter shares write a prefix of their slice.
static uint64_t read_write_slice(const wq::ReadGeom& g, int every_kb) {
  return g.wave_steps / (uint64_t)every_kb * 256u;
}

size_t wq_probe_read_write_bytes(size_t bytes, int every_kb) {
  if (bytes < 16 || bytes % 16 || every_kb < 8 || every_kb % 8) return 0;
  wq::ReadGeom g;
  if (wq::read_geom(bytes, &g) != WQ_SUCCESS) return 0;
  return (size_t)g.grid * wq::kReadWaves * read_write_slice(g, every_kb);
}

wq_status wq_probe_read_write(const void* src, size_t bytes, void* dst, int every_kb, uint32_t* sink, void* stream) {
  if (!src || !dst || !sink || bytes < 16 || bytes % 16 || every_kb < 8 || every_kb % 8)
    return WQ_ERROR_INVALID_VALUE;
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || ((uintptr_t)sink & 3u)) return WQ_ERROR_MISALIGNED;
  wq::ReadGeom g;
  const wq_status st = wq::read_geom(bytes, &g);
  if (st != WQ_SUCCESS) return st;
  const uint64_t slice = read_write_slice(g, every_kb);
  if (slice >= (1ull << 31)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  hipLaunchKernelGGL(wq::probe_read_kernel<true>, dim3(g.grid), dim3(wq::kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(src), (uint64_t)(bytes / 16), sink,
                     static_cast<char*>(dst), (uint32_t)slice, (uint32_t)every_kb);
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
