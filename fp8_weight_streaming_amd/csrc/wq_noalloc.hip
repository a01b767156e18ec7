// wq_noalloc.hip -- wq_gemm_nvfp4_tiled_noalloc: the tiled NVFP4 product with
// its split-K scratch in a static device buffer, for callers that cannot
// allocate device memory.
//
// The buffer is a file-scope __device__ array.  Its name in host code is only
// a host-side stand-in, so the device address is looked up once per device
// (hipGetSymbolAddress, on the first call with that device current) and that
// address, never the name, is what the kernels receive.  The split-tile
// kernel's arrival counters at the start of the buffer must be zero before
// its first use; the first call on each device clears them with a small fill
// kernel on the caller's stream, and every product leaves them zero again.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wq.h"
#include "wq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[WQ_NOALLOC_SCRATCH_BYTES];
static_assert(wq::kSplitCounterBytes < WQ_NOALLOC_SCRATCH_BYTES, "the counters fit the buffer");

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null until looked up)
bool g_cleared[kMaxDevices];   // counters cleared on that device
std::mutex g_scratch_mu;

constexpr int kClearThreads = 256;

__global__ __launch_bounds__(kClearThreads) void clear_kernel(uint32_t* __restrict__ p, uint32_t n) {
  for (uint32_t i = blockIdx.x * kClearThreads + threadIdx.x; i < n; i += gridDim.x * kClearThreads) p[i] = 0u;
}

// The current device's copy of the buffer, looked up on the first call,
// whose counters the first call also clears (on `stream`, before the
// product it launches there).
wq_status scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WQ_ERROR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WQ_ERROR_DEVICE;
    g_scratch[dev] = p;
  }
  if (!g_cleared[dev]) {
    constexpr uint32_t n = (uint32_t)(wq::kSplitCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(clear_kernel, dim3((n + kClearThreads - 1) / kClearThreads), dim3(kClearThreads), 0, stream,
                       static_cast<uint32_t*>(g_scratch[dev]), n);
    if (hipGetLastError() != hipSuccess) return WQ_ERROR_LAUNCH;
    g_cleared[dev] = true;
  }
  *out = g_scratch[dev];
  return WQ_SUCCESS;
}

}  // namespace

extern "C" wq_status wq_gemm_nvfp4_tiled_noalloc(const uint8_t* tiled, float global_scale, const uint16_t* x,
                                                 float* y, int M, int K, int N, void* stream) {
  // argument errors first, with no HIP call (as every other entry point)
  const wq_status st = wq::check_gemm_args(wq::kFmtNvfp4Tiled, tiled, nullptr, x, y, M, K, N);
  if (st != WQ_SUCCESS) return st;
  const size_t need = wq_gemm_workspace_bytes(wq::kFmtNvfp4Tiled, M, K, N);
  if (need > (size_t)WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERROR_SCRATCH_LIMIT;
  void* ws = nullptr;
  const wq_status sd = scratch_on_current_device(static_cast<hipStream_t>(stream), &ws);
  if (sd != WQ_SUCCESS) return sd;
  // past the counters, the buffer needs no initialization: every part is
  // written before it is read
  return wq_gemm_nvfp4_tiled(tiled, global_scale, x, y, M, K, N, need ? ws : nullptr, need ? need : 0, stream);
}
