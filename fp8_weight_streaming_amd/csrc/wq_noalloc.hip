// wq_noalloc.hip -- wq_gemm_nvfp4_tiled_noalloc: the tiled NVFP4 product with
// its split-K scratch in a static device buffer, for callers that cannot
// allocate device memory.
//
// The buffer is a file-scope __device__ array.  Its name in host code is only
// a host-side stand-in, so the device address is looked up once per device
// (hipGetSymbolAddress, on the first call with that device current) and that
// address, never the name, is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "wq.h"
#include "wq_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[WQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null until looked up)
std::mutex g_scratch_mu;

// The current device's copy of the buffer, looked up on the first call.
wq_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return WQ_ERROR_DEVICE;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WQ_ERROR_DEVICE;
    g_scratch[dev] = p;
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
  void* ws = nullptr;
  const wq_status sd = scratch_on_current_device(&ws);
  if (sd != WQ_SUCCESS) return sd;
  const size_t need = wq_gemm_workspace_bytes(wq::kFmtNvfp4Tiled, M, K, N);
  if (need > (size_t)WQ_NOALLOC_SCRATCH_BYTES) return WQ_ERROR_SCRATCH_LIMIT;
  // the partial sums need no initialization: every chunk's plane is written
  // before the reduction reads it
  return wq_gemm_nvfp4_tiled(tiled, global_scale, x, y, M, K, N, need ? ws : nullptr, need ? need : 0, stream);
}
