// wq_tile.hip -- conversion between the plain NVFP4 / FP8-row layouts and
// the tiled layouts that wq's kernels stream fastest (a load-time, untimed
// step).
//
// The crit-hub engine card "mtp7-device-confidence" (section "Design", row
// "Weights") keeps its NVFP4 scales in a swizzled tile order chosen for its
// kernels; this is the CDNA4 counterpart.  The tiled form holds exactly the
// same bytes, permuted, so tile followed by untile is the identity.
//
// Tiled layout, for T = ceil(M/16) row tiles and S = ceil(K/256) steps:
// block (t, s), at byte (t*S + s)*2304, describes rows 16t..16t+15 and
// k = 256s .. 256s+255 (rows >= M and k >= K read as zero codes and zero
// scales).  Within a block:
//   bytes [1024h + 16l + 4j, +4), h = 0..1, lane l = c + 16g (c = 0..15,
//     g = 0..3), j = 0..3: plain code bytes [128s + 64h + 16j + 4g, +4) of
//     row 16t + c (eight E2M1 codes, low nibble first);
//   bytes [2048 + 8(16p + c) + 4h + j], p = 0..1: the E4M3 scale of row
//     16t + c for block 16s + 8h + 2j + p.
//
// Tiled FP8-row layout, for T = ceil(M/16) row tiles and S = ceil(K/128)
// steps: block (t, s), at byte (t*S + s)*2048, holds rows 16t..16t+15 and
// k = 128s .. 128s+127 (rows >= M and k >= K read as zero bytes):
//   bytes [1024h + 16l, +16), h = 0..1, lane l = c + 16g: plain bytes
//     [128s + 64h + 16g, +16) of row 16t + c.
// The row scales stay a separate FP32 array.
//
// Gate/up layout of a chained MLP layer (wq_nvfp4_tile_glu): the tiled NVFP4
// layout of a 2F-row matrix whose tile t holds gate rows 8t..8t+7 in rows
// 0..7 and up rows 8t..8t+7 in rows 8..15, so that each tile's epilogue
// finds both inputs of the gated unit for the same eight outputs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kTileThreads = 256;

// One thread per (tile, step, lane): 32 code bytes and 8 scale bytes.  With
// codes1 set, M = 2F rows are interleaved from two F-row matrices (codes,
// scales: gate; codes1, scales1: up) as described above.
__global__ __launch_bounds__(kTileThreads) void tile_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales,
                                                            const uint8_t* __restrict__ codes1,
                                                            const uint8_t* __restrict__ scales1, int M, int K,
                                                            uint8_t* __restrict__ tiled, int64_t slots) {
  const int64_t id = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (id >= slots) return;
  const int S = (K + kTileStepK - 1) / kTileStepK;
  const int l = (int)(id & 63);
  const int64_t ts = id >> 6;
  const int s = (int)(ts % S);
  const int64_t t = ts / S;
  const int c = l & 15, g = l >> 4;
  int64_t row = t * kTileRows + c;
  int64_t rows = M;
  if (codes1) {
    row = t * (kTileRows / 2) + (c & 7);
    rows = M / 2;
    if (c >= 8) {
      codes = codes1;
      scales = scales1;
    }
  }
  const int64_t rowb = K / 2, srowb = K / 16;
  uint8_t* blk = tiled + ts * kTileBlockBytes;
  for (int h = 0; h < 2; ++h) {
    uint32_t w[4];
    for (int j = 0; j < 4; ++j) {
      const int64_t b0 = (int64_t)128 * s + 64 * h + 16 * j + 4 * g;  // first code byte in the row
      uint32_t v = 0;
      if (row < rows && b0 < rowb) v = *reinterpret_cast<const uint32_t*>(codes + row * rowb + b0);
      w[j] = v;
    }
    *reinterpret_cast<uint4*>(blk + 1024 * h + 16 * l) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  // the 8 scale bytes of entry (p = l / 32, c) are written by the lanes with g even
  if ((g & 1) == 0) {
    const int p = l >> 5;
    uint32_t sv[2] = {0u, 0u};
    for (int h = 0; h < 2; ++h)
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)16 * s + 8 * h + 2 * j + p;
        const uint32_t b = (row < rows && col < srowb) ? scales[row * srowb + col] : 0u;
        sv[h] |= b << (8 * j);
      }
    *reinterpret_cast<uint2*>(blk + kTileCodeBytes + 8 * (16 * p + c)) = make_uint2(sv[0], sv[1]);
  }
}

__global__ __launch_bounds__(kTileThreads) void untile_kernel(const uint8_t* __restrict__ tiled, int M, int K,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int64_t slots) {
  const int64_t id = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (id >= slots) return;
  const int S = (K + kTileStepK - 1) / kTileStepK;
  const int l = (int)(id & 63);
  const int64_t ts = id >> 6;
  const int s = (int)(ts % S);
  const int64_t t = ts / S;
  const int c = l & 15, g = l >> 4;
  const int64_t row = t * kTileRows + c;
  if (row >= M) return;
  const int64_t rowb = K / 2, srowb = K / 16;
  const uint8_t* blk = tiled + ts * kTileBlockBytes;
  for (int h = 0; h < 2; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(blk + 1024 * h + 16 * l);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    for (int j = 0; j < 4; ++j) {
      const int64_t b0 = (int64_t)128 * s + 64 * h + 16 * j + 4 * g;
      if (b0 < rowb) *reinterpret_cast<uint32_t*>(codes + row * rowb + b0) = w[j];
    }
  }
  if ((g & 1) == 0) {
    const int p = l >> 5;
    const uint2 sv = *reinterpret_cast<const uint2*>(blk + kTileCodeBytes + 8 * (16 * p + c));
    const uint32_t sw[2] = {sv.x, sv.y};
    for (int h = 0; h < 2; ++h)
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)16 * s + 8 * h + 2 * j + p;
        if (col < srowb) scales[row * srowb + col] = (uint8_t)(sw[h] >> (8 * j));
      }
  }
}

// One thread per (tile, step, lane): two 16-byte pieces of one row.
__global__ __launch_bounds__(kTileThreads) void fp8_tile_kernel(const uint8_t* __restrict__ w, int M, int K,
                                                                uint8_t* __restrict__ tiled, int64_t slots) {
  const int64_t id = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (id >= slots) return;
  const int S = (K + kFp8TileStepK - 1) / kFp8TileStepK;
  const int l = (int)(id & 63);
  const int64_t ts = id >> 6;
  const int s = (int)(ts % S);
  const int64_t t = ts / S;
  const int c = l & 15, g = l >> 4;
  const int64_t row = t * kTileRows + c;
  uint8_t* blk = tiled + ts * kFp8TileBlockBytes;
  for (int h = 0; h < 2; ++h) {
    const int64_t k = (int64_t)kFp8TileStepK * s + 64 * h + 16 * g;  // K % 16 == 0: a piece is all in or all out
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < M && k < K) v = *reinterpret_cast<const uint4*>(w + row * K + k);
    *reinterpret_cast<uint4*>(blk + 1024 * h + 16 * l) = v;
  }
}

__global__ __launch_bounds__(kTileThreads) void fp8_untile_kernel(const uint8_t* __restrict__ tiled, int M, int K,
                                                                  uint8_t* __restrict__ w, int64_t slots) {
  const int64_t id = (int64_t)blockIdx.x * kTileThreads + threadIdx.x;
  if (id >= slots) return;
  const int S = (K + kFp8TileStepK - 1) / kFp8TileStepK;
  const int l = (int)(id & 63);
  const int64_t ts = id >> 6;
  const int s = (int)(ts % S);
  const int64_t t = ts / S;
  const int c = l & 15, g = l >> 4;
  const int64_t row = t * kTileRows + c;
  if (row >= M) return;
  const uint8_t* blk = tiled + ts * kFp8TileBlockBytes;
  for (int h = 0; h < 2; ++h) {
    const int64_t k = (int64_t)kFp8TileStepK * s + 64 * h + 16 * g;
    if (k < K) *reinterpret_cast<uint4*>(w + row * K + k) = *reinterpret_cast<const uint4*>(blk + 1024 * h + 16 * l);
  }
}

bool fp8_shape_ok(int M, int K) {
  return M >= 1 && K >= 16 && K % 16 == 0 && K <= (1 << 24) && (uint64_t)M * (uint64_t)K < (1ull << 40);
}

int64_t fp8_tile_slots(int M, int K) {
  return (int64_t)((M + kTileRows - 1) / kTileRows) * ((K + kFp8TileStepK - 1) / kFp8TileStepK) * 64;
}

bool shape_ok(int M, int K) {
  return M >= 1 && K >= 32 && K % 32 == 0 && K <= (1 << 24) && (uint64_t)M * (uint64_t)(K / 2) < (1ull << 40);
}

int64_t tile_slots(int M, int K) {
  return (int64_t)((M + kTileRows - 1) / kTileRows) * ((K + kTileStepK - 1) / kTileStepK) * 64;
}

}  // namespace
}  // namespace wq

extern "C" {

size_t wq_nvfp4_tiled_bytes(int M, int K) {
  if (!wq::shape_ok(M, K)) return 0;
  return (size_t)(wq::tile_slots(M, K) / 64) * wq::kTileBlockBytes;
}

wq_status wq_nvfp4_tile(const uint8_t* codes, const uint8_t* scales, int M, int K, uint8_t* tiled, void* stream) {
  if (!codes || !scales || !tiled) return WQ_ERROR_INVALID_VALUE;
  if (M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (!wq::shape_ok(M, K)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)codes & 15u) || ((uintptr_t)scales & 15u) || ((uintptr_t)tiled & 15u)) return WQ_ERROR_MISALIGNED;
  const int64_t slots = wq::tile_slots(M, K);
  const int grid = (int)((slots + wq::kTileThreads - 1) / wq::kTileThreads);
  hipLaunchKernelGGL(wq::tile_kernel, dim3(grid), dim3(wq::kTileThreads), 0, static_cast<hipStream_t>(stream), codes,
                     scales, nullptr, nullptr, M, K, tiled, slots);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_nvfp4_tile_glu(const uint8_t* gate_codes, const uint8_t* gate_scales, const uint8_t* up_codes,
                            const uint8_t* up_scales, int F, int K, uint8_t* tiled, void* stream) {
  if (!gate_codes || !gate_scales || !up_codes || !up_scales || !tiled) return WQ_ERROR_INVALID_VALUE;
  if (F < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (F % 8 != 0 || F > (1 << 29) || !wq::shape_ok(2 * F, K)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)gate_codes & 15u) || ((uintptr_t)gate_scales & 15u) || ((uintptr_t)up_codes & 15u) ||
      ((uintptr_t)up_scales & 15u) || ((uintptr_t)tiled & 15u))
    return WQ_ERROR_MISALIGNED;
  const int64_t slots = wq::tile_slots(2 * F, K);
  const int grid = (int)((slots + wq::kTileThreads - 1) / wq::kTileThreads);
  hipLaunchKernelGGL(wq::tile_kernel, dim3(grid), dim3(wq::kTileThreads), 0, static_cast<hipStream_t>(stream),
                     gate_codes, gate_scales, up_codes, up_scales, 2 * F, K, tiled, slots);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_nvfp4_untile(const uint8_t* tiled, int M, int K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (!codes || !scales || !tiled) return WQ_ERROR_INVALID_VALUE;
  if (M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (!wq::shape_ok(M, K)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)codes & 15u) || ((uintptr_t)scales & 15u) || ((uintptr_t)tiled & 15u)) return WQ_ERROR_MISALIGNED;
  const int64_t slots = wq::tile_slots(M, K);
  const int grid = (int)((slots + wq::kTileThreads - 1) / wq::kTileThreads);
  hipLaunchKernelGGL(wq::untile_kernel, dim3(grid), dim3(wq::kTileThreads), 0, static_cast<hipStream_t>(stream), tiled,
                     M, K, codes, scales, slots);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

size_t wq_fp8_tiled_bytes(int M, int K) {
  if (!wq::fp8_shape_ok(M, K)) return 0;
  return (size_t)(wq::fp8_tile_slots(M, K) / 64) * wq::kFp8TileBlockBytes;
}

wq_status wq_fp8_tile(const uint8_t* w, int M, int K, uint8_t* tiled, void* stream) {
  if (!w || !tiled) return WQ_ERROR_INVALID_VALUE;
  if (M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (!wq::fp8_shape_ok(M, K)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)w & 15u) || ((uintptr_t)tiled & 15u)) return WQ_ERROR_MISALIGNED;
  const int64_t slots = wq::fp8_tile_slots(M, K);
  const int grid = (int)((slots + wq::kTileThreads - 1) / wq::kTileThreads);
  hipLaunchKernelGGL(wq::fp8_tile_kernel, dim3(grid), dim3(wq::kTileThreads), 0, static_cast<hipStream_t>(stream), w,
                     M, K, tiled, slots);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_fp8_untile(const uint8_t* tiled, int M, int K, uint8_t* w, void* stream) {
  if (!w || !tiled) return WQ_ERROR_INVALID_VALUE;
  if (M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (!wq::fp8_shape_ok(M, K)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (((uintptr_t)w & 15u) || ((uintptr_t)tiled & 15u)) return WQ_ERROR_MISALIGNED;
  const int64_t slots = wq::fp8_tile_slots(M, K);
  const int grid = (int)((slots + wq::kTileThreads - 1) / wq::kTileThreads);
  hipLaunchKernelGGL(wq::fp8_untile_kernel, dim3(grid), dim3(wq::kTileThreads), 0, static_cast<hipStream_t>(stream),
                     tiled, M, K, w, slots);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

}  // extern "C"
