// wq_quant.hip -- load-time round-to-nearest quantizers: BF16 weights to
// row-scaled FP8-E4M3 and to NVFP4 (E2M1 codes, E4M3 block scales, FP32
// tensor scale) on the GPU.
//
// The crit landing page (section on Models) produces FP8 and NVFP4 weights
// by post-training round-to-nearest quantization, and its Gemma case study
// re-encodes BF16 projections and the output head to FP8 at load; the
// crit-hub engine card "mtp7-device-confidence" (section "Model")
// re-encodes its draft layer as row-scaled FP8 and its head as NVFP4.
//
// FP8-row, per row:  r = fp32(max|w| / 448),  q = E4M3(fp32(w / r))
//   (a zero row gives r = 0 and q = 0).
// NVFP4, per 16 k, with the caller's tensor scale g:
//   s = E4M3(fp32(max|w| / fp32(6 g))),  d = fp32(e4m3(s) * g),
//   code = E2M1(fp32(w / d))  (all codes 0 when d = 0).
// E4M3 and E2M1 round to nearest, ties to even, onto the finite values
// (saturating at 448 and 6), keeping the sign bit of their argument.  The
// divisions are correctly rounded FP32 divisions.  Inputs must be finite.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kQuantThreads = 256;

// fp32 -> E4M3 (FN) byte, round to nearest even, saturating (finite v)
__device__ __forceinline__ uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {  // below 2^-6: steps of 2^-9 (a * 512 is exact)
    mag = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal
  } else {
    const uint32_t au = __float_as_uint(a);
    const uint32_t e = (au >> 23) - 127u + 7u;  // 1..15
    const uint32_t man = au & 0x7FFFFFu;
    uint32_t keep = man >> 20;
    const uint32_t rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;  // may carry into the exponent
    mag = min((e << 3) + keep, 0x7Eu);
  }
  return sign | mag;
}

// E4M3 byte -> fp32 (exact; the byte is never the NaN code here)
__device__ __forceinline__ float e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e == 0 ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (b & 0x80u) ? -mag : mag;
}

// fp32 -> E2M1 code, round to nearest even, saturating (finite v)
__device__ __forceinline__ uint32_t e2m1_rne(float v) {
  const float a = fabsf(v);
  const uint32_t mag = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return mag | ((__float_as_uint(v) >> 28) & 8u);
}

__device__ __forceinline__ float bf16_value(uint32_t bits) { return __uint_as_float(bits << 16); }

// One workgroup per row: the row's max |w| (on the BF16 bit patterns, whose
// order is the order of the magnitudes), then the codes.
__global__ __launch_bounds__(kQuantThreads) void quant_fp8row_kernel(const uint16_t* __restrict__ w, int K,
                                                                     uint8_t* __restrict__ q,
                                                                     float* __restrict__ row_scale) {
  __shared__ uint32_t wmax[kQuantThreads / 64];
  const int64_t row = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(w + row * K);
  const int n8 = K / 8;
  uint32_t mx = 0;
  for (int i = threadIdx.x; i < n8; i += kQuantThreads) {
    const uint4 v = src[i];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) mx = max(mx, max(p[j] & 0x7FFFu, (p[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const float r = __fdiv_rn(bf16_value(mx), 448.0f);
  if (threadIdx.x == 0) row_scale[row] = r;
  uint2* dst = reinterpret_cast<uint2*>(q + row * K);
  for (int i = threadIdx.x; i < n8; i += kQuantThreads) {
    const uint4 v = src[i];
    const uint32_t p[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2] = {0u, 0u};
    if (r > 0.0f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = e4m3_rne(__fdiv_rn(bf16_value(p[j] & 0xFFFFu), r));
        const uint32_t hi = e4m3_rne(__fdiv_rn(bf16_value(p[j] >> 16), r));
        o[j >> 1] |= (lo | (hi << 8)) << (16 * (j & 1));
      }
    }
    dst[i] = make_uint2(o[0], o[1]);
  }
}

// One thread per block of 16 k.
__global__ __launch_bounds__(kQuantThreads) void quant_nvfp4_kernel(const uint16_t* __restrict__ w, int64_t blocks,
                                                                    float g, uint8_t* __restrict__ codes,
                                                                    uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x;
  if (b >= blocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(w) + 2 * b;
  const uint4 v0 = src[0], v1 = src[1];
  const uint32_t p[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) mx = max(mx, max(p[j] & 0x7FFFu, (p[j] >> 16) & 0x7FFFu));
  const float six_g = 6.0f * g;
  const uint32_t s = e4m3_rne(__fdiv_rn(bf16_value(mx), six_g));
  const float d = e4m3_value(s) * g;
  uint32_t o[2] = {0u, 0u};
  if (d > 0.0f) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // element 2j (low nibble) and 2j + 1 (high nibble) of the block
      const uint32_t lo = e2m1_rne(__fdiv_rn(bf16_value(p[j] & 0xFFFFu), d));
      const uint32_t hi = e2m1_rne(__fdiv_rn(bf16_value(p[j] >> 16), d));
      o[j >> 2] |= (lo | (hi << 4)) << (8 * (j & 3));
    }
  }
  reinterpret_cast<uint2*>(codes)[b] = make_uint2(o[0], o[1]);
  scales[b] = (uint8_t)s;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace wq

extern "C" {

wq_status wq_quantize_fp8row(const uint16_t* w, int M, int K, uint8_t* q, float* row_scale, void* stream) {
  if (!w || !q || !row_scale || M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (K % 16 != 0 || K > (1 << 24) || (uint64_t)M * (uint64_t)K >= (1ull << 40) || M > 0x7FFFFFFF)
    return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (!wq::aligned16(w) || !wq::aligned16(q) || !wq::aligned16(row_scale)) return WQ_ERROR_MISALIGNED;
  hipLaunchKernelGGL(wq::quant_fp8row_kernel, dim3(M), dim3(wq::kQuantThreads), 0, static_cast<hipStream_t>(stream),
                     w, K, q, row_scale);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_quantize_nvfp4(const uint16_t* w, int M, int K, float global_scale, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (!w || !codes || !scales || M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  if (!(global_scale > 0.0f) || global_scale > 3.4e38f) return WQ_ERROR_INVALID_VALUE;
  if (K % 32 != 0 || K > (1 << 24) || (uint64_t)M * (uint64_t)K >= (1ull << 40)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (!wq::aligned16(w) || !wq::aligned16(codes) || !wq::aligned16(scales)) return WQ_ERROR_MISALIGNED;
  const int64_t blocks = (int64_t)M * (K / 16);
  const int64_t grid = (blocks + wq::kQuantThreads - 1) / wq::kQuantThreads;
  if (grid > 0x7FFFFFFF) return WQ_ERROR_UNSUPPORTED_SHAPE;
  hipLaunchKernelGGL(wq::quant_nvfp4_kernel, dim3((unsigned)grid), dim3(wq::kQuantThreads), 0,
                     static_cast<hipStream_t>(stream), w, blocks, global_scale, codes, scales);
  return hipGetLastError() == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

}  // extern "C"
