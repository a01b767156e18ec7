// wq_kernels.hip -- gfx950 kernels of the verify-pass skinny GEMM
//     Y[n][m] = sum_k W[m][k] * X[n][k],  N <= 8 columns,
// for W in NVFP4 (E2M1 codes, one E4M3 scale per 16 k, FP32 tensor scale)
// or in row-scaled FP8-E4M3, X in BF16, Y in FP32.
//
// The crit-hub engine card "mtp7-device-confidence" (section "Design", row
// "GEMVs") runs this product on an RTX 5090 by reading the weight bytes
// straight into BF16 tensor-core fragments.  What is kept here: weights are
// read once, in their stored bytes, and widened to BF16 only in registers.
// What is rebuilt for CDNA4 (one 1024-thread workgroup per CU, wave64):
//
//  * One wave owns a tile of 16 weight rows and walks its K range in
//    segments of 64 bytes per row (one 16-byte buffer load per lane, four
//    lanes per row), PF segments in flight.
//  * E2M1 -> BF16 and E4M3 -> BF16 use gfx950's scaled conversion
//    instructions with scale 1.0, which are exact.  Those instructions
//    apply only the exponent of their scale, so an E4M3 block scale (which
//    has mantissa bits) cannot ride on them.  Instead the NVFP4 path puts
//    the two 16-k scale blocks of a 32-k MFMA step on different A rows:
//    A = X arranged as 16 rows (block b, column n), zero where the k slot
//    belongs to the other block, B = the 16 weight rows' codes.  The
//    16x16x32 BF16 MFMA then returns per-block partial sums, and each lane
//    applies its row's block scale with one FP32 FMA per partial.  Every
//    product is exact; only the FP32 sums round.
//  * The N activation columns of the current K chunk live in LDS, staged
//    once per (matrix, chunk) by the whole workgroup, laid out so that each
//    MFMA's A operand is one conflict-free 16-byte read per lane.
//  * In a verify pass K is split into chunks only to fit LDS (<= 8704 k).
//    Large split matrices of an all-tiled pass keep their chunk sums in LDS
//    (blocked splits); others write them to the workspace for reduce_kernel,
//    which adds them in chunk order.  Results never depend on timing.
//  * A verify pass is one launch over a table of matrices: the units
//    (matrix, chunk, 16-row tile) are split into one contiguous run per
//    workgroup, balanced by bytes on the host, with a dynamic tail.
//  * A single tiled product with few tiles per CU (split_kernel) cuts its
//    steps into one run per workgroup and one piece per wave; tiles whose K
//    chunks end in different workgroups are finished by the last one to
//    arrive (an arrival counter per tile), adding the parts in chunk order.
//  * Output writes are what the stream pays for beyond its reads, and they
//    cost least when the whole chip writes at once: from N = 4 up each wave
//    holds its last pair of tiles' outputs until the chip-wide 100 MHz clock
//    enters a new window (or its next tile ends), so that writes bunch; a
//    run short enough for all its pairs to wait in the LDS past its X chunk
//    (a single product's, a tail claim's) writes them at its end.
//
// Numerics do not depend on N: a column's A rows, its MFMA sums, its FMA
// rescale chain and its chunk sum are the same whatever the other columns
// hold.  N only selects which LDS rows exist and which lanes read them.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "wq_internal.h"

namespace wq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(3))) unsigned u32x3;

// Raw buffer resource word 3 for gfx9-family raw (untyped) buffer access.
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy for the weight stream: default (temporal).  Each 128-byte line
// of codes is read by two consecutive segments and each scale line by many;
// the non-temporal hint made the L2 drop lines between those reads (about
// 1.5x the HBM traffic and 35% lower throughput on MI355X).
constexpr int kAuxStream = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

// Tiled NVFP4 reads every line whole within one wave instruction, so the
// non-temporal policy is safe there and streams faster (6.0 vs 5.7 TB/s).
constexpr int kAuxTiled = 2;
__device__ __forceinline__ u32x4 bload16t(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxTiled));
}
__device__ __forceinline__ u32x2 bload8t(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAuxTiled));
}
// Same, with base and size pinned to scalar registers (they are wave-uniform;
// the pinning keeps the compiler from treating the resource as divergent).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint64_t bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0, (int)n,
                                           kRsrcWord3);
}

// Output stores of the tiled stream are written through the L2 (device
// scope, sc1).  With the weight loads non-temporal, the default write-back
// policy left dirty output lines to leave the L2 later as evictions, which
// cost the read stream more: over the dense 64-layer pass on MI355X, paired
// full-line stores ran at 6.17 / 5.93 / 5.74 TB/s (N = 2 / 4 / 8) written
// back and 6.44 / 6.33 / 6.07 TB/s written through; system scope measured
// the same as device scope, and the non-temporal hint was slower.
constexpr int kAuxOut = 16;
__device__ __forceinline__ void bstore4(float v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)off, 0, kAuxOut);
}
__device__ __forceinline__ void bstore2(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, (int)off, 0, kAuxOut);
}
// A buffer offset past every output buffer (outputs are < 2 GiB): the
// hardware range check drops stores there.
constexpr uint32_t kDropOffset = 0x80000000u;
// Device-scope (sc1) loads: they take no line from a cache that another XCD
// may not see, so they return what a write-through store of any workgroup
// left in memory once that store has completed.  With write-through stores
// on the other side, data passes between workgroups of one launch with no
// L2 writeback or invalidate (the single-launch chain's phases).
constexpr int kAuxCoherent = 16;

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxStream));
}
__device__ __forceinline__ u32x2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAuxStream));
}
__device__ __forceinline__ uint32_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kAuxStream);
}

// Eight E2M1 codes (one dword, low nibble first) -> eight exact BF16 values.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Eight E4M3 codes (two dwords, low byte first) -> eight exact BF16 values.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ bf16x8 lds_read16(const char* lds, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds + off);
}

// ---- staging of one K chunk of X into LDS --------------------------------
// LDS layout: piece (kc, n) = X[n][k0 + 8kc .. k0 + 8kc + 7] (16 bytes) at
// byte (kc * N + n) * 16, for kc < kc_pad (pieces past the chunk are zero).
constexpr int kStageLoads = 8;
// One batch: the pieces p0 + j * blockDim.x, j < kStageLoads, into registers
// (eight 16-byte loads in flight per thread before any LDS store: staging
// is a few rounds of L2/HBM latency, and at the start of every run) ...
template <int N>
__device__ __forceinline__ void stage_x_load(u32x4 (&v)[kStageLoads], const uint16_t* __restrict__ x, int K, int k0,
                                             int klen, int kc_pad, int p0) {
  const int valid = klen / 8;
  const int total = kc_pad * N;
#pragma unroll
  for (int j = 0; j < kStageLoads; ++j) {
    const int p = p0 + j * (int)blockDim.x;
    const int n = p / kc_pad, kc = p - n * kc_pad;
    v[j] = u32x4{0u, 0u, 0u, 0u};
    if (p < total && kc < valid) v[j] = *reinterpret_cast<const u32x4*>(x + (size_t)n * K + k0 + 8 * kc);
  }
}
// ... and from registers into LDS.
template <int N>
__device__ __forceinline__ void stage_x_store(const u32x4 (&v)[kStageLoads], char* lds, int kc_pad, int p0) {
  const int total = kc_pad * N;
#pragma unroll
  for (int j = 0; j < kStageLoads; ++j) {
    const int p = p0 + j * (int)blockDim.x;
    const int n = p / kc_pad, kc = p - n * kc_pad;
    if (p < total) *reinterpret_cast<u32x4*>(lds + (size_t)(kc * N + n) * 16) = v[j];
  }
}
// The batches after the first, whose registers v0 were loaded earlier (the
// tiled runs load them before their first weight loads, so that X, needed
// first, is not queued behind the weights).
template <int N>
__device__ void stage_x_rest(const u32x4 (&v0)[kStageLoads], char* lds, const uint16_t* __restrict__ x, int K, int k0,
                             int klen, int kc_pad) {
  stage_x_store<N>(v0, lds, kc_pad, (int)threadIdx.x);
  for (int p0 = (int)threadIdx.x + kStageLoads * (int)blockDim.x; p0 < kc_pad * N;
       p0 += kStageLoads * (int)blockDim.x) {
    u32x4 v[kStageLoads];
    stage_x_load<N>(v, x, K, k0, klen, kc_pad, p0);
    stage_x_store<N>(v, lds, kc_pad, p0);
  }
}
// All batches (the plain-layout kernels).
template <int N>
__device__ void stage_x(char* lds, const uint16_t* __restrict__ x, int K, int k0, int klen, int kc_pad) {
  for (int p0 = threadIdx.x; p0 < kc_pad * N; p0 += kStageLoads * (int)blockDim.x) {
    u32x4 v[kStageLoads];
    stage_x_load<N>(v, x, K, k0, klen, kc_pad, p0);
    stage_x_store<N>(v, lds, kc_pad, p0);
  }
}

// All pieces of one K chunk in flight at once, with direct buffer-to-LDS
// loads (the tiled verify-pass kernels): instruction j of wave w writes the
// 64 consecutive pieces q = j * blockDim.x + 64 w + lane of the LDS order
// (q = kc * N + n at byte 16 q; a buffer-to-LDS load puts lane l's 16 bytes
// at its base plus 16 l).  Pieces past the chunk's last k read past the
// end of X, which the range check returns as zeros.  No registers hold X on
// the way, so a chunk of any size is one round trip, where staging through
// registers (eight 16-byte loads per thread per round) took two or three
// at N = 8.  The caller waits for the loads and synchronizes.
template <int N, int AUX = 0>
__device__ __forceinline__ void stage_x_direct(char* lds, const uint16_t* __restrict__ x, int K, int k0, int klen,
                                               int kc_pad) {
  const __amdgpu_buffer_rsrc_t rx = make_rsrc_uniform(x, (uint64_t)N * (uint64_t)K * 2u);
  const int valid = klen / 8;
  const int total = kc_pad * N;
  const int lane = (int)(threadIdx.x & 63);
  const int wbase = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u));
  for (int q0 = wbase; q0 < total; q0 += (int)blockDim.x) {
    const int q = q0 + lane;
    const int kc = q / N, n = q - kc * N;
    // (N K 2 < 2^31: an offset of 2^31 is past every X)
    const uint32_t off = kc < valid ? (uint32_t)((n * K + k0 + 8 * kc) * 2) : 0x80000000u;
    if (q < total)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (__attribute__((address_space(3))) void*)(lds + (size_t)q0 * 16), 16,
                                               off, 0, 0, AUX);
  }
}

// FP32 -> BF16 bits, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---- staging of an RMS-normalized X (chained MLP layers) -----------------
// X[n][k] = BF16(h[n][k] * r[n] * gamma[k]), r[n] = 1 / sqrt(ss[n] / K + eps),
// with ss[n] the sum of the nparts partial sums of squares of column n
// -- the RMSNorm of a pre-norm transformer layer, computed
// once per workgroup from the FP32 residual stream instead of by a kernel of
// its own.  Every workgroup computes the same bits; the pieces of 16 bytes
// numbered 256j .. 256j + 255 are also written to aout by the workgroup
// whose units [u0, u1) hold unit j mod units (the units of all workgroups
// partition the matrix's), so that the normalized input is visible to the
// caller.
// r[n] goes to the 512 bytes past the zero block.  Every thread calls this.
constexpr int kNormLoads = 2;
// Registers of one batch (the first one is loaded before the run's first
// weight loads): each lane's partial sum of squares (nparts <= 64: one per
// lane) and the h / gamma pieces p0 + j * blockDim.x, j < kNormLoads.  Piece
// p is (kc, n) = (p / N, p mod N), k-major: the N lanes of one kc load the
// same gamma piece (one request) and write consecutive LDS pieces.
struct NormBatch {
  f32x4 h0[kNormLoads], h1[kNormLoads];
  u32x4 gm[kNormLoads];
  float ss;
};
// COH: h and its partial sums of squares were written in the same launch
// (the single-launch chain), so they are read with device-scope loads.
template <int N, bool COH>
__device__ __forceinline__ void norm_load(NormBatch& b, const DevMat& mt, int kc_pad, int p0) {
  const int K = mt.K;
  const int valid = K / 8;
  const int total = kc_pad * N;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc_uniform(mt.h, (uint64_t)N * (uint64_t)K * 4u);
#pragma unroll
  for (int j = 0; j < kNormLoads; ++j) {
    const int p = p0 + j * (int)blockDim.x;
    const int kc = p / N, n = p - kc * N;
    b.h0[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    b.h1[j] = b.h0[j];
    b.gm[j] = u32x4{0u, 0u, 0u, 0u};
    if (p < total && kc < valid) {
      if constexpr (COH) {
        const uint32_t off = (uint32_t)((n * K + 8 * kc) * 4);
        b.h0[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)off, 0, kAuxCoherent));
        b.h1[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)off + 16, 0, kAuxCoherent));
      } else {
        const float* hp = mt.h + (size_t)n * K + 8 * kc;
        b.h0[j] = *reinterpret_cast<const f32x4*>(hp);
        b.h1[j] = *reinterpret_cast<const f32x4*>(hp + 4);
      }
      b.gm[j] = *reinterpret_cast<const u32x4*>(mt.gamma + 8 * kc);
    }
  }
}
template <int N, bool COH>
__device__ __forceinline__ void norm_first(NormBatch& b, const DevMat& mt, int kc_pad) {
  const int wv = (int)(threadIdx.x >> 6), ln = (int)(threadIdx.x & 63);
  if constexpr (COH) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc_uniform(mt.ssp, (uint64_t)N * (uint64_t)mt.nparts * 4u);
    const uint32_t off = (wv < N && ln < mt.nparts) ? (uint32_t)((wv * mt.nparts + ln) * 4) : kDropOffset;
    b.ss = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off, 0, kAuxCoherent));
  } else {
    b.ss = (wv < N && ln < mt.nparts) ? mt.ssp[(size_t)wv * mt.nparts + ln] : 0.0f;
  }
  norm_load<N, COH>(b, mt, kc_pad, (int)threadIdx.x);
}
template <int N>
__device__ __forceinline__ void norm_store(const NormBatch& b, char* lds, const DevMat& mt, int kc_pad, int p0,
                                           const float* rl, int64_t u0, int64_t u1, int64_t units) {
  const int K = mt.K;
  const int valid = K / 8;
  const int total = kc_pad * N;
#pragma unroll
  for (int j = 0; j < kNormLoads; ++j) {
    const int p = p0 + j * (int)blockDim.x;
    if (p >= total) continue;
    const int kc = p / N, n = p - kc * N;
    const float r = rl[n];
    const float hv[8] = {b.h0[j].x, b.h0[j].y, b.h0[j].z, b.h0[j].w, b.h1[j].x, b.h1[j].y, b.h1[j].z, b.h1[j].w};
    u32x4 o = {0u, 0u, 0u, 0u};
    if (kc < valid) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float glo = __uint_as_float(b.gm[j][i] << 16), ghi = __uint_as_float(b.gm[j][i] & 0xFFFF0000u);
        const float lo = (hv[2 * i] * r) * glo, hi = (hv[2 * i + 1] * r) * ghi;
        o[i] = bf16_rne(lo) | (bf16_rne(hi) << 16);
      }
      const int64_t owner = (int64_t)(p >> 8) % units;
      if (owner >= u0 && owner < u1) *reinterpret_cast<u32x4*>(mt.aout + (size_t)n * K + 8 * kc) = o;
    }
    *reinterpret_cast<u32x4*>(lds + (size_t)(kc * N + n) * 16) = o;
  }
}
// Everything after norm_first (every thread calls it; it holds a barrier).
template <int N, bool COH>
__device__ void stage_norm(NormBatch& b, char* lds, const DevMat& mt, int kc_pad, int64_t u0, int64_t u1,
                           int64_t units) {
  float* rl = reinterpret_cast<float*>(lds + kZeroOffset<N>() + kZeroBytes<N>());
  // wave n sums column n's partials (lane l holds p = l; nparts <= 64) by a
  // butterfly over the lanes (a fixed order, so every workgroup agrees)
  {
    const int wv = (int)(threadIdx.x >> 6), ln = (int)(threadIdx.x & 63);
    if (wv < N) {
      float ss = b.ss;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
      if (ln == 0) rl[wv] = __fdiv_rn(1.0f, __fsqrt_rn(__fdiv_rn(ss, (float)mt.K) + mt.eps));
    }
  }
  __syncthreads();
  norm_store<N>(b, lds, mt, kc_pad, (int)threadIdx.x, rl, u0, u1, units);
  for (int p0 = (int)threadIdx.x + kNormLoads * (int)blockDim.x; p0 < kc_pad * N;
       p0 += kNormLoads * (int)blockDim.x) {
    norm_load<N, COH>(b, mt, kc_pad, p0);
    norm_store<N>(b, lds, mt, kc_pad, p0, rl, u0, u1, units);
  }
}

// ---- epilogue: lanes 0..31 hold sum[r] for n = 4*(lane/16) + r ----------
// Unsplit tiles store y = mscale * sum.  Tiles of a K-split matrix store the
// raw chunk sum into the workspace; reduce_kernel, launched after this
// kernel on the same stream, adds the chunks in chunk order.
template <int N>
__device__ __forceinline__ void finish_tile(const DevMat& mt, int chunk, int tile, const float sum[4],
                                            float mscale) {
  const int lane = threadIdx.x & 63;
  const int m = tile * 16 + (lane & 15);
  const int nb = 4 * (lane >> 4);
  if (lane >= 32 || m >= mt.M) return;
  if (mt.nchunks == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (nb + r < N) mt.y[(size_t)(nb + r) * mt.M + m] = mscale * sum[r];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (nb + r < N) mt.part[((size_t)chunk * N + nb + r) * mt.M + m] = sum[r];
  }
}

// ---- one NVFP4 unit: 16 rows x one K chunk --------------------------------
// The weight stream is a ring of PF segments per lane.  Loads are issued
// unconditionally (offsets past the chunk are clamped to its last segment,
// which is then fetched again from cache and never used) so that the
// compiler sees straight-line code and keeps PF loads in flight.
template <int N, int PF, bool SALIGN>
__device__ void nvfp4_unit(const DevMat& mt, int chunk, int tile, const char* lds) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int k0 = chunk * mt.kc;
  const int klen = min(mt.kc, mt.K - k0);
  const int nseg = (klen + 127) >> 7;
  const uint64_t rowb = (uint64_t)mt.K >> 1, srowb = (uint64_t)mt.K >> 4;
  const uint64_t m0 = (uint64_t)tile * 16;
  const uint64_t cstart = m0 * rowb + (uint64_t)(k0 >> 1);
  const uint64_t sstart = m0 * srowb + (uint64_t)(k0 >> 4);
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(mt.w + cstart, (uint64_t)mt.M * rowb - cstart);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(mt.s + sstart, (uint64_t)mt.M * srowb - sstart);
  const uint32_t voc = (uint32_t)(c * rowb) + 16u * g;
  const uint32_t vos = (uint32_t)(c * srowb);

  // A operand (X): lane (i = c, group g) is live when its row's block b = i/8
  // matches the block of its k slots (g/2) and its column n = i%8 exists.
  const bool active = ((c >> 3) == (g >> 1)) && ((c & 7) < N);
  const uint32_t xoff = active ? (uint32_t)((g * N + (c & 7)) * 16) : kZeroOffset<N>();
  const uint32_t xstep = active ? 256u * N : 0u;

  // scale bytes this lane applies: parity p of the 8 blocks of a segment
  const uint32_t psel = (lane >> 5) ? 0x07050301u : 0x06040200u;

  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  u32x4 cw[PF];
  u32x2 sw[PF];
  // Scale rows are 4-byte aligned when K % 64 == 0 (SALIGN); otherwise the
  // eight scale bytes of a segment are fetched as four 2-byte loads and
  // joined only when the segment is consumed.
  uint32_t sh[SALIGN ? 1 : PF][4];
  const int last = nseg - 1;
  auto load = [&](int seg, int slot) {
    seg = min(seg, last);
    cw[slot] = bload16(rc, voc + 64u * seg);
    if constexpr (SALIGN) {
      sw[slot] = bload8(rs, vos + 8u * seg);
    } else {
      const uint32_t o = vos + 8u * seg;
#pragma unroll
      for (int j = 0; j < 4; ++j) sh[slot][j] = bload2(rs, o + 2 * j);
    }
  };
  auto compute = [&](int slot, int seg) {
    const u32x4 d = cw[slot];
    u32x2 q;
    if constexpr (SALIGN) {
      q = sw[slot];
    } else {
      q = u32x2{sh[slot][0] | (sh[slot][1] << 16), sh[slot][2] | (sh[slot][3] << 16)};
    }
    // 4x4 dword transpose across the row's four lanes: afterwards lane
    // group g holds, for MFMA step t, bytes [16t + 4g, 16t + 4g + 4) of the
    // row's 64-byte segment, i.e. k = 32t + 8g .. 32t + 8g + 7.
    const u32x2 t0 = __builtin_amdgcn_permlane32_swap(d.x, d.z, false, false);
    const u32x2 t1 = __builtin_amdgcn_permlane32_swap(d.y, d.w, false, false);
    const u32x2 t2 = __builtin_amdgcn_permlane16_swap(t0.x, t1.x, false, false);
    const u32x2 t3 = __builtin_amdgcn_permlane16_swap(t0.y, t1.y, false, false);
    const uint32_t e[4] = {t2.x, t2.y, t3.x, t3.y};
    // block scales for steps t = 0..3 (blocks 2t + p of the segment); blocks
    // past the chunk get scale 0 (their X is zero, but a NaN scale is not)
    const int vb = (klen - 128 * seg) >> 4;
    const uint32_t smask = vb >= 8 ? 0xFFFFFFFFu : ((1u << (4 * vb)) - 1u);
    const uint32_t sb = __builtin_amdgcn_perm(q.y, q.x, psel) & smask;
    const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, true);
    const float st[4] = {s01.x, s01.y, s23.x, s23.y};
    const uint32_t xo = xoff + (uint32_t)seg * xstep;
    bf16x8 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = lds_read16(lds, xo + t * 64u * N);
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = e2m1x8_to_bf16(e[t]);
    f32x4 part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(st[t], part[t][r], acc[r]);
  };

#pragma unroll
  for (int i = 0; i < PF; ++i) load(i, i);
  int s0 = 0;
  for (; s0 + PF <= nseg; s0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      compute(i, s0 + i);
      load(s0 + i + PF, i);
    }
  }
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (s0 + i < nseg) compute(i, s0 + i);

  // lanes l and l+32 hold blocks 0 and 1 of the same (n, m): add in that order
  float sum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const u32x2 sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[r]), false, false);
    sum[r] = acc[r] + __uint_as_float(sw2.y);
  }
  finish_tile<N>(mt, chunk, tile, sum, mt.g);
}

// ---- a wave's tiles of one run, tiled NVFP4 or tiled FP8-row ----------------
// NVFP4 (FP8 = false): the arithmetic of nvfp4_unit, on weights stored by
// wq_nvfp4_tile.  A step of 256 k is one 2304-byte block per 16-row tile, so
// each lane's loads are 16 bytes of one contiguous 1 KB (codes, twice) plus
// 8 bytes of one contiguous 256 B (scales), with the codes already in the
// order the MFMA B operand wants and the scales already split by parity.
//
// FP8-row (FP8 = true): the arithmetic of fp8_unit, on weights stored by
// wq_fp8_tile.  A step of 128 k is one 2048-byte block per tile; each of a
// lane's two 16-byte loads is the 16 row bytes fp8_unit gathers for one
// 64-k segment, so the MFMA sequence (and the result) is fp8_unit's.  The
// row scale of the lane's row comes with every step (a 4-byte load that
// hits the cache), so that every step issues the same memory operations.
//
// The wave takes the consecutive tiles [first, end) of one matrix and K
// chunk (all nst steps long).  They lie back to back in memory, so the
// wave's whole share is one sequential stream, and it is streamed as ONE
// sequence of steps: the ring keeps PF steps in flight across tile
// boundaries.
// Greedy key of one logit: the order of (value, -row) as an unsigned 64-bit
// number, so that a max over keys gives the largest value and, among equal
// values, the lowest row.  NaN sorts above every number (the first NaN row
// wins) and -0 is taken as +0.
__device__ __forceinline__ uint64_t greedy_key(float v, int m) {
  uint32_t o;
  if (v != v) {
    o = 0xFFFFFFFFu;
  } else {
    const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
    o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)m);
}

// What a finished tile does with its sums (EPI):
//  kEpiStore   store y (or the chunk's partial sums), paired as below;
//  kEpiArgmax  the same, and keep, per lane and register r, the greedy key
//              of the lane's outputs (lanes 0..31: column 4 * (lane / 16) + r,
//              rows 16 t + lane % 16);
//  kEpiGlu     gate/up tiles (rows c < 8 gate, c >= 8 up of f = 8 t + c % 8):
//              store s[n][f] = BF16(silu(gate) * up), silu(v) = v / (1 + e^-v).
//
// stage() stages the run's X into LDS between two workgroup barriers.  The
// run calls it once on every path, after issuing its first PF steps of
// weight loads, so that their round trip overlaps the staging; pre(), called
// first, issues the staging's first loads, so that X does not wait for the
// weights (a wave's loads complete in order).
constexpr int kEpiStore = 0;
constexpr int kEpiArgmax = 1;
constexpr int kEpiGlu = 2;
// Units [first, end) are tiles first - ubase .. end - 1 - ubase of chunk
// `chunk`.  ptile0 >= 0 marks a blocked split matrix (DevMat::tb) whose
// block starts at tile ptile0 (BLK kernels only): the chunk sums of the
// block's tiles wait in LDS (one 512-byte slot per tile of the block, placed
// as part_a_slots says) for the next chunk, which adds its own to them, in
// chunk order as reduce_kernel does, and the last chunk stores y.
//
// VALU (NVFP4 only): the step on the vector ALUs instead of the matrix cores,
// the other side of the MFMA/VALU comparison.  Lane l = c + 16 g holds, for
// half h and MFMA step j, the eight codes of row c at k = 128 h + 32 j + 8 g
// + 0..7 of its step (one 16-k scale block, whose scale is the lane's byte
// j); it widens them to BF16 (exact), forms for every column n the eight
// products with X by four BF16 dot-2 instructions (FP32 sums), and adds them,
// times the block scale, to its FP32 sum for column n.  At a tile's end the
// four lanes of row c (g = 0..3) add their sums (a fixed butterfly) and the
// results are laid out as the MFMA epilogue expects them (lanes 0..31: rows
// n = 4 (lane / 16) + r of m = lane % 16; lanes 32..63: zero), so the same
// epilogue follows.
template <int N, int PF, bool FP8, int EPI, bool BLK, bool VALU = false, typename Pre, typename Stage>
__device__ void tiled_run(const DevMat& mt, int chunk, int64_t first, int64_t end, int64_t ubase, int ptile0,
                          char* lds, uint64_t* bestk, Pre&& pre, Stage&& stage) {
  static_assert(!(VALU && FP8), "the vector-ALU step is the NVFP4 one");
  pre();
  if (first >= end) {
    stage();
    return;
  }
  constexpr int kStep = FP8 ? kFp8TileStepK : kTileStepK;
  constexpr uint32_t kBlock = FP8 ? kFp8TileBlockBytes : kTileBlockBytes;
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int k0 = chunk * mt.kc;
  const int klen = min(mt.kc, mt.K - k0);
  const int nst = (klen + kStep - 1) / kStep;
  const int cnt = (int)(end - first);
  const int tile0 = (int)(first - ubase);
  const uint32_t steps_per_row = (uint32_t)((mt.K + kStep - 1) / kStep);
  const uint32_t base_step = (uint32_t)(k0 / kStep);
  const uint64_t total = (uint64_t)mt.ntiles * steps_per_row * kBlock;  // < 2^32 (checked on the host)
  const __amdgpu_buffer_rsrc_t rw = make_rsrc_uniform(mt.w, total);
  const uint32_t vc = 16u * lane;
  const uint32_t vs = (uint32_t)kTileCodeBytes + 8u * (uint32_t)(((lane >> 5) << 4) + c);
  // FP8 row scales: rows past M read as 0 (range check)
  const __amdgpu_buffer_rsrc_t rr = make_rsrc_uniform(mt.rs, FP8 ? (uint64_t)mt.M * 4u : 0u);

  // A operand (X) in LDS.  NVFP4: rows (scale block b, column n), so a lane
  // is live where its k slots belong to its block; FP8: rows are columns.
  bool active;
  uint32_t xoff, xstep;
  if constexpr (FP8) {
    active = c < N;
    xoff = active ? (uint32_t)((2 * g * N + c) * 16) : kZeroOffset<N>();
    xstep = active ? 256u * N : 0u;
  } else {
    active = ((c >> 3) == (g >> 1)) && ((c & 7) < N);
    xoff = active ? (uint32_t)((g * N + (c & 7)) * 16) : kZeroOffset<N>();
    xstep = active ? 512u * N : 0u;
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 c0[PF], c1[PF];
  u32x2 sw[PF];     // NVFP4 block scales
  uint32_t rv[PF];  // FP8 row scale bits

  // next step to load: tile li, step lst (past the end: the last step again)
  int li = 0, lst = 0;
  auto load_next = [&](int slot) {
    const bool past = li >= cnt;
    const uint32_t ti = (uint32_t)(past ? cnt - 1 : li);
    const uint32_t ts = (uint32_t)(past ? nst - 1 : lst);
    const uint32_t b = (((uint32_t)tile0 + ti) * steps_per_row + base_step + ts) * kBlock;
    c0[slot] = bload16t(rw, b + vc);
    c1[slot] = bload16t(rw, b + 1024u + vc);
    if constexpr (FP8)
      rv[slot] = __builtin_amdgcn_raw_buffer_load_b32(rr, (int)(((tile0 + ti) * 16u + c) * 4u), 0, 0);
    else
      sw[slot] = bload8t(rw, b + vs);
    if (++lst == nst) { lst = 0; ++li; }
  };
  // NVFP4: half a step (128 k) of one slot
  auto half = [&](const u32x4& e, uint32_t sb, uint32_t xo) {
    const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, true);
    const float stv[4] = {s01.x, s01.y, s23.x, s23.y};
    bf16x8 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = lds_read16(lds, xo + t * 64u * N);
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = e2m1x8_to_bf16(e[t]);
    f32x4 part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(stv[t], part[t][r], acc[r]);
  };
  // NVFP4 on the vector ALUs: half h of the step cs
  float accv[N];
#pragma unroll
  for (int n = 0; n < N; ++n) accv[n] = 0.f;
  auto half_valu = [&](const u32x4& e, uint32_t sb, int h, int cs) {
    const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, true);
    const float stv[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8 w = e2m1x8_to_bf16(e[j]);
      const uint32_t xb = (uint32_t)((32 * cs + 16 * h + 4 * j + g) * N) * 16u;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        const bf16x8 xv = lds_read16(lds, xb + 16u * n);
        float d = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[0], w[1]}, bf16x2{xv[0], xv[1]}, 0.f, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[2], w[3]}, bf16x2{xv[2], xv[3]}, d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[4], w[5]}, bf16x2{xv[4], xv[5]}, d, false);
        d = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{w[6], w[7]}, bf16x2{xv[6], xv[7]}, d, false);
        accv[n] = __builtin_fmaf(stv[j], d, accv[n]);
      }
    }
  };
  // FP8: one 64-k segment (16 bytes of the lane's row)
  auto segment = [&](const u32x4& d, uint32_t xo) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) a[u] = lds_read16(lds, xo + u * 16u * N);
#pragma unroll
    for (int u = 0; u < 2; ++u) b[u] = e4m3x8_to_bf16(d[2 * u], d[2 * u + 1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
  };
  // Outputs: y (scaled by g) for an unsplit matrix, else this chunk's plane
  // of the partial sums, both [N][M].  Tiles are written in pairs (global
  // tiles 2j and 2j + 1, consecutive in the wave's share): a tile's sums wait
  // in registers for the next tile's, and then each store instruction writes
  // two whole 128-byte lines, rows n and n + 4 of 32 consecutive m.  A tile
  // without its partner in the share is written alone, as half lines.
  //
  // Every step issues the same min(N, 4) stores; only on the step that
  // writes a pair (the pair's last tile, or with deferred outputs the step
  // that releases the held pair) do their offsets point into the buffer,
  // otherwise the range check drops them.  An equal count of memory
  // operations on every step keeps the compiler's vmcnt waits exact across
  // the epilogue (a conditional store makes it wait for everything).
  constexpr int kStores = N < 4 ? N : 4;
  const bool blocked = BLK && ptile0 >= 0;
  const bool split = mt.nchunks > 1 && !blocked;
  // blocked: chunk sums come from (after the first chunk) and go to (before
  // the last) the block's LDS slots; only the last chunk stores
  const bool from_lds = blocked && chunk > 0;
  const bool to_lds = blocked && chunk < mt.nchunks - 1;
  float* const obase = split ? mt.part + (size_t)chunk * N * mt.M : mt.y;
  // (no output buffer -- head acceptance without logits -- drops every store)
  const int F = mt.M / 2;  // kEpiGlu: outputs per column
  const __amdgpu_buffer_rsrc_t ro =
      EPI == kEpiGlu ? make_rsrc_uniform(mt.sout, (uint64_t)N * (uint64_t)F * 2u)
                     : make_rsrc_uniform(obase, obase ? (uint64_t)N * (uint64_t)mt.M * 4u : 0u);
  uint32_t sbits[4] = {0u, 0u, 0u, 0u};  // kEpiGlu: BF16 outputs
  const float gscale = split ? 1.0f : mt.g;
  float sum[4] = {0.f, 0.f, 0.f, 0.f};
  float prev[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t so[4] = {kDropOffset, kDropOffset, kDropOffset, kDropOffset};
  // Deferred outputs (N >= kDeferMinN): an emitted pair is held in psum /
  // pso and written at the first step on which the chip-wide 100 MHz clock
  // has entered a new window of 2^kDeferWindowBits ticks, or at the end of
  // the next tile, whichever comes first.  Waves all over the chip then
  // write in the same short intervals instead of at random moments: writes
  // that reach memory while reads stream past cost a read/write turnaround
  // each when they arrive alone, far less when they arrive together.
  constexpr bool kDefer = EPI == kEpiStore && N >= kDeferMinN;
  float psum[4] = {0.f, 0.f, 0.f, 0.f};
  uint32_t pso[4] = {kDropOffset, kDropOffset, kDropOffset, kDropOffset};
  bool pending = false;
  uint32_t pwin = 0;
  // Held outputs (the 8-wave tiled kernels, N >= kDeferMinN): when every
  // pair this wave emits in the run fits in its share of the LDS between
  // the run's X chunk and the zero block, the pairs' sums wait there and are
  // written after the run's last step, so that a short run's outputs (a
  // single product's, a tail claim's) reach memory at its end rather than
  // one pair at a time while the whole chip streams.  Slot j holds the j-th
  // pair emitted ([r][lane] floats): the pair of the j-th odd tile of the
  // run, or the run's last tile alone when that tile is even, so its
  // offsets follow from j.  Long runs (the dense verify pass) keep the
  // clock-window deferral.
  constexpr bool kHoldable = (EPI == kEpiStore || EPI == kEpiArgmax) && PF == kPrefetchTiled && N >= kDeferMinN;
  const int tlast = tile0 + cnt - 1;
  const int nodd = ((tlast + 1) >> 1) - (tile0 >> 1);  // odd tiles: each ends a pair
  const int npairs = nodd + ((tlast & 1) == 0 ? 1 : 0);
  const uint32_t xend = (uint32_t)nst * (uint32_t)kStep * 2u * N;  // bytes of the staged X chunk
  constexpr uint32_t kHoldSlot = 256u * kStores;
  const int nwv = (int)(blockDim.x >> 6);
  const int hslots =
      kHoldable ? min(kHoldMax, (int)((kZeroOffset<N>() - min(xend, kZeroOffset<N>())) / nwv / kHoldSlot)) : 0;
  const bool hold = kHoldable && !blocked && obase != nullptr && npairs <= hslots;
  char* const hbase =
      kHoldable ? lds + xend + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * hslots * kHoldSlot
                : lds;
  int hcount = 0;
  bool emitted = false;

  // next step to compute: tile ci, step cst
  int ci = 0, cst = 0;
  auto compute_next = [&](int slot) {
    const uint32_t xo = xoff + (uint32_t)cst * xstep;
    if constexpr (FP8) {
      segment(c0[slot], xo);
      segment(c1[slot], xo + 128u * N);
    } else if constexpr (VALU) {
      half_valu(c0[slot], sw[slot].x, 0, cst);
      half_valu(c1[slot], sw[slot].y, 1, cst);
    } else {
      half(c0[slot], sw[slot].x, xo);
      half(c1[slot], sw[slot].y, xo + 256u * N);
    }
    const bool fin = cst == nst - 1;
    if constexpr (VALU) {
      if (fin) {
        // the four k groups of row c, then the MFMA epilogue's layout
#pragma unroll
        for (int n = 0; n < N; ++n) {
          accv[n] += __shfl_xor(accv[n], 16);
          accv[n] += __shfl_xor(accv[n], 32);
        }
        const int nb = (lane & 16) ? 4 : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float v = 0.f;
#pragma unroll
          for (int n = 0; n < N; ++n) v = (n == nb + r) ? accv[n] : v;
          acc[r] = lane < 32 ? v : 0.f;
        }
#pragma unroll
        for (int n = 0; n < N; ++n) accv[n] = 0.f;
      }
    }
    if (fin && EPI == kEpiGlu) {
      // sums sit at lane 16 * (n / 4) + c (and again 32 lanes up); the gate
      // row c < 8 and the up row c + 8 of one f are 8 lanes apart
      const float gs = c < 8 ? mt.g : mt.g2;
      const int f = 8 * (tile0 + ci) + (c & 7);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[r]), false, false);
        const float v = gs * (__uint_as_float(p.x) + __uint_as_float(p.y));
        acc[r] = 0.f;
        const float up = __shfl_xor(v, 8);
        const int n = r + 4 * ((lane >> 4) & 1);
        const bool live = lane < 32 && c < 8 && n < N && f < F;
        so[r] = live ? (uint32_t)((n * F + f) * 2) : kDropOffset;
        sbits[r] = bf16_rne(__fdiv_rn(v, 1.0f + expf(-v)) * up);
      }
    } else if (fin) {
      const int t = tile0 + ci;
      const bool odd = (t & 1) != 0;
      // emit a pair (odd tile), or a lone even tile at the end of the share
      const bool emit = odd || ci == cnt - 1;
      if constexpr (kHoldable) emitted = emit;
      // store lanes: n = r + 4 * (lane / 32), m = m0 + lane % 32, where
      // m % 32 < 16 comes from the even tile and the rest from the odd one
      const int m = 16 * (odd ? t - 1 : t) + (lane & 31);
      const bool half_ok = (lane & 16) ? odd : (!odd || ci > 0);
      // the FP8 row scale of the lane's row (m = 16 t + c); 1 for partials
      const float rscale = split ? 1.0f : __uint_as_float(rv[slot]);
      // blocked: lane l and l + 32 hold the same (n, m), so both read the
      // slot of lane l % 32; lanes 0..31 write it
      f32x4 pin = {0.f, 0.f, 0.f, 0.f}, pout;
      const int pslot = tile0 + ci - ptile0;
      const int na = part_a_slots<N>(mt.kc);
      const uint32_t poff = (pslot < na ? 2u * (uint32_t)mt.kc * N + (uint32_t)pslot * kPartTileBytes
                                        : kPartOffset<N>() + (uint32_t)(pslot - na) * kPartTileBytes) +
                            (uint32_t)(lane & 31) * 16u;
      if (from_lds) pin = *reinterpret_cast<const f32x4*>(lds + poff);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // the swap gives every lane the low half's value (.x) and the high
        // half's (.y).  NVFP4: lanes l and l+32 hold blocks 0 and 1 of the
        // same (n, m); they are added in that order, so both lanes hold the
        // same sum.  FP8: lanes 0..31 hold rows n < 8 (the upper half holds
        // rows 8..15, which are zero), copied to both halves.
        const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[r]), false, false);
        float cur;
        if (blocked) {
          // the running sum over chunks: 0 + s_0 + s_1 + ..., in that order
          const float sc = FP8 ? __uint_as_float(p.x) : __uint_as_float(p.x) + __uint_as_float(p.y);
          const float run = pin[r] + sc;
          pout[r] = run;
          cur = FP8 ? rscale * run : gscale * run;
        } else {
          cur = FP8 ? rscale * __uint_as_float(p.x) : gscale * (__uint_as_float(p.x) + __uint_as_float(p.y));
        }
        acc[r] = 0.f;
        // sums sit at lane 16 * (n / 4) + m % 16 (and again 32 lanes up):
        // the 16-lane swap brings the even tile to rows 0 and 2 and the odd
        // tile to rows 1 and 3
        const u32x2 q = __builtin_amdgcn_permlane16_swap(__float_as_uint(odd ? prev[r] : cur), __float_as_uint(cur),
                                                         false, false);
        sum[r] = __uint_as_float(lane < 32 ? q.x : q.y);
        prev[r] = cur;
        if constexpr (EPI == kEpiArgmax) {
          const int mo = (tile0 + ci) * 16 + c;  // the lane's own row
          const bool own = lane < 32 && mo < mt.M && 4 * (lane >> 4) + r < N;
          const uint64_t key = own ? greedy_key(cur, mo) : 0ull;
          bestk[r] = key > bestk[r] ? key : bestk[r];
        }
        const int n = r + 4 * (lane >> 5);
        const bool live = emit && half_ok && m < mt.M && n < N && !to_lds;
        so[r] = live ? (uint32_t)((n * mt.M + m) * 4) : kDropOffset;
      }
      if (to_lds && lane < 32) *reinterpret_cast<f32x4*>(lds + poff) = pout;
    }
    bool held = false;
    if constexpr (kHoldable) {
      if (hold) {
        // the same min(N, 4) stores on every step, all dropped; a finished
        // pair goes to its slot
        held = true;
#pragma unroll
        for (int r = 0; r < kStores; ++r) bstore4(sum[r], ro, kDropOffset + 4u * r);
        if (fin && emitted) {
#pragma unroll
          for (int r = 0; r < kStores; ++r)
            *reinterpret_cast<float*>(hbase + (uint32_t)hcount * kHoldSlot + 256u * r + 4u * lane) = sum[r];
          ++hcount;
        }
      }
    }
    if (!held) {
      if constexpr (kDefer) {
        // the same min(N, 4) stores on every step; real offsets only when
        // the held pair is written (a new window, the end of a tile, or a
        // new pair to hold)
        const uint32_t win = (uint32_t)(__builtin_amdgcn_s_memrealtime() >> kDeferWindowBits);
        const bool emit_now = fin && so[0] != kDropOffset;
        const bool fl = pending && (win != pwin || fin);
#pragma unroll
        for (int r = 0; r < kStores; ++r) bstore4(psum[r], ro, fl ? pso[r] : kDropOffset + 4u * r);
        if (fl) pending = false;
        if (emit_now) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            psum[r] = sum[r];
            pso[r] = so[r];
          }
          pending = true;
          pwin = win;
        }
      } else {
#pragma unroll
        for (int r = 0; r < kStores; ++r) {
          if constexpr (EPI == kEpiGlu)
            bstore2(sbits[r], ro, fin ? so[r] : kDropOffset);
          else
            bstore4(sum[r], ro, fin ? so[r] : kDropOffset);
        }
      }
    }
    if (++cst == nst) { cst = 0; ++ci; }
  };

  const int Q = cnt * nst;
  // The prologue issues each step's memory operations in the order the
  // loop does (the stores, here all dropped and each to its own offset so
  // none is merged away, then the loads), so that at the loop header the
  // count of operations after each slot's load is the same on entry and on
  // the back edge and the vmcnt waits can be exact.
#pragma unroll
  for (int i = 0; i < PF; ++i) {
#pragma unroll
    for (int r = 0; r < kStores; ++r) {
      if constexpr (EPI == kEpiGlu)
        bstore2(0u, ro, kDropOffset + 4u * (4 * i + r));
      else
        bstore4(0.0f, ro, kDropOffset + 4u * (4 * i + r));
    }
    load_next(i);
  }
  stage();
  int q0 = 0;
  for (; q0 + PF <= Q; q0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      compute_next(i);
      load_next(i);
    }
  }
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (q0 + i < Q) compute_next(i);
  if constexpr (kDefer) {
    // the last pair of the run, if still held
    if (pending) {
#pragma unroll
      for (int r = 0; r < kStores; ++r) bstore4(psum[r], ro, pso[r]);
    }
  }
  if (kHoldable && hold) {
    // the held pairs, with the offsets the epilogue gives them
    for (int j = 0; j < hcount; ++j) {
      const bool podd = j < nodd;
      const int t = podd ? (tile0 | 1) + 2 * j : tlast;
      const int m = 16 * (podd ? t - 1 : t) + (lane & 31);
      const bool half_ok = (lane & 16) ? podd : (!podd || t > tile0);
#pragma unroll
      for (int r = 0; r < kStores; ++r) {
        const int n = r + 4 * (lane >> 5);
        const bool live = half_ok && m < mt.M && n < N;
        bstore4(*reinterpret_cast<const float*>(hbase + (uint32_t)j * kHoldSlot + 256u * r + 4u * lane), ro,
                live ? (uint32_t)((n * mt.M + m) * 4) : kDropOffset);
      }
    }
  }
}

// ---- single products with few tiles per CU: tiles split across waves --------
// A product of T tiles x S steps is cut into C short K chunks ("tile-chunks"
// of s steps; chunk-major order: every tile's chunk 0, then chunk 1, ...).
// Each workgroup takes a run of whole tile-chunks of about U / G steps and
// splits the run's steps into one equal piece per wave, so that every CU
// streams about the same bytes with all its waves from the start, however
// few tiles there are.  A wave streams its piece as one sequence (a tile's
// steps of one chunk are contiguous in the tiled layout, the next tile's
// follow) and leaves the sums of each tile-chunk it touched in an LDS slot;
// the workgroup adds, per tile-chunk, its waves' slots in wave order (k
// order).  With one chunk the tile is stored as y; otherwise the tile-chunk
// sum is a part in the workspace, and the workgroup whose part is the C-th
// to arrive at the tile (an arrival counter per tile) adds the C parts in
// chunk order and stores y.  The cut depends on (M, K) and the grid only, so
// column n has the same bits for every N.

// s_waitcnt that waits only for the vector-memory count to reach V (the
// gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 at
// their maximum, i.e. not waited for).
template <int V>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(V >= 0 && V < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}

// Steps [e0, e1) of chunk `chunk` (chunk-local index e = tile * nst + step)
// streamed by this wave; the sums of the j-th tile it touches go to LDS at
// slots + 512 j (lanes 0..31: four floats, rows n = 4 (lane / 16) + r of
// output m = 16 tile + lane % 16).  X of the chunk was requested before this
// call; once the wave's first PF steps of weight loads are in flight, it
// waits for X alone (loads complete in order) and synchronizes the workgroup.
template <int N, bool FP8>
__device__ void split_piece(const DevMat& mt, int chunk, int nst, int e0, int e1, const char* lds, char* slots) {
  constexpr int PF = kSplitPrefetch;
  constexpr int kStep = FP8 ? kFp8TileStepK : kTileStepK;
  constexpr uint32_t kBlock = FP8 ? kFp8TileBlockBytes : kTileBlockBytes;
  constexpr int kLoads = FP8 ? 2 : 3;  // vector-memory loads per step
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int cnt = e1 - e0;
  if (cnt <= 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    return;
  }
  const uint32_t steps_per_row = (uint32_t)((mt.K + kStep - 1) / kStep);
  const uint32_t base_step = (uint32_t)(chunk * (mt.kc / kStep));
  const uint64_t total = (uint64_t)mt.ntiles * steps_per_row * kBlock;  // < 2^32 (checked on the host)
  const __amdgpu_buffer_rsrc_t rw = make_rsrc_uniform(mt.w, total);
  const uint32_t vc = 16u * lane;
  const uint32_t vs = (uint32_t)kTileCodeBytes + 8u * (uint32_t)(((lane >> 5) << 4) + c);
  bool active;
  uint32_t xoff, xstep;
  if constexpr (FP8) {
    active = c < N;
    xoff = active ? (uint32_t)((2 * g * N + c) * 16) : kZeroOffset<N>();
    xstep = active ? 256u * N : 0u;
  } else {
    active = ((c >> 3) == (g >> 1)) && ((c & 7) < N);
    xoff = active ? (uint32_t)((g * N + (c & 7)) * 16) : kZeroOffset<N>();
    xstep = active ? 512u * N : 0u;
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 c0[PF], c1[PF];
  u32x2 sw[PF];
  const int t_first = e0 / nst;
  // next step to load (past the end: the last one again)
  int lt = t_first, ls = e0 - t_first * nst, ln = 0;
  auto load_next = [&](int slot) {
    const uint32_t b = ((uint32_t)lt * steps_per_row + base_step + (uint32_t)ls) * kBlock;
    c0[slot] = bload16t(rw, b + vc);
    c1[slot] = bload16t(rw, b + 1024u + vc);
    if constexpr (!FP8) sw[slot] = bload8t(rw, b + vs);
    if (ln < cnt) {
      ++ln;
      if (ln < cnt && ++ls == nst) { ls = 0; ++lt; }
    }
  };
  auto half = [&](const u32x4& e, uint32_t sb, uint32_t xo) {
    const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, false);
    const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(sb, true);
    const float stv[4] = {s01.x, s01.y, s23.x, s23.y};
    bf16x8 a[4], b[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) a[t] = lds_read16(lds, xo + t * 64u * N);
#pragma unroll
    for (int t = 0; t < 4; ++t) b[t] = e2m1x8_to_bf16(e[t]);
    f32x4 part[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      part[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], b[t], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(stv[t], part[t][r], acc[r]);
  };
  auto segment = [&](const u32x4& d, uint32_t xo) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) a[u] = lds_read16(lds, xo + u * 16u * N);
#pragma unroll
    for (int u = 0; u < 2; ++u) b[u] = e4m3x8_to_bf16(d[2 * u], d[2 * u + 1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
  };
  // next step to compute
  int ct = t_first, cs = e0 - t_first * nst, cn = 0;
  auto compute_next = [&](int slot) {
    const uint32_t xo = xoff + (uint32_t)cs * xstep;
    if constexpr (FP8) {
      segment(c0[slot], xo);
      segment(c1[slot], xo + 128u * N);
    } else {
      half(c0[slot], sw[slot].x, xo);
      half(c1[slot], sw[slot].y, xo + 256u * N);
    }
    ++cn;
    if (cs == nst - 1 || cn == cnt) {
      // the swap gives every lane the low half's value (.x) and the high
      // half's (.y): NVFP4 blocks 0 and 1 of one (n, m), added in that
      // order; FP8 rows n < 8 (the high half is zero)
      f32x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const u32x2 p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[r]), __float_as_uint(acc[r]), false, false);
        o[r] = FP8 ? __uint_as_float(p.x) : __uint_as_float(p.x) + __uint_as_float(p.y);
        acc[r] = 0.f;
      }
      if (lane < 32) *reinterpret_cast<f32x4*>(slots + 512 * (ct - t_first) + 16 * lane) = o;
    }
    if (++cs == nst) { cs = 0; ++ct; }
  };
#pragma unroll
  for (int i = 0; i < PF; ++i) load_next(i);
  wait_vmcnt<PF * kLoads>();
  __syncthreads();
  int q0 = 0;
  for (; q0 + PF <= cnt; q0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      compute_next(i);
      load_next(i);
    }
  }
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (q0 + i < cnt) compute_next(i);
}

// Tile-chunk parts in the workspace: part (chunk, tile) holds 16 rows x N
// columns, float (m, n) at word m N + n; lane l < 32 of a workgroup's sums
// holds columns n = 4 (l / 16) + r of row m = l % 16.
template <int N>
__device__ __forceinline__ void store_part(const f32x4& v, __amdgpu_buffer_rsrc_t r, uint32_t base, int lane) {
  const int h = lane >> 4, m = lane & 15;
  const int cnt = N - 4 * h;  // columns this lane holds (lanes 0..31 only)
  const uint32_t off = base + (uint32_t)(m * N + 4 * h) * 4u;
  if (lane >= 32 || cnt <= 0) return;
  // written through to memory (device scope): a completed store is what
  // another workgroup's device-scope load returns
  if (cnt >= 4) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kAuxOut);
  else if (cnt == 3)
    __builtin_amdgcn_raw_buffer_store_b96(u32x3{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2])},
                                          r, (int)off, 0, kAuxOut);
  else if (cnt == 2) __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f32x2{v[0], v[1]}), r, (int)off, 0, kAuxOut);
  else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, (int)off, 0, kAuxOut);
}
template <int N>
__device__ __forceinline__ f32x4 load_part(__amdgpu_buffer_rsrc_t r, uint32_t base, int lane) {
  const int h = (lane >> 4) & 1, m = lane & 15;
  const int cnt = N - 4 * h;
  const uint32_t off = base + (uint32_t)(m * N + 4 * h) * 4u;
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (cnt >= 4) v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAuxOut));
  else if (cnt == 3) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b96(r, (int)off, 0, kAuxOut);
    v = f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), 0.f};
  } else if (cnt == 2) {
    const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAuxOut));
    v = f32x4{__uint_as_float(w[0]), __uint_as_float(w[1]), 0.f, 0.f};
  } else if (cnt == 1) {
    v[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kAuxOut));
  }
  return v;
}

template <int N, bool FP8>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(DevMat mt, uint32_t* __restrict__ counters,
                                                              float* __restrict__ parts, int slots_per_wave) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  constexpr int kW = kSplitThreads / 64;
  constexpr int kStep = FP8 ? kFp8TileStepK : kTileStepK;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int S = (mt.K + kStep - 1) / kStep;
  const int T = mt.ntiles, C = mt.nchunks;
  const int s_full = mt.kc / kStep, s_last = S - (C - 1) * s_full;
  // The run: workgroups [G c / C, G (c + 1) / C) take chunk c, each an
  // equal share of its tiles [ta, tb) (whole tile-chunks), so that a run
  // never leaves its chunk and X is staged once.
  const int G = gridDim.x, g = blockIdx.x;
  const int ch = (C * (g + 1) - 1) / G;
  const int g0 = G * ch / C, gc = G * (ch + 1) / C - g0;
  const int ta = T * (g - g0) / gc, tb = T * (g - g0 + 1) / gc;
  const int la = ta * (ch == C - 1 ? s_last : s_full), lb = tb * (ch == C - 1 ? s_last : s_full);
  char* const slots = lds + kPartOffset<N>();
  char* const my_slots = slots + (size_t)wave * slots_per_wave * 512;
  __shared__ int s_arrive[kSplitArrivalsMax];  // tile-chunks (c T + t) this workgroup wrote parts of
  __shared__ int s_tile0[kSplitThreads / 64], s_tile1[kSplitThreads / 64];
  __shared__ int s_narrive;
  if (threadIdx.x == 0) s_narrive = 0;
  for (int i = threadIdx.x; i < kZeroBytes<N>() / 16; i += blockDim.x)
    *reinterpret_cast<u32x4*>(lds + kZeroOffset<N>() + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  const __amdgpu_buffer_rsrc_t rr = make_rsrc_uniform(mt.rs, FP8 ? (uint64_t)mt.M * 4u : 0u);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc_uniform(mt.y, (uint64_t)N * mt.M * 4u);
  const __amdgpu_buffer_rsrc_t rp = make_rsrc_uniform(parts, (uint64_t)C * T * kSplitPartBytes);
  auto store_y = [&](int t, const f32x4& v) {
    const int m = 16 * t + (lane & 15);
    // the output scale of lane l's row m = 16 t + l % 16 (rows past M read 0)
    const float sc = FP8 ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rr, (int)(m * 4), 0, 0)) : mt.g;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * (lane >> 4) + r;
      if (lane < 32 && n < N && m < mt.M) bstore4(sc * v[r], ro, (uint32_t)((n * mt.M + m) * 4));
    }
  };

  if (ta < tb) {
    const int nst = ch == C - 1 ? s_last : s_full;
    const int k0 = ch * mt.kc;
    const int klen = min(mt.kc, mt.K - k0);
    // this chunk of X is requested before the pieces' first weight loads;
    // split_piece waits for it
    stage_x_direct<N>(lds, mt.x, mt.K, k0, klen, nst * (kStep / 8));
    __builtin_amdgcn_sched_barrier(0);
    const int e0 = la + (lb - la) * wave / kW, e1 = la + (lb - la) * (wave + 1) / kW;
    // each wave's first and last tile, for the sums below
    if (lane == 0) {
      s_tile0[wave] = e0 / nst;
      s_tile1[wave] = e0 < e1 ? (e1 - 1) / nst : -1;
    }
    split_piece<N, FP8>(mt, ch, nst, e0, e1, lds, my_slots);
    __syncthreads();
    // per tile of the run: the sums of the waves that touched it, in wave
    // order (every wave's slot read issued before the additions)
    int wt0[kW], wt1[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      wt0[w] = s_tile0[w];
      wt1[w] = s_tile1[w];
    }
    for (int t = ta + wave; t < tb; t += kW) {
      f32x4 v[kW];
      bool use[kW];
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const int t0 = wt0[w], t1 = wt1[w];
        use[w] = t >= t0 && t <= t1;
        const int j = use[w] ? t - t0 : 0;
        v[w] = *reinterpret_cast<const f32x4*>(slots + ((size_t)w * slots_per_wave + j) * 512 + 16 * (lane & 31));
      }
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kW; ++w)
        if (use[w])
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[r] += v[w][r];
      if (C == 1) {
        store_y(t, sum);
      } else {
        store_part<N>(sum, rp, (uint32_t)(ch * T + t) * kSplitPartBytes, lane);
        if (lane == 0) {
          const int i = atomicAdd(&s_narrive, 1);
          if (i < kSplitArrivalsMax) s_arrive[i] = ch * T + t;  // (the host keeps i below the bound)
        }
      }
    }
  }
  // arrivals, once every wave's part stores have completed (written
  // through, so visible device-wide): one per part, all at once
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int narrive = min(s_narrive, kSplitArrivalsMax);
  if (narrive == 0) return;
  __shared__ int s_done[kSplitArrivalsMax];  // the tile, if this part completed it, else -1
  if ((int)threadIdx.x < narrive) {
    const int t = s_arrive[threadIdx.x] % T;
    const uint32_t old = __hip_atomic_fetch_add(&counters[t], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_done[threadIdx.x] = (int)old + 1 == C ? t : -1;
  }
  __syncthreads();
  // the tiles this workgroup completes: the C parts in chunk order
  for (int i = wave; i < narrive; i += kW) {
    const int t = s_done[i];
    if (t < 0) continue;
    // (every part's load in flight at once, then added in chunk order)
    f32x4 v[kSplitChunksMax];
#pragma unroll
    for (int j = 0; j < kSplitChunksMax; ++j)
      if (j < C) v[j] = load_part<N>(rp, (uint32_t)(j * T + t) * kSplitPartBytes, lane);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kSplitChunksMax; ++j)
      if (j < C)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum[r] += v[j][r];
    store_y(t, sum);
    if (lane == 0) __hip_atomic_store(&counters[t], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---- one FP8-row unit ------------------------------------------------------
template <int N, int PF>
__device__ void fp8_unit(const DevMat& mt, int chunk, int tile, const char* lds) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const int k0 = chunk * mt.kc;
  const int klen = min(mt.kc, mt.K - k0);
  const int nseg = (klen + 63) >> 6;
  const uint64_t rowb = (uint64_t)mt.K;
  const uint64_t m0 = (uint64_t)tile * 16;
  const uint64_t cstart = m0 * rowb + (uint64_t)k0;
  const __amdgpu_buffer_rsrc_t rc = make_rsrc(mt.w + cstart, (uint64_t)mt.M * rowb - cstart);
  const uint32_t voc = (uint32_t)(c * rowb) + 16u * g;

  // A operand (X): rows i < N hold column i; k slots of group g at step u are
  // k = 16g + 8u .. 16g + 8u + 7 of the segment.
  const bool active = c < N;
  const uint32_t xoff = active ? (uint32_t)((2 * g * N + c) * 16) : kZeroOffset<N>();
  const uint32_t xstep = active ? 128u * N : 0u;
  // In a chunk whose length is not a multiple of 64, lanes past its end in
  // the last segment hold bytes of the next chunk or row; they are zeroed
  // (an E4M3 NaN times a zero X would still be NaN).
  const int tail_bytes = klen & 63;
  const bool lane_past_tail = 16 * g >= tail_bytes;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 cw[PF];
  const int last = nseg - 1;
  auto load = [&](int seg, int slot) { cw[slot] = bload16(rc, voc + 64u * min(seg, last)); };
  auto compute = [&](int slot, int seg) {
    u32x4 d = cw[slot];
    if (tail_bytes != 0 && seg == last && lane_past_tail) d = u32x4{0u, 0u, 0u, 0u};
    const uint32_t xo = xoff + (uint32_t)seg * xstep;
    bf16x8 a[2], b[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) a[u] = lds_read16(lds, xo + u * 16u * N);
#pragma unroll
    for (int u = 0; u < 2; ++u) b[u] = e4m3x8_to_bf16(d[2 * u], d[2 * u + 1]);
#pragma unroll
    for (int u = 0; u < 2; ++u) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u], b[u], acc, 0, 0, 0);
  };

#pragma unroll
  for (int i = 0; i < PF; ++i) load(i, i);
  int s0 = 0;
  for (; s0 + PF <= nseg; s0 += PF) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      compute(i, s0 + i);
      load(s0 + i + PF, i);
    }
  }
#pragma unroll
  for (int i = 0; i < PF; ++i)
    if (s0 + i < nseg) compute(i, s0 + i);

  const int m = tile * 16 + c;
  const float rsc = (lane < 32 && m < mt.M) ? mt.rs[m] : 0.0f;
  const float sum[4] = {acc[0], acc[1], acc[2], acc[3]};
  finish_tile<N>(mt, chunk, tile, sum, rsc);
}

// ---- grid barrier of the single-launch chain --------------------------------
// A split barrier: a workgroup arrives once its stores of a phase are
// issued and waits, later, before it reads what the other workgroups stored
// (so that it can issue its next weight loads in between).  ctl->count
// counts every arrival of the launch; a workgroup's b-th wait ends once the
// count has reached b times the grid (its target, kept in LDS), so the
// barrier costs the last arrival's one atomic and the waiters' next poll.
// Every wait is bounded: after kSpinLimit polls it sets ctl->error and goes
// on, so that the grid always drains even if a workgroup never arrives (the
// results are then not defined).  Only a launch that keeps every workgroup
// resident (a cooperative launch) may use it.  grid_finish, after a
// workgroup's last wait, counts it out; the last one sets count and done
// back to zero for the next launch (every other workgroup has passed every
// wait by then).
//
// There are no fences.  Everything one phase hands to the next (s, the
// down sums, h, the sums of squares) is stored through the L2 and read with
// device-scope loads (kAuxCoherent), so it never sits in a cache another
// XCD cannot see; an arrival is counted only after the workgroup's stores
// have completed (s_waitcnt), and a waiting workgroup issues its reads
// only after it has seen the barrier open.  An agent-scope release fence
// is a writeback of the XCD's whole L2: per-workgroup timelines showed the
// last arrival landing 15-20 us after the workgroup's stores had drained.
struct GridSync {
  ChainCtl* ctl;
  uint32_t* s_target;  // LDS: the count that opens this workgroup's next wait
};
constexpr uint32_t kSpinLimit = 1u << 19;

__device__ __forceinline__ void grid_arrive(const GridSync& gs) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's stores have completed
  __syncthreads();                // ... and every other wave's
  if (threadIdx.x == 0) {
    *gs.s_target += gridDim.x;
    __hip_atomic_fetch_add(&gs.ctl->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__device__ __forceinline__ void grid_wait(const GridSync& gs) {
  if (threadIdx.x == 0) {
    ChainCtl* c = gs.ctl;
    const uint32_t target = *gs.s_target;
    // (relaxed device-scope polls: each reads the counter from memory)
    for (uint32_t it = 0; __hip_atomic_load(&c->count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target; ++it) {
      if (it == kSpinLimit) {
        __hip_atomic_fetch_or(&c->error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void grid_finish(const GridSync& gs) {
  if (threadIdx.x == 0) {
    ChainCtl* c = gs.ctl;
    if (__hip_atomic_fetch_add(&c->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
      __hip_atomic_store(&c->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&c->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---- the persistent kernel -------------------------------------------------
// Workgroup w processes units [range[w].begin, range[w+1].begin) of the
// global unit list (matrix-major, then chunk, then tile; then tile, then
// chunk for a blocked split).  For a single
// matrix (mats == nullptr) the split is computed here, equal by units.
// SYNC (the single-launch chain, one matrix, no ranges table: equal
// shares): the first staging of the call first waits at the grid barrier
// (the matrix's X is made by the previous phase), after the run's first
// weight loads are issued; a workgroup with no units waits at the end.
template <int N, int MODE, bool SYNC = false>
__device__ __forceinline__ void stream_body(const DevMat* __restrict__ mats, const WgRange* __restrict__ ranges,
                                            const DevMat& one, char* lds, const GridSync* gs = nullptr) {
  // wave-uniform values are pinned to scalar registers so that buffer
  // resources built from them stay uniform
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  constexpr int nwaves = threads_for_mode<MODE>() / 64;

  int64_t u, u_end;
  int mi;
  if (mats == nullptr || ranges == nullptr) {
    const int64_t total = mats ? (int64_t)mats[0].nchunks * mats[0].ntiles : (int64_t)one.nchunks * one.ntiles;
    u = total * blockIdx.x / gridDim.x;
    u_end = total * (blockIdx.x + 1) / gridDim.x;
    mi = 0;
  } else {
    u = ranges[blockIdx.x].begin;
    u_end = ranges[blockIdx.x + 1].begin;
    mi = ranges[blockIdx.x].mat;
  }

  uint64_t bestk[4] = {0ull, 0ull, 0ull, 0ull};  // head acceptance

  // zero block read by lanes whose A-operand slots must be zero
  for (int i = threadIdx.x; i < kZeroBytes<N>() / 16; i += blockDim.x)
    *reinterpret_cast<u32x4*>(lds + kZeroOffset<N>() + 16 * i) = u32x4{0u, 0u, 0u, 0u};

  // a verify pass: after its static range the workgroup claims chunks of
  // the dynamic tail until none is left
  // (only the tiled kernel has the claim loop: plans of other kernels have no
  // tail, and the loop's presence alone slowed the plain-layout kernels)
  DynSched* dyn = ((MODE == kModeTiled || MODE == kModeTiledValu) && mats)
                      ? reinterpret_cast<DynSched*>(const_cast<WgRange*>(ranges) + gridDim.x + 1)
                      : nullptr;
  // a pass without a tail takes no claims (a claim is a device-scope round
  // trip that the last workgroup's exit would wait for)
  if (dyn && dyn->count == 0) dyn = nullptr;
  __shared__ uint32_t s_claim;
  bool waited = false;
  int bchunk = 0;  // blocked split: the next chunk of the current block
  // the barrier at the start of a staging (protects the LDS still read by
  // the previous run; with SYNC the first one is the grid barrier)
  auto sync_first = [&]() {
    if constexpr (SYNC) {
      if (!waited) {
        waited = true;
        grid_wait(*gs);
        return;
      }
    }
    __syncthreads();
  };

  for (;;) {
  while (u < u_end) {
    const DevMat mt = mats ? mats[mi] : one;
    const int64_t mend = mt.unit0 + (int64_t)mt.nchunks * mt.ntiles;
    if (u >= mend) { ++mi; continue; }
    const int64_t local = u - mt.unit0;
    // The segment: units [first, run_end) of one K chunk, tile = unit - ubase.
    // A blocked split's units are tile-major (tile * nchunks + chunk) and a
    // range holds whole tiles: the run takes them block_tiles at a time, all
    // chunks of such a block in turn (bchunk counts them), and moves u past
    // the block after its last chunk.
    int chunk, ptile0 = -1;
    int64_t first, run_end, ubase;
    if (mt.tb > 0) {
      const int nc = mt.nchunks;
      const int t0 = (int)(local / nc);
      const int t1 = min(t0 + block_tiles<N>(mt.kc), (int)((min(u_end, mend) - mt.unit0) / nc));
      chunk = bchunk;
      first = t0;
      run_end = t1;
      ubase = 0;
      ptile0 = t0;
      if (++bchunk == nc) {
        bchunk = 0;
        u = mt.unit0 + (int64_t)t1 * nc;
      }
    } else {
      chunk = (int)(local / mt.ntiles);
      ubase = mt.unit0 + (int64_t)chunk * mt.ntiles;
      first = u;
      run_end = min(u_end, ubase + mt.ntiles);
      u = run_end;
    }
    const int k0 = chunk * mt.kc;
    const int klen = min(mt.kc, mt.K - k0);
    // X is staged (zero-padded) to whole steps of the format, which every
    // lane of the last step reads
    const int seg_k = mt.fmt == kFmtNvfp4Tiled    ? kTileStepK
                      : mt.fmt == kFmtFp8RowTiled ? kFp8TileStepK
                      : mt.fmt == kFmtNvfp4       ? 128
                                                  : 64;
    const int kc_pad = ((klen + seg_k - 1) / seg_k) * (seg_k / 8);
    // every wave calls this once per run (the barriers protect the LDS
    // still read by the previous run, then publish the new X)
    // The 16-wave chain kernel (kModeTiledWide) issues the first batch of X
    // before its weight loads (its staging is on the critical path of a
    // short launch); the verify pass measured about 1% slower that way and
    // stages after them.  With SYNC, X is made by the previous phase, so
    // nothing of it may be loaded before the grid barrier.
    constexpr bool kEarlyX = MODE == kModeTiledWide && !SYNC;
    u32x4 xpre[kStageLoads];
    auto pre = [&]() {
      if constexpr (kEarlyX) stage_x_load<N>(xpre, mt.x, mt.K, k0, klen, kc_pad, (int)threadIdx.x);
    };
    auto stage = [&]() {
      sync_first();
      if constexpr (kEarlyX) {
        stage_x_rest<N>(xpre, lds, mt.x, mt.K, k0, klen, kc_pad);
      } else if constexpr (MODE == kModeTiled || MODE == kModeTiledArgmax || MODE == kModeTiledValu) {
        stage_x_direct<N>(lds, mt.x, mt.K, k0, klen, kc_pad);
        __builtin_amdgcn_s_waitcnt(0);  // this wave's loads (and every older one) are done
      } else if constexpr (SYNC) {
        // X (s) was written earlier in this launch: device-scope loads
        stage_x_direct<N, kAuxCoherent>(lds, mt.x, mt.K, k0, klen, kc_pad);
        __builtin_amdgcn_s_waitcnt(0);
      } else {
        stage_x<N>(lds, mt.x, mt.K, k0, klen, kc_pad);
      }
      __syncthreads();
    };
    // tiled formats: wave w takes the w-th of nwaves equal shares of the
    // run's consecutive tiles
    const int64_t len = run_end - first;
    const int64_t share0 = first + len * wave / nwaves, share1 = first + len * (wave + 1) / nwaves;
    if constexpr (MODE == kModeTiled) {
      if (mt.fmt == kFmtFp8RowTiled)
        tiled_run<N, kPrefetchTiled, true, kEpiStore, true>(mt, chunk, share0, share1, ubase, ptile0, lds, bestk, pre,
                                                             stage);
      else
        tiled_run<N, kPrefetchTiled, false, kEpiStore, true>(mt, chunk, share0, share1, ubase, ptile0, lds, bestk, pre,
                                                              stage);
    } else if constexpr (MODE == kModeTiledValu) {
      if (mt.fmt == kFmtFp8RowTiled)
        tiled_run<N, kPrefetchTiled, true, kEpiStore, true>(mt, chunk, share0, share1, ubase, ptile0, lds, bestk, pre,
                                                             stage);
      else
        tiled_run<N, kPrefetchTiled, false, kEpiStore, true, true>(mt, chunk, share0, share1, ubase, ptile0, lds,
                                                                    bestk, pre, stage);
    } else if constexpr (MODE == kModeTiledArgmax) {
      if (mt.fmt == kFmtFp8RowTiled)
        tiled_run<N, kPrefetchTiled, true, kEpiArgmax, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, pre,
                                                               stage);
      else
        tiled_run<N, kPrefetchTiled, false, kEpiArgmax, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, pre,
                                                                stage);
    } else if constexpr (MODE == kModeTiledGlu) {
      NormBatch nb;
      auto pre_norm = [&]() {
        if constexpr (!SYNC) norm_first<N, false>(nb, mt, kc_pad);
      };
      auto stage_norm_x = [&]() {
        sync_first();
        if constexpr (SYNC) norm_first<N, true>(nb, mt, kc_pad);
        stage_norm<N, SYNC>(nb, lds, mt, kc_pad, first - mt.unit0, run_end - mt.unit0,
                            (int64_t)mt.nchunks * mt.ntiles);
        __syncthreads();
      };
      tiled_run<N, kPrefetchWide, false, kEpiGlu, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, pre_norm,
                                                  stage_norm_x);
    } else if constexpr (MODE == kModeTiledWide) {
      if (mt.fmt == kFmtFp8RowTiled)
        tiled_run<N, kPrefetchWide, true, kEpiStore, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, pre, stage);
      else
        tiled_run<N, kPrefetchWide, false, kEpiStore, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, pre, stage);
    } else {
      // (written out rather than through stage(): a by-reference lambda on
      // this path kept the descriptor out of scalar registers and made the
      // 128-VGPR kernels spill)
      __syncthreads();
      stage_x<N>(lds, mt.x, mt.K, k0, klen, kc_pad);
      __syncthreads();
      auto staged = []() {};
      if (MODE == kModeMixed && mt.fmt == kFmtNvfp4Tiled) {
        tiled_run<N, 1, false, kEpiStore, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, staged, staged);
      } else if (MODE == kModeMixed && mt.fmt == kFmtFp8RowTiled) {
        tiled_run<N, 1, true, kEpiStore, false>(mt, chunk, share0, share1, ubase, -1, lds, bestk, staged, staged);
      } else {
        for (int64_t uu = first + wave; uu < run_end; uu += nwaves) {
          const int tile = (int)(uu - ubase);
          if constexpr (MODE == kModeNvfp4Aligned) {
            nvfp4_unit<N, kPrefetch, true>(mt, chunk, tile, lds);
          } else if constexpr (MODE == kModeNvfp4) {
            nvfp4_unit<N, kPrefetchGeneric, false>(mt, chunk, tile, lds);
          } else if constexpr (MODE == kModeFp8) {
            fp8_unit<N, kPrefetch>(mt, chunk, tile, lds);
          } else {
            if (mt.fmt == kFmtNvfp4)
              nvfp4_unit<N, kPrefetchGeneric, false>(mt, chunk, tile, lds);
            else
              fp8_unit<N, kPrefetchGeneric>(mt, chunk, tile, lds);
          }
        }
      }
    }
  }
  if (!dyn) break;
  __syncthreads();  // every wave has read the previous claim
  if (threadIdx.x == 0) {
    // this launch's values of the counter are L (count + grid) + i
    const uint64_t raw = __hip_atomic_fetch_add(&dyn->next, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_claim = (uint32_t)(raw % ((uint64_t)dyn->count + gridDim.x));
  }
  __syncthreads();
  const uint32_t idx = s_claim;
  if (idx >= (uint32_t)dyn->count) break;
  const DynClaim* const claims = reinterpret_cast<const DynClaim*>(dyn + 1);
  u = claims[idx].begin;
  u_end = claims[idx + 1].begin;
  mi = claims[idx].mat;
  }
  if constexpr (SYNC) {
    if (!waited) grid_wait(*gs);
  }

  if constexpr (MODE == kModeTiledArgmax) {
    // the wave's best row per column: over the 16 row lanes of each half
    // (lanes 0..15 hold columns r, lanes 16..31 columns 4 + r) ...
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        const uint64_t o = __shfl_xor(bestk[r], off);
        bestk[r] = o > bestk[r] ? o : bestk[r];
      }
    // ... then over the waves (LDS past the zero block), one key per column
    uint64_t* wb = reinterpret_cast<uint64_t*>(lds + kZeroOffset<N>() + kZeroBytes<N>());
    if (lane == 0 || lane == 16)
#pragma unroll
      for (int r = 0; r < 4; ++r) wb[wave * 8 + (lane >> 2) + r] = bestk[r];
    __syncthreads();
    if (threadIdx.x < 8) {
      uint64_t b = 0ull;
      for (int w = 0; w < nwaves; ++w) {
        const uint64_t o = wb[w * 8 + threadIdx.x];
        b = o > b ? o : b;
      }
      one.best[(size_t)blockIdx.x * 8 + threadIdx.x] = b;
    }
  }
}

template <int N, int MODE>
__global__ __launch_bounds__(threads_for_mode<MODE>()) void stream_kernel(const DevMat* __restrict__ mats,
                                                                          const WgRange* __restrict__ ranges,
                                                                          DevMat one) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  stream_body<N, MODE>(mats, ranges, one, lds);
}

// The verify pass with the column count read from device memory (the
// crit-hub engine card, section "Design", row "Decode": the round's graph
// runs the verify pass for the drafts made, chosen on the device).  One
// kernel holds the tiled pass for every N; the plan is the one for N = 8,
// whose LDS, descriptors and partial-sum space cover every smaller N, and
// the body for n computes exactly what stream_kernel<n, kModeTiled> does.
__device__ __forceinline__ int device_n(const int32_t* n_dev) {
  const int n = __builtin_amdgcn_readfirstlane(*n_dev);
  return n < 1 ? 1 : n > 8 ? 8 : n;
}

// (inlined: as a called function each body needed a 280-byte stack frame
// and ran slower)
template <int N>
__device__ __forceinline__ void dyn_body(const DevMat* __restrict__ mats, const WgRange* __restrict__ ranges,
                                                   char* lds) {
  const DevMat none{};
  stream_body<N, kModeTiled>(mats, ranges, none, lds);
}

__global__ __launch_bounds__(kThreadsTiled) void stream_kernel_dyn(const DevMat* __restrict__ mats,
                                                                   const WgRange* __restrict__ ranges,
                                                                   const int32_t* __restrict__ n_dev) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  switch (device_n(n_dev)) {
    case 1: dyn_body<1>(mats, ranges, lds); break;
    case 2: dyn_body<2>(mats, ranges, lds); break;
    case 3: dyn_body<3>(mats, ranges, lds); break;
    case 4: dyn_body<4>(mats, ranges, lds); break;
    case 5: dyn_body<5>(mats, ranges, lds); break;
    case 6: dyn_body<6>(mats, ranges, lds); break;
    case 7: dyn_body<7>(mats, ranges, lds); break;
    default: dyn_body<8>(mats, ranges, lds); break;
  }
}

// ---- residual update of a chained MLP layer ---------------------------------
// Block (p, n) owns outputs m = kChainThreads p + i of column n:
//   h[n][m] += g * (part[0][n][m] + part[1][n][m] + ...)   (chunk order)
// for a down product split in K (one chunk: its y, already scaled, is
// added), and writes the sum of their squares (after the update) to
// ssp[n][p], the partials from which the next layer's RMSNorm takes its
// scale.  With no descriptor it only writes ssp.  The
// sum over a block is a fixed tree (butterfly within a wave, then the waves
// in order), so every run gives the same bits.
// The work of block (p, n) as above, by threads 0 .. kChainThreads - 1 of the
// calling workgroup (every thread calls it: it holds two barriers).
// COH (the single-launch chain): the down sums and h are read with
// device-scope loads and h and ssp written through the L2, since other
// workgroups of the same launch read and wrote them.
template <bool COH>
__device__ __forceinline__ void chain_reduce_block(float* __restrict__ h, const DevMat* __restrict__ down, int D,
                                                   int N, int n, int p, int P, float* __restrict__ ssp,
                                                   float* wsum) {
  const int t = (int)threadIdx.x;
  const int m = p * kChainThreads + t;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(h, (uint64_t)N * (uint64_t)D * 4u);
  auto ld = [&](const float* base, uint64_t elems, size_t i) -> float {
    if constexpr (COH)
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(base, elems * 4u), (int)(i * 4), 0,
                                                                  kAuxCoherent));
    else
      return base[i];
  };
  float v = 0.0f;
  if (t < kChainThreads && m < D) {
    const size_t o = (size_t)n * D + m;
    v = ld(h, (uint64_t)N * D, o);
    if (down) {
      const int nchunks = down->nchunks;
      float acc = 0.0f;
      if (nchunks > 1) {
        // eight chunks' loads in flight at a time, then added in chunk order
        constexpr int kBatch = 8;
        for (int c0 = 0; c0 < nchunks; c0 += kBatch) {
          float v[kBatch];
#pragma unroll
          for (int j = 0; j < kBatch; ++j)
            v[j] = c0 + j < nchunks ? ld(down->part, (uint64_t)nchunks * N * D, (size_t)(c0 + j) * N * D + o) : 0.0f;
#pragma unroll
          for (int j = 0; j < kBatch; ++j)
            if (c0 + j < nchunks) acc += v[j];
        }
        acc = down->g * acc;
      } else {
        acc = ld(down->y, (uint64_t)N * D, o);
      }
      v = v + acc;
      if constexpr (COH)
        bstore4(v, rh, (uint32_t)(o * 4));
      else
        h[o] = v;
    }
  }
  float sq = v * v;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off);
  if (t < kChainThreads && (t & 63) == 0) wsum[t >> 6] = sq;
  __syncthreads();
  if (t == 0) {
    float s = 0.0f;
    for (int w = 0; w < kChainThreads / 64; ++w) s += wsum[w];
    if constexpr (COH)
      bstore4(s, make_rsrc(ssp, (uint64_t)N * P * 4u), (uint32_t)((n * P + p) * 4));
    else
      ssp[(size_t)n * P + p] = s;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kChainThreads) void chain_reduce_kernel(float* __restrict__ h,
                                                                     const DevMat* __restrict__ down, int D, int N,
                                                                     float* __restrict__ ssp) {
  __shared__ float wsum[kChainThreads / 64];
  chain_reduce_block<false>(h, down, D, N, blockIdx.y, blockIdx.x, gridDim.x, ssp, wsum);
}

// ---- a whole chain in one launch ------------------------------------------------
// The phases of the multi-launch chain, in the same order and with the same
// arithmetic (so the same bits), with a grid barrier between phases instead
// of a kernel boundary: the sums of squares of h; then per layer the
// gate/up phase (its first weight loads issued before the barrier that
// publishes h), the down phase (likewise for s), and the residual update.
// Shares of the streaming phases are equal splits of each matrix's units.
template <int N>
__global__ __launch_bounds__(kThreads) void chain_kernel(const DevMat* __restrict__ mats, ChainCtl* ctl,
                                                         float* __restrict__ h, float* __restrict__ ssp, int layers,
                                                         int D, const WgRange* __restrict__ ranges_gate_up,
                                                         const WgRange* __restrict__ ranges_down) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ uint32_t s_target;
  __shared__ float wsum[kChainThreads / 64];
  if (threadIdx.x == 0) s_target = 0;  // (only thread 0 reads or writes it)
  const GridSync gs{ctl, &s_target};
  const int P = (D + kChainThreads - 1) / kChainThreads;
  const DevMat none{};
  for (int b = blockIdx.x; b < N * P; b += gridDim.x)
    chain_reduce_block<true>(h, nullptr, D, N, b / P, b % P, P, ssp, wsum);
  grid_arrive(gs);
  for (int l = 0; l < layers; ++l) {
    stream_body<N, kModeTiledGlu, true>(mats + 2 * l, ranges_gate_up, none, lds, &gs);
    grid_arrive(gs);
    stream_body<N, kModeTiledWide, true>(mats + 2 * l + 1, ranges_down, none, lds, &gs);
    grid_arrive(gs);
    grid_wait(gs);
    for (int b = blockIdx.x; b < N * P; b += gridDim.x)
      chain_reduce_block<true>(h, mats + 2 * l + 1, D, N, b / P, b % P, P, ssp, wsum);
    if (l + 1 < layers) grid_arrive(gs);
  }
  grid_finish(gs);
}

hipError_t launch_chain_reduce(float* h, const DevMat* down, int D, int N, float* ssp, hipStream_t stream) {
  const int parts = (D + kChainThreads - 1) / kChainThreads;
  hipLaunchKernelGGL(chain_reduce_kernel, dim3(parts, N), dim3(kChainThreads), 0, stream, h, down, D, N, ssp);
  return hipGetLastError();
}

// ---- split-K reduction -----------------------------------------------------
// One thread per output (n, m) of a split matrix: y = scale * sum over chunks
// of the partial sums, added in chunk order.  Block b handles outputs
// [task.begin, task.begin + task.count) of matrix task.mat (for a single
// matrix, mats == nullptr and the tasks are consecutive 4096-output runs).
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(const DevMat* __restrict__ mats,
                                                                const ReduceTask* __restrict__ tasks, DevMat one,
                                                                int N, const int32_t* __restrict__ n_dev) {
  // device N: the tasks were laid out for 8 columns; those past N * M end here
  if (n_dev) N = device_n(n_dev);
  ReduceTask t;
  if (mats == nullptr) {
    const int64_t total = (int64_t)N * one.M;
    t.mat = 0;
    t.begin = (int64_t)blockIdx.x * kReduceRun;
    t.count = (int32_t)min<int64_t>(kReduceRun, total - t.begin);
  } else {
    t = tasks[blockIdx.x];
  }
  const DevMat mt = mats ? mats[t.mat] : one;
  const int64_t plane = (int64_t)N * mt.M;
  if (n_dev) t.count = (int32_t)max<int64_t>(0, min<int64_t>(t.count, plane - t.begin));
  for (int i = threadIdx.x; i < t.count; i += blockDim.x) {
    const int64_t o = t.begin + i;  // = n * M + m
    const int m = (int)(o % mt.M);
    float acc = 0.0f;
#pragma unroll 8
    for (int c = 0; c < mt.nchunks; ++c) acc += mt.part[c * plane + o];
    // row scales exist only for FP8-row; both NVFP4 layouts use g
    const float scale = (mt.fmt == kFmtFp8Row || mt.fmt == kFmtFp8RowTiled) ? mt.rs[m] : mt.g;
    mt.y[o] = scale * acc;
  }
}

hipError_t launch_reduce(const DevMat* mats, const ReduceTask* tasks, const DevMat& one, int grid, int N,
                         hipStream_t stream, const int32_t* n_dev) {
  hipLaunchKernelGGL(reduce_kernel, dim3(grid), dim3(kReduceThreads), 0, stream, mats, tasks, one, N, n_dev);
  return hipGetLastError();
}

// The dynamic-LDS limit of a kernel is raised once per device (the
// attribute is per device; a bit per device ordinal, set after success).
static hipError_t allow_lds(const void* fn, std::atomic<uint64_t>& done, uint32_t max_bytes = kMaxLdsBytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)max_bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

hipError_t launch_stream_dyn(const DevMat* mats, const WgRange* ranges, const int32_t* n_dev, int grid,
                             size_t lds_bytes, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&stream_kernel_dyn), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stream_kernel_dyn, dim3(grid), dim3(kThreadsTiled), lds_bytes, stream, mats, ranges, n_dev);
  return hipGetLastError();
}

template <int N>
static std::atomic<uint64_t>& chain_lds_set() {
  static std::atomic<uint64_t> done{0};
  return done;
}

template <int N>
static hipError_t launch_chain_n(const DevMat* mats, ChainCtl* ctl, float* h, float* ssp, int layers, int D, int grid,
                                 const WgRange* rgu, const WgRange* rdn, hipStream_t stream) {
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&chain_kernel<N>), chain_lds_set<N>());
  if (e != hipSuccess) return e;
  void* args[] = {&mats, &ctl, &h, &ssp, &layers, &D, &rgu, &rdn};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&chain_kernel<N>), dim3(grid), dim3(kThreads), args,
                                    lds_bytes_for(N) + kArgLdsBytes, stream);
}

template <int N>
static int chain_blocks_n() {
  if (allow_lds(reinterpret_cast<const void*>(&chain_kernel<N>), chain_lds_set<N>()) != hipSuccess) return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(&chain_kernel<N>), kThreads,
                                                   lds_bytes_for(N) + kArgLdsBytes) != hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_chain_persistent(int N, const DevMat* mats, ChainCtl* ctl, float* h, float* ssp, int layers, int D,
                                   int grid, const WgRange* rgu, const WgRange* rdn, hipStream_t stream) {
  switch (N) {
    case 1: return launch_chain_n<1>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 2: return launch_chain_n<2>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 3: return launch_chain_n<3>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 4: return launch_chain_n<4>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 5: return launch_chain_n<5>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 6: return launch_chain_n<6>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 7: return launch_chain_n<7>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    case 8: return launch_chain_n<8>(mats, ctl, h, ssp, layers, D, grid, rgu, rdn, stream);
    default: return hipErrorInvalidValue;
  }
}

int chain_persistent_blocks_per_cu(int N) {
  switch (N) {
    case 1: return chain_blocks_n<1>();
    case 2: return chain_blocks_n<2>();
    case 3: return chain_blocks_n<3>();
    case 4: return chain_blocks_n<4>();
    case 5: return chain_blocks_n<5>();
    case 6: return chain_blocks_n<6>();
    case 7: return chain_blocks_n<7>();
    case 8: return chain_blocks_n<8>();
    default: return 0;
  }
}

// ---- greedy draft acceptance -------------------------------------------------
// keys [groups][8]: each workgroup's best greedy key per column.  Column n's
// target token is the row of the largest key; draft j (j = 1..N-1) is
// accepted while it equals the token of column j - 1.
constexpr int kAcceptThreads = 512;
__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(const uint64_t* __restrict__ keys, int groups, int N,
                                                               const int32_t* __restrict__ drafts,
                                                               int32_t* __restrict__ tokens,
                                                               int32_t* __restrict__ accepted) {
  __shared__ int32_t tok[8];
  const int n = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (n < N) {
    uint64_t b = 0ull;
    for (int g = lane; g < groups; g += 64) {
      const uint64_t o = keys[(size_t)g * 8 + n];
      b = o > b ? o : b;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint64_t o = __shfl_xor(b, off);
      b = o > b ? o : b;
    }
    if (lane == 0) {
      const int32_t t = (int32_t)(0xFFFFFFFFu - (uint32_t)(b & 0xFFFFFFFFull));
      tok[n] = t;
      tokens[n] = t;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int a = 0;
    while (a < N - 1 && drafts[a] == tok[a]) ++a;
    accepted[0] = a;
  }
}

hipError_t launch_accept(const uint64_t* keys, int groups, int N, const int32_t* drafts, int32_t* tokens,
                         int32_t* accepted, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(kAcceptThreads), 0, stream, keys, groups, N, drafts, tokens,
                     accepted);
  return hipGetLastError();
}

// ---- host-side launchers ---------------------------------------------------
template <int N, bool FP8>
static hipError_t launch_split_nf(const DevMat& one, uint32_t* counters, float* parts, int slots_per_wave, int grid,
                                  size_t lds_bytes, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e =
      allow_lds(reinterpret_cast<const void*>(&split_kernel<N, FP8>), lds_set, 160u * 1024u - kSplitStaticLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((split_kernel<N, FP8>), dim3(grid), dim3(kSplitThreads), lds_bytes, stream, one, counters,
                     parts, slots_per_wave);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_split_n(const DevMat& one, uint32_t* counters, float* parts, int slots_per_wave, int grid,
                                 size_t lds_bytes, hipStream_t stream) {
  return one.fmt == kFmtFp8RowTiled
             ? launch_split_nf<N, true>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream)
             : launch_split_nf<N, false>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
}

hipError_t launch_split(int N, const DevMat& one, uint32_t* counters, float* parts, int slots_per_wave, int grid,
                        size_t lds_bytes, hipStream_t stream) {
  switch (N) {
    case 1: return launch_split_n<1>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 2: return launch_split_n<2>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 3: return launch_split_n<3>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 4: return launch_split_n<4>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 5: return launch_split_n<5>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 6: return launch_split_n<6>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 7: return launch_split_n<7>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    case 8: return launch_split_n<8>(one, counters, parts, slots_per_wave, grid, lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int N, int MODE>
static hipError_t launch_nm(const DevMat* mats, const WgRange* ranges, const DevMat& one, int grid,
                            size_t lds_bytes, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_lds(reinterpret_cast<const void*>(&stream_kernel<N, MODE>), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((stream_kernel<N, MODE>), dim3(grid), dim3(threads_for_mode<MODE>()), lds_bytes, stream, mats,
                     ranges, one);
  return hipGetLastError();
}

template <int N>
static hipError_t launch_n(int mode, const DevMat* mats, const WgRange* ranges, const DevMat& one, int grid,
                           size_t lds_bytes, hipStream_t stream) {
  switch (mode) {
    case kModeNvfp4Aligned: return launch_nm<N, kModeNvfp4Aligned>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeNvfp4: return launch_nm<N, kModeNvfp4>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeFp8: return launch_nm<N, kModeFp8>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeMixed: return launch_nm<N, kModeMixed>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeTiled: return launch_nm<N, kModeTiled>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeTiledArgmax: return launch_nm<N, kModeTiledArgmax>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeTiledGlu: return launch_nm<N, kModeTiledGlu>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeTiledWide: return launch_nm<N, kModeTiledWide>(mats, ranges, one, grid, lds_bytes, stream);
    case kModeTiledValu: return launch_nm<N, kModeTiledValu>(mats, ranges, one, grid, lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream(int N, int mode, const DevMat* mats, const WgRange* ranges, const DevMat& one,
                         int grid, size_t lds_bytes, hipStream_t stream) {
  switch (N) {
    case 1: return launch_n<1>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 2: return launch_n<2>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 3: return launch_n<3>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 4: return launch_n<4>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 5: return launch_n<5>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 6: return launch_n<6>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 7: return launch_n<7>(mode, mats, ranges, one, grid, lds_bytes, stream);
    case 8: return launch_n<8>(mode, mats, ranges, one, grid, lds_bytes, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
