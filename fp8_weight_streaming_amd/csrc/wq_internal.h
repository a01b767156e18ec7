// wq_internal.h -- device-side descriptors and launch constants shared by
// the host planner (wq_api.cpp) and the kernels (wq_kernels.hip).
#ifndef WQ_INTERNAL_H
#define WQ_INTERNAL_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wq.h"

namespace wq {

constexpr int kFmtNvfp4 = 0;
constexpr int kFmtFp8Row = 1;
constexpr int kFmtNvfp4Tiled = 2;
constexpr int kFmtFp8RowTiled = 3;

// Tiled NVFP4 storage: blocks of 16 rows x 256 k, each 2048 bytes of codes
// (two 1 KB halves in MFMA lane order) followed by 256 bytes of block
// scales (grouped by the scale parity each lane applies).
constexpr int kTileRows = 16;
constexpr int kTileStepK = 256;
constexpr int kTileCodeBytes = 2048;
constexpr int kTileBlockBytes = 2304;
// Tiled FP8-row storage: blocks of 16 rows x 128 k (2048 bytes, two 1 KB
// halves of 16 row bytes per MFMA lane).
constexpr int kFp8TileStepK = 128;
constexpr int kFp8TileBlockBytes = 2048;

// One persistent workgroup per CU: 16 waves of 64 lanes (8 waves with twice
// the registers each for the tiled-NVFP4 kernel, whose ring spans tiles).
constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kThreadsTiled = 512;
// Segments (64 bytes of one row per lane group of four lanes) in flight.
constexpr int kPrefetch = 8;
// Shallower pipeline for the variants that also carry unaligned-scale or
// mixed-format code, to stay within 128 VGPRs.
constexpr int kPrefetchGeneric = 4;
// Steps (2304-byte blocks) in flight per lane for tiled NVFP4.
constexpr int kPrefetchTiled = 6;
// Largest K chunk whose N <= 8 BF16 columns are staged in LDS at once.  The
// chunking does not depend on N, so column n of a result has the same bits
// for every N > n.
constexpr int kKcMax = 8704;
// LDS: X chunk as (k/8, n) pieces of 16 bytes, then a zero block read by the
// lanes whose A-operand slots are structurally zero.
template <int N>
__host__ __device__ constexpr uint32_t kZeroOffset() { return (uint32_t)kKcMax * 2u * N; }
// The zero block must cover the largest offset an idle lane adds to it:
// tiled NVFP4 reads at up to 256N (second half) + 3*64N (MFMA step) + 16.
template <int N>
__host__ __device__ constexpr uint32_t kZeroBytes() { return 512u * N; }
__host__ __device__ constexpr uint32_t lds_bytes_for(int n) { return (uint32_t)kKcMax * 2u * n + 512u * n; }
// Head acceptance (kModeTiledArgmax) adds, past the zero block, each wave's
// best keys: 8 waves x 8 columns x 8 bytes.
constexpr uint32_t kArgLdsBytes = 512;
// LDS per workgroup on gfx950 (160 KB), less what the kernels declare
// statically (at most 32 bytes): the most dynamic LDS a launch may ask for.
constexpr uint32_t kLdsLimit = 160u * 1024u - 256u;
// A large split matrix of an all-tiled verify pass is processed in blocks of
// tiles: one workgroup computes every K chunk of a block in turn and keeps
// the block's chunk sums in LDS (32 lanes x 4 floats per tile), so no
// partial sums leave the CU and no reduction launch follows.  Its K chunks
// are at most kKcBlocked long, which leaves LDS free between its X chunk and
// the zero block; a block holds as many tiles as that space and the LDS past
// the zero block allow (127 at N = 8).
constexpr int kKcBlocked = 6144;
constexpr uint32_t kPartTileBytes = 512;
constexpr int kPartTilesMax = 256;
// slots past the zero block at n columns
__host__ __device__ constexpr int part_tiles_for(int n) {
  return (int)((kLdsLimit - lds_bytes_for(n)) / kPartTileBytes);
}
template <int N>
__host__ __device__ constexpr uint32_t kPartOffset() { return kZeroOffset<N>() + kZeroBytes<N>(); }
// A block's 512-byte slots at N columns for a blocked matrix with K chunks of
// kc: the first part_a_slots at LDS byte 2 kc N (past its own X chunk, below
// the zero block), the rest past the zero block, within kLdsLimit.
template <int N>
__host__ __device__ constexpr int part_a_slots(int kc) {
  return (int)((2u * (uint32_t)(kKcMax - kc) * (uint32_t)N) / kPartTileBytes);
}
template <int N>
__host__ __device__ constexpr int block_tiles(int kc) {
  return part_a_slots<N>(kc) + part_tiles_for(N) < kPartTilesMax ? part_a_slots<N>(kc) + part_tiles_for(N)
                                                                  : kPartTilesMax;
}
constexpr uint32_t kMaxLdsBytes = kLdsLimit;
static_assert(lds_bytes_for(8) + kArgLdsBytes <= kLdsLimit, "LDS budget exceeded");
static_assert(part_tiles_for(8) >= 32, "too few tiles per block at N = 8");
// idle-lane reads: tiled NVFP4 at 256N + 192N + 16, plain NVFP4 at 192N + 16,
// FP8-row at 16N + 16 bytes past the zero block's start
static_assert(kZeroBytes<1>() >= 448u * 1 + 16u && kZeroBytes<8>() >= 448u * 8 + 16u, "zero block too small");
static_assert(kMaxLdsBytes <= 160u * 1024u, "LDS budget exceeded");

// Device-side descriptor of one matrix (built on the host).
struct DevMat {
  const uint8_t* w;   // NVFP4 codes [M][K/2], FP8 codes [M][K], or tiled NVFP4 / FP8 blocks
  const uint8_t* s;   // NVFP4 block scales [M][K/16] (null for FP8-row)
  const float* rs;    // FP8 row scales [M] (null for NVFP4)
  const uint16_t* x;  // BF16 [N][K]
  float* y;           // FP32 [N][M]
  float* part;        // split-K partial sums [nchunks][N][M] (null if nchunks == 1)
  float g;            // NVFP4 per-tensor scale
  int fmt, M, K;
  int kc;             // K chunk length (multiple of the format's segment)
  int nchunks;
  int ntiles;         // ceil(M / 16)
  int64_t unit0;      // index of this matrix's first unit in the pass
  uint64_t* best;     // head acceptance: greedy keys [workgroup][8] (null otherwise)
  // Gate/up product of a chained MLP layer (kModeTiledGlu) only: rows
  // 16t..16t+7 of a tile are gate rows 8t..8t+7 (tensor scale g), rows
  // 16t+8..16t+15 the up rows of the same f (tensor scale g2).  X is not
  // read from `x`: it is RMSNorm(h) * gamma, rounded to BF16, made while
  // staging from the residual h [N][K], gamma [K] and the sum-of-squares
  // partials ssp [N][nparts] of h.  Outputs: s [N][M/2] (BF16), and the
  // staged X itself, a [N][K] (BF16).
  const float* h;
  const float* ssp;
  const uint16_t* gamma;
  uint16_t* aout;
  uint16_t* sout;
  float g2;
  float eps;
  int nparts;
  // Blocked split (large split matrices of all-tiled verify passes): 1,
  // else 0.  The matrix's units are then tile-major (unit = tile * nchunks +
  // chunk), a workgroup's range holds whole tiles, and the workgroup takes
  // them block_tiles<N>(kc) at a time, every chunk of such a block in turn
  // (a launch of a blocked plan has kLdsLimit bytes of dynamic LDS).
  int tb;
  int pad2;
};

// First unit (and the matrix holding it) of each workgroup's run.
struct WgRange {
  int64_t begin;
  int32_t mat;
  int32_t pad;
};

// The dynamic tail of a verify pass, stored right after the grid + 1
// ranges: units [begin, end) are handed out as `count` claims, in order, to
// whichever workgroup asks next (an atomic counter), so that workgroups
// that streamed their static range faster take more.  `next` starts at 0
// (the plan's upload zeroes it) and only grows: a launch takes every claim
// once and each workgroup one value past the last claim (the one that ends
// its loop), count + grid values in all, so launch L's claims are
// L (count + grid) + i and nothing is reset between launches.  A plan
// without a tail (count 0) takes no claims.  The claims follow (count + 1
// entries, the last one only ending the one before): claim i is units
// [claims[i].begin, claims[i + 1].begin), whose first unit is in matrix
// claims[i].mat.
struct DynSched {
  int64_t begin;
  int64_t end;
  int32_t chunk;  // units per claim outside blocked matrices
  int32_t count;
  uint64_t next;
};
struct DynClaim {
  int64_t begin;
  int32_t mat;
  int32_t pad;
};
// Share of a pass's cost left to the dynamic tail, and its chunk sizes:
// units per workgroup / 32, within [8, 16] (16 for the dense 64-layer
// pass).  A chunk's fixed cost (X restaging, the ring's ramp) wants it
// large, the balance at the end wants it small next to a workgroup's work;
// passes under kDynMinUnitsPerWg units per workgroup have no tail.  (Dense
// 64-layer pass, one box, N = 2 / 4 / 8: a 3% share 1800 / 1858 / 1977 us,
// 5% 1775 / 1839 / 1961, 6% 1776 / 1837 / 1960, 8% 1800 / 1843 / 1973.)
constexpr double kDynShare = 0.05;
constexpr int kDynChunkMin = 8;
constexpr int kDynChunkMax = 16;
constexpr int kDynMinUnitsPerWg = 256;

// One run of outputs of a split matrix for reduce_kernel.
struct ReduceTask {
  int64_t begin;  // first output index (n * M + m)
  int32_t mat;
  int32_t count;  // outputs in the run (<= kReduceRun)
};
constexpr int kReduceThreads = 256;
// One output per thread: a split product can have few outputs (40,960 for
// 5120 rows at N = 8), and the sum over chunks is one round of loads.
constexpr int kReduceRun = kReduceThreads;

// Kernel variants: which unit bodies a launch contains.
constexpr int kModeNvfp4Aligned = 0;  // NVFP4 only, K % 64 == 0 for every matrix
constexpr int kModeNvfp4 = 1;         // NVFP4 only, any K % 32 == 0
constexpr int kModeFp8 = 2;           // FP8-row only
constexpr int kModeMixed = 3;         // any formats
constexpr int kModeTiled = 4;         // tiled NVFP4 and tiled FP8-row only
constexpr int kModeTiledArgmax = 5;   // one tiled matrix, greedy keys per workgroup (head acceptance)
// Chained MLP layers: few tiles per workgroup, so 16 waves (with a shallower
// ring, to fit their registers) let every tile of a workgroup stream at once.
constexpr int kModeTiledGlu = 6;      // tiled NVFP4 gate/up with RMSNorm staging and SwiGLU outputs
constexpr int kModeTiledWide = 7;     // tiled NVFP4 / FP8 at 16 waves, static ranges only
constexpr int kModeTiledValu = 8;     // kModeTiled with the NVFP4 steps on the vector ALUs (the MFMA comparison)
constexpr int kPrefetchWide = 3;

template <int MODE>
__host__ __device__ constexpr int threads_for_mode() {
  return (MODE == kModeTiled || MODE == kModeTiledArgmax || MODE == kModeTiledValu) ? kThreadsTiled : kThreads;
}
constexpr int waves_for_mode(int mode) {
  return ((mode == kModeTiled || mode == kModeTiledArgmax || mode == kModeTiledValu) ? kThreadsTiled : kThreads) / 64;
}

// Chained-layer residual update: one workgroup of kChainThreads per
// kChainThreads outputs of one column; also each block's sum of squares.
constexpr int kChainThreads = 256;

// Grid barrier of the single-launch chain (in the workspace, zero before
// the first launch): arrivals so far in this launch (barrier b is open once
// count reaches b times the grid), workgroups finished (the last one sets
// both back to zero), and a sticky flag set if a wait gave up (see
// kSpinLimit).
struct ChainCtl {
  uint32_t count;
  uint32_t done;
  uint32_t error;
  uint32_t pad;
};

hipError_t launch_stream(int N, int mode, const DevMat* mats, const WgRange* ranges, const DevMat& one,
                         int grid, size_t lds_bytes, hipStream_t stream);
// Single tiled products with few tiles per CU (split_kernel): the first
// kSplitCounterBytes of a single product's workspace hold one arrival counter
// per tile (zero between calls: each call leaves them zero, so the workspace
// must be zero before its first use); every single product's other scratch
// (tile-chunk parts, chunk partial sums) lies past them.
constexpr size_t kSplitCounterBytes = 16384;
constexpr int kSplitMaxTiles = (int)(kSplitCounterBytes / 4);
// A tile-chunk part: 16 rows x N <= 8 columns of FP32.
constexpr size_t kSplitPartBytes = 512;
// Tiles per CU below which a single tiled product splits tiles across waves
// and workgroups (above it, whole tiles per workgroup balance within 1/8).
constexpr int kSplitTilesPerCu = 8;
// Tile-chunk parts one workgroup may write (its LDS list of arrivals), and
// K chunks at most (the parts a finishing workgroup adds).
constexpr int kSplitArrivalsMax = 64;
constexpr int kSplitChunksMax = 24;
// Threads per workgroup of the split kernel, and steps in flight per lane.
constexpr int kSplitThreads = 512;
constexpr int kSplitPrefetch = 3;
// Most output pairs a wave holds in LDS until the end of a short run.
constexpr int kHoldMax = 8;
// Tiled-stream outputs held until the chip-wide 100 MHz clock enters a new
// window of 2^kDeferWindowBits ticks (10.24 us), from kDeferMinN columns up.
// Measured over the dense 64-layer pass (us per pass at N = 2 / 4 / 8):
// written at once 1783 / 1870 / 2030; windows of 5.12 us 1793 / 1860 /
// 1923, 10.24 us 1793 / 1840 / 1899, 20.48 us 1794 / 1855 / 1939.
constexpr int kDeferWindowBits = 10;
constexpr int kDeferMinN = 4;
// LDS the split kernel declares statically (its arrival lists), kept free
// of its dynamic LDS.
constexpr uint32_t kSplitStaticLds = 1024;
hipError_t launch_split(int N, const DevMat& one, uint32_t* counters, float* parts, int slots_per_wave, int grid,
                        size_t lds_bytes, hipStream_t stream);
hipError_t launch_reduce(const DevMat* mats, const ReduceTask* tasks, const DevMat& one, int grid, int N,
                         hipStream_t stream, const int32_t* n_dev = nullptr);
// the tiled verify pass with N read from n_dev (a plan prepared for N = 8)
hipError_t launch_stream_dyn(const DevMat* mats, const WgRange* ranges, const int32_t* n_dev, int grid,
                             size_t lds_bytes, hipStream_t stream);
// h[n][m] += the down product of `down` (a device-side descriptor: its
// chunk partial sums in chunk order, times g; or its y for one chunk),
// then ssp[n][p] = sum of h[n][m]^2 over block p's outputs.  down == null:
// ssp only.
hipError_t launch_chain_reduce(float* h, const DevMat* down, int D, int N, float* ssp, hipStream_t stream);
// All layers of a chain in one cooperative launch of `grid` workgroups.
// ranges_gate_up / ranges_down: the workgroups' unit ranges of the two
// streaming phases (built for `grid` workgroups), or null for equal splits.
hipError_t launch_chain_persistent(int N, const DevMat* mats, ChainCtl* ctl, float* h, float* ssp, int layers, int D,
                                   int grid, const WgRange* ranges_gate_up, const WgRange* ranges_down,
                                   hipStream_t stream);
// Workgroups of the single-launch chain that fit on the device at once.
int chain_persistent_blocks_per_cu(int N);
// Host-side argument checks of the single-matrix products (no HIP call).
wq_status check_gemm_args(int fmt, const void* w, const void* s, const void* x, const void* y, int M, int K, int N);
hipError_t launch_accept(const uint64_t* keys, int groups, int N, const int32_t* drafts, int32_t* tokens,
                         int32_t* accepted, hipStream_t stream);

}  // namespace wq

#endif
