// wq_api.cpp -- host side of libwq: argument validation, K-split planning,
// workspace layout and the launches behind the C ABI in include/wq.h.
//
// Validation never touches the HIP runtime, so every argument error is
// reported without a device (and with nothing enqueued).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "wq.h"
#include "wq_internal.h"

namespace wq {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---- device facts, cached per device ---------------------------------------
struct DeviceInfo {
  bool probed = false;
  bool ok = false;
  int cus = 0;
};
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Returns the CU count of the current device, or 0 if there is no usable
// gfx950 device.
int current_cus() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.probed) {
    d.probed = true;
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0 &&
        p.multiProcessorCount > 0) {
      d.ok = true;
      d.cus = p.multiProcessorCount;
    }
  }
  return d.ok ? d.cus : 0;
}

// ---- K-split plan ------------------------------------------------------------
struct Split {
  int kc = 0;
  int nchunks = 0;
  int ntiles = 0;
  int tb = 0;  // 1 for a blocked split (all-tiled verify passes), else 0
};

int seg_k(int fmt) {
  return fmt == kFmtNvfp4Tiled ? kTileStepK : fmt == kFmtFp8RowTiled ? kFp8TileStepK : fmt == kFmtNvfp4 ? 128 : 64;
}
bool is_nvfp4(int fmt) { return fmt == kFmtNvfp4 || fmt == kFmtNvfp4Tiled; }
bool is_fp8(int fmt) { return fmt == kFmtFp8Row || fmt == kFmtFp8RowTiled; }
bool is_tiled(int fmt) { return fmt == kFmtNvfp4Tiled || fmt == kFmtFp8RowTiled; }

Split make_split(int fmt, int M, int K, int kc) {
  Split s;
  s.kc = kc;
  s.nchunks = (int)ceil_div(K, kc);
  s.ntiles = (int)ceil_div(M, 16);
  return s;
}

// In a verify pass many matrices share the machine, so K is split only as
// far as the LDS budget requires.
Split verify_split(int fmt, int M, int K) {
  const int sk = seg_k(fmt);
  const int n = (int)ceil_div(K, kKcMax);
  const int kc = (int)(ceil_div(ceil_div(K, n), sk) * sk);
  return make_split(fmt, M, K, kc);
}

// A split matrix computed in blocks inside a verify pass: chunks of at most
// kKcBlocked k, so that the space between its X chunk and the zero block
// holds chunk-sum slots at every N (the chunking does not depend on N).
Split blocked_split(int fmt, int M, int K) {
  const int sk = seg_k(fmt);
  const int n = (int)std::max(ceil_div(K, kKcMax), ceil_div(K, kKcBlocked));
  const int kc = (int)(ceil_div(ceil_div(K, n), sk) * sk);
  return make_split(fmt, M, K, kc);
}

// A single product may split K further so that every wave of every CU has
// a unit of work.  Candidate splits are scored by the work of the busiest
// wave: rounds of units times (segments per unit + a ramp of kPrefetch
// segments), plus, for any split, the reduce launch (about 4 us on MI355X,
// taken as 6 tiled steps or 12 segments of the other formats); a split must
// save at least 10% over the next-coarser best to be taken, since it also
// costs partial-sum traffic.
Split gemm_split(int fmt, int M, int K, int cus) {
  const int sk = seg_k(fmt);
  const int64_t slots = (int64_t)cus * waves_for_mode(is_tiled(fmt) ? kModeTiled : kModeNvfp4);
  const int64_t ntiles = ceil_div(M, 16);
  const int nmin = (int)ceil_div(K, kKcMax);
  const int nmax = std::max(nmin, (int)std::min<int64_t>(64, ceil_div(K, sk)));
  Split best = verify_split(fmt, M, K);
  double best_cost = 1e300;
  for (int n = nmin; n <= nmax; ++n) {
    const int kc = (int)(ceil_div(ceil_div(K, n), sk) * sk);
    const int nc = (int)ceil_div(K, kc);
    if (nc != n && n != nmin) continue;  // this n rounds to a split already scored
    const int64_t units = ntiles * nc;
    const int64_t rounds = ceil_div(units, slots);
    const double reduce_cost = nc > 1 ? (is_tiled(fmt) ? 6.0 : 12.0) : 0.0;
    const double cost = (double)rounds * ((double)(kc / sk) + kPrefetch) + reduce_cost;
    if (cost < 0.9 * best_cost) {
      best_cost = cost;
      best = make_split(fmt, M, K, kc);
    }
  }
  return best;
}

// A single tiled product with fewer than kSplitTilesPerCu tiles per CU is
// computed by split_kernel: K is cut into C chunks of s steps (the last one
// shorter); the workgroups are shared out among the chunks, each taking an
// equal share of its chunk's tiles, and each workgroup's steps are cut into
// one equal piece per wave; with C > 1, every tile's C parts are added in
// chunk order by the workgroup whose part arrives last.  s is chosen by the
// bytes the busiest CU moves at N = 8 (the most X): the weights of its run,
// its X chunk (mostly served by the L2: counted at half weight) and, for
// C > 1, the parts written and read (512 bytes each way) plus the arrival
// round trips at the end (taken as 128 KB of streaming, and 8 KB more per
// chunk).  Fitted to sweeps of s on MI355X: 5120 x 17408 at N = 8 took
// 17.96 / 16.96 / 16.72 / 17.28 / 18.56 us with 8 / 6 / 4 / 3 / 2 chunks,
// 17408 x 5120 at N = 1 14.0 / 17.8 / 18.0 us with 1 / 2 / 3.
// Nothing depends on N, so neither do the results' bits.
struct TileSplit {
  bool ok = false;
  Split chunks;
  int grid = 0;
  int slots = 0;  // LDS slots per wave: the most tiles one wave's piece touches
};

TileSplit tile_split_plan(int fmt, int M, int K, int cus) {
  TileSplit p;
  if (!is_tiled(fmt) || cus <= 0) return p;
  const int sk = seg_k(fmt);
  const int64_t T = ceil_div(M, kTileRows);
  if (T >= (int64_t)kSplitTilesPerCu * cus || T > kSplitMaxTiles) return p;
  const int64_t S = ceil_div(K, sk);
  if (T * S >= (1ll << 31)) return p;
  const double step_bytes = is_nvfp4(fmt) ? (double)kTileBlockBytes : (double)kFp8TileBlockBytes;
  const int W = kSplitThreads / 64;
  double best = 1e300;
  for (int64_t s = 1; s <= std::min<int64_t>(S, kKcMax / sk); ++s) {
    const int64_t C = ceil_div(S, s);
    if (C > kSplitChunksMax || ceil_div(S, C) != s) continue;  // the balanced chunking of C only
    const int64_t sl = S - (C - 1) * s;
    const int64_t G = std::min<int64_t>(cus, T * C);
    if (G < C) continue;
    const int64_t tiles_max = ceil_div(T, G / C);  // a chunk gets at least G / C workgroups
    const int64_t run_max = tiles_max * s;
    const double tail = C > 1 ? (double)(T * C) * 1024.0 / (double)G + 131072.0 + 8192.0 * (double)C : 0.0;
    const int64_t smin = std::min(s, sl);
    const int64_t slots = ceil_div(ceil_div(run_max, W), smin) + 1;
    if (tiles_max > kSplitArrivalsMax) continue;
    if (lds_bytes_for(8) + (uint64_t)W * slots * kSplitPartBytes + kSplitStaticLds > 160u * 1024u) continue;
    const double cost = (double)run_max * step_bytes + 8.0 * (double)(s * sk) + tail;
    if (cost < best) {
      best = cost;
      p.ok = true;
      p.chunks = make_split(fmt, M, K, (int)(s * sk));
      p.grid = (int)G;
      p.slots = (int)slots;
    }
  }
  return p;
}

size_t tile_split_bytes(const TileSplit& p) {
  return kSplitCounterBytes + align_up((size_t)p.chunks.nchunks * p.chunks.ntiles * kSplitPartBytes, kAlign);
}

// ---- validation ------------------------------------------------------------------
wq_status check_shape(int fmt, int M, int K, int N) {
  if (fmt != kFmtNvfp4 && fmt != kFmtFp8Row && fmt != kFmtNvfp4Tiled && fmt != kFmtFp8RowTiled)
    return WQ_ERROR_INVALID_VALUE;
  if (N < 1 || N > 8 || M < 1 || K < 1) return WQ_ERROR_INVALID_VALUE;
  const int mult = is_nvfp4(fmt) ? 32 : 16;
  if (K % mult != 0 || K > (1 << 24)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  const uint64_t wbytes = is_nvfp4(fmt) ? (uint64_t)M * (uint64_t)(K / 2) : (uint64_t)M * (uint64_t)K;
  if (wbytes >= (1ull << 40)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  // outputs are addressed with 32-bit buffer offsets below 2 GiB
  if ((uint64_t)N * (uint64_t)M * 4u >= (1ull << 31)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  // a tiled matrix is addressed with 32-bit buffer offsets
  if (fmt == kFmtNvfp4Tiled &&
      (uint64_t)((M + kTileRows - 1) / kTileRows) * ((K + kTileStepK - 1) / kTileStepK) * kTileBlockBytes >= (1ull << 32))
    return WQ_ERROR_UNSUPPORTED_SHAPE;
  if (fmt == kFmtFp8RowTiled &&
      (uint64_t)((M + kTileRows - 1) / kTileRows) * ((K + kFp8TileStepK - 1) / kFp8TileStepK) * kFp8TileBlockBytes >=
          (1ull << 32))
    return WQ_ERROR_UNSUPPORTED_SHAPE;
  return WQ_SUCCESS;
}

// Tiled NVFP4 carries its scales inside `w`; `s` is not used for it.
wq_status check_ptrs(int fmt, const void* w, const void* s, const void* x, const void* y) {
  if (fmt == kFmtNvfp4Tiled) s = w;
  if (!w || !s || !x || !y) return WQ_ERROR_INVALID_VALUE;
  if (!aligned16(w) || !aligned16(s) || !aligned16(x) || !aligned16(y)) return WQ_ERROR_MISALIGNED;
  return WQ_SUCCESS;
}

// Workspace bytes of the split-K scratch (chunk partial sums) of one matrix.
size_t split_scratch_bytes(const Split& s, int M, int N) {
  if (s.nchunks <= 1 || s.tb > 0) return 0;
  return align_up((size_t)s.nchunks * N * M * sizeof(float), kAlign);
}

// Workspace of a single product: the split-kernel counters come first in
// every single product's workspace (they must stay zero between calls, and
// no other single product writes there), then its own scratch.
size_t gemm_workspace(int fmt, int M, int K, int N, int cus) {
  const TileSplit ts = tile_split_plan(fmt, M, K, cus);
  if (ts.ok) return tile_split_bytes(ts);
  const size_t part = split_scratch_bytes(gemm_split(fmt, M, K, cus), M, N);
  return part ? kSplitCounterBytes + part : 0;
}

DevMat dev_mat(int fmt, const void* w, const void* s, float g, const uint16_t* x, float* y, int M, int K,
               const Split& sp, char* scratch, int N, int64_t unit0) {
  DevMat d{};
  d.w = static_cast<const uint8_t*>(w);
  d.s = fmt == kFmtNvfp4 ? static_cast<const uint8_t*>(s) : nullptr;  // tiled NVFP4: inside w
  d.rs = is_fp8(fmt) ? static_cast<const float*>(s) : nullptr;
  d.x = x;
  d.y = y;
  d.g = g;
  d.fmt = fmt;
  d.M = M;
  d.K = K;
  d.kc = sp.kc;
  d.nchunks = sp.nchunks;
  d.ntiles = sp.ntiles;
  d.unit0 = unit0;
  d.tb = sp.tb;
  if (sp.nchunks > 1 && sp.tb == 0) d.part = reinterpret_cast<float*>(scratch);
  return d;
}

wq_status gemm(int fmt, const void* w, const void* s, float g, const uint16_t* x, float* y, int M, int K,
               int N, void* ws, size_t ws_bytes, void* stream) {
  wq_status st = check_gemm_args(fmt, w, s, x, y, M, K, N);
  if (st != WQ_SUCCESS) return st;
  if (ws && !aligned16(ws)) return WQ_ERROR_MISALIGNED;
  const int cus = current_cus();
  if (cus <= 0) return WQ_ERROR_DEVICE;
  const TileSplit ts = tile_split_plan(fmt, M, K, cus);
  if (ts.ok) {
    if (!ws || ws_bytes < tile_split_bytes(ts)) return WQ_ERROR_WORKSPACE;
    const DevMat one = dev_mat(fmt, w, s, g, x, y, M, K, ts.chunks, nullptr, N, 0);
    const hipError_t e = launch_split(
        N, one, static_cast<uint32_t*>(ws), reinterpret_cast<float*>(static_cast<char*>(ws) + kSplitCounterBytes),
        ts.slots, ts.grid, lds_bytes_for(N) + (size_t)(kSplitThreads / 64) * ts.slots * kSplitPartBytes,
        static_cast<hipStream_t>(stream));
    return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
  }
  const Split sp = gemm_split(fmt, M, K, cus);
  const size_t need = split_scratch_bytes(sp, M, N);
  if (need > 0 && (!ws || ws_bytes < kSplitCounterBytes + need)) return WQ_ERROR_WORKSPACE;
  const DevMat one =
      dev_mat(fmt, w, s, g, x, y, M, K, sp, need ? static_cast<char*>(ws) + kSplitCounterBytes : nullptr, N, 0);
  const int64_t units = (int64_t)sp.nchunks * sp.ntiles;
  const int grid = (int)std::min<int64_t>(cus, units);
  const int mode = fmt == kFmtFp8Row ? kModeFp8
                   : is_tiled(fmt) ? kModeTiled
                   : (K % 64 == 0 ? kModeNvfp4Aligned : kModeNvfp4);
  hipError_t e = launch_stream(N, mode, nullptr, nullptr, one, grid, lds_bytes_for(N),
                               static_cast<hipStream_t>(stream));
  if (e == hipSuccess && sp.nchunks > 1)
    e = launch_reduce(nullptr, nullptr, one, (int)ceil_div((int64_t)N * M, kReduceRun), N,
                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

// ---- verify pass layout ------------------------------------------------------
// The pass's matrices in the order of the unit list (and of the device
// table): large split matrices computed in blocks first, then the rest, each
// in the caller's order.  Every per-matrix array below is in this order.
struct PassLayout {
  std::vector<wq_matrix> descs;
  std::vector<Split> splits;
  std::vector<size_t> scratch_off;
  std::vector<ReduceTask> tasks;  // reduction runs of the split matrices
  size_t table_bytes = 0, ranges_bytes = 0, tasks_bytes = 0, scratch_bytes = 0, total = 0;
  int grid = 0;
  int64_t units = 0;
  int64_t dyn_chunks = 0;  // upper bound on the tail's claim entries, for sizing
  uint32_t lds_extra = 0;  // LDS for blocked chunk sums
};

wq_status check_descs(const wq_matrix* descs, int count, int N) {
  if (!descs || count < 1 || N < 1 || N > 8) return WQ_ERROR_INVALID_VALUE;
  for (int i = 0; i < count; ++i) {
    const wq_matrix& d = descs[i];
    wq_status st = check_shape(d.fmt, d.M, d.K, N);
    if (st != WQ_SUCCESS) return st;
    st = check_ptrs(d.fmt, d.w, d.scales, d.x, d.y);
    if (st != WQ_SUCCESS) return st;
  }
  return WQ_SUCCESS;
}

bool all_tiled(const wq_matrix* descs, int count) {
  for (int i = 0; i < count; ++i)
    if (!is_tiled(descs[i].fmt)) return false;
  return true;
}

// Balancing cost of one unit (16 rows of K chunk c): its weight bytes plus a
// fixed per-unit overhead.
double unit_cost(const wq_matrix& d, const Split& sp, int c) {
  const int klen = std::min(sp.kc, d.K - c * sp.kc);
  const double bytes_per_k = is_nvfp4(d.fmt) ? 16.0 * 0.5625 : 16.0;
  return bytes_per_k * klen + 4096.0;
}
double tile_cost(const wq_matrix& d, const Split& sp) {
  double t = 0.0;
  for (int c = 0; c < sp.nchunks; ++c) t += unit_cost(d, sp, c);
  return t;
}

// A split matrix of an all-tiled pass is blocked when an average
// workgroup's share of the pass holds at least this many of its tiles:
// each block costs a restaging of X per chunk, which smaller shares (a
// single decode layer, say) do not amortize; they keep the reduction.
constexpr double kBlockMinTiles = 32.0;

PassLayout pass_layout(const wq_matrix* in, int count, int N, int cus) {
  PassLayout L;
  std::vector<Split> sp(count);
  double total = 0.0;
  for (int i = 0; i < count; ++i) {
    sp[i] = verify_split(in[i].fmt, in[i].M, in[i].K);
    total += tile_cost(in[i], sp[i]) * sp[i].ntiles;
    L.units += (int64_t)sp[i].nchunks * sp[i].ntiles;
  }
  L.grid = (int)std::min<int64_t>(cus, L.units);
  const double share = total / L.grid;
  const bool tiled = all_tiled(in, count);
  std::vector<char> blk(count, 0);
  for (int i = 0; i < count; ++i) {
    if (!tiled || sp[i].nchunks <= 1) continue;
    const Split b = blocked_split(in[i].fmt, in[i].M, in[i].K);
    if (share >= kBlockMinTiles * tile_cost(in[i], b)) {
      blk[i] = 1;
      // its units follow its own (finer) chunking
      L.units += (int64_t)b.nchunks * b.ntiles - (int64_t)sp[i].nchunks * sp[i].ntiles;
      sp[i] = b;
    }
  }
  L.grid = (int)std::min<int64_t>(cus, L.units);
  int64_t blocked_tiles = 0;
  for (int pass = 0; pass < 2; ++pass)
    for (int i = 0; i < count; ++i) {
      if (blk[i] != (pass == 0)) continue;
      L.descs.push_back(in[i]);
      L.splits.push_back(sp[i]);
      if (blk[i]) {
        // the kernel places the block's slots (part_a_slots, block_tiles) in
        // all the LDS a workgroup may have
        L.splits.back().tb = 1;
        L.lds_extra = kLdsLimit - lds_bytes_for(N);
        blocked_tiles += sp[i].ntiles;
      }
    }
  L.scratch_off.resize(count);
  for (int i = 0; i < count; ++i) {
    if (L.splits[i].nchunks <= 1 || L.splits[i].tb > 0) continue;
    const int64_t outs = (int64_t)N * L.descs[i].M;
    for (int64_t b = 0; b < outs; b += kReduceRun)
      L.tasks.push_back(ReduceTask{b, i, (int32_t)std::min<int64_t>(kReduceRun, outs - b)});
  }
  L.table_bytes = align_up((size_t)count * sizeof(DevMat), kAlign);
  // claims: at most one per kDynChunkMin units, or per tile of a blocked
  // matrix, plus one per matrix (a claim may end at a blocked matrix's end),
  // plus the end entry
  L.dyn_chunks = ceil_div(L.units, kDynChunkMin) + blocked_tiles + count + 1;
  L.ranges_bytes = align_up((size_t)(L.grid + 1) * sizeof(WgRange) + sizeof(DynSched) +
                                (size_t)L.dyn_chunks * sizeof(DynClaim),
                            kAlign);
  L.tasks_bytes = align_up(L.tasks.size() * sizeof(ReduceTask), kAlign);
  size_t off = 0;
  for (int i = 0; i < count; ++i) {
    L.scratch_off[i] = off;
    off += split_scratch_bytes(L.splits[i], L.descs[i].M, N);
  }
  L.scratch_bytes = off;
  L.total = L.table_bytes + L.ranges_bytes + L.tasks_bytes + L.scratch_bytes;
  return L;
}

// Units per chunk of a pass's dynamic tail.
int dyn_chunk_units(int64_t units, int grid) {
  return (int)std::max<int64_t>(kDynChunkMin, std::min<int64_t>(kDynChunkMax, units / ((int64_t)grid * 32)));
}

// Splits the first (1 - kDynShare) of the pass's cost into grid runs of
// (nearly) equal cost, where a unit's cost is the weight bytes of its 16
// rows in its K chunk plus a fixed per-unit overhead; the rest of the unit
// list is the dynamic tail (*dyn_begin onwards).  Units of one (matrix,
// chunk) cost the same, so each boundary inside such a group is found by
// division.  Only all-tiled passes of at least kDynMinUnitsPerWg units per
// workgroup have a tail (smaller passes, and the plain-layout kernels, which
// ramp up per unit, measured slower with one).
std::vector<WgRange> balance(const wq_matrix* descs, int count, const PassLayout& L, bool tiled_only,
                             int64_t* dyn_begin) {
  auto unit_cost = [&](int i, int c) { return wq::unit_cost(descs[i], L.splits[i], c); };
  double total = 0.0;
  for (int i = 0; i < count; ++i)
    for (int c = 0; c < L.splits[i].nchunks; ++c) total += unit_cost(i, c) * L.splits[i].ntiles;
  const bool tail = tiled_only && L.units >= (int64_t)L.grid * kDynMinUnitsPerWg;
  const double stat = tail ? total * (1.0 - kDynShare) : total;
  std::vector<WgRange> ranges(L.grid + 1, WgRange{0, 0, 0});
  int w = 1;
  double acc = 0.0;
  int64_t u = 0;
  const int last = tail ? L.grid : L.grid - 1;  // with a tail, range grid's end is a boundary too
  for (int i = 0; i < count; ++i) {
    const Split& sp = L.splits[i];
    if (sp.tb > 0) {
      // blocked split: units are tile-major and a range holds whole tiles
      // (every chunk of a tile runs in one workgroup)
      double tile_cost = 0.0;
      for (int c = 0; c < sp.nchunks; ++c) tile_cost += unit_cost(i, c);
      const double end = acc + tile_cost * sp.ntiles;
      while (w <= last && stat * w / L.grid < end) {
        const double need = (stat * w / L.grid - acc) / tile_cost;
        int64_t j = need <= 0.0 ? 0 : (int64_t)std::ceil(need);
        if (j > sp.ntiles) j = sp.ntiles;
        ranges[w] = WgRange{u + j * sp.nchunks, i, 0};
        ++w;
      }
      acc = end;
      u += (int64_t)sp.nchunks * sp.ntiles;
      continue;
    }
    for (int c = 0; c < sp.nchunks; ++c) {
      const double uc = unit_cost(i, c);
      const double end = acc + uc * sp.ntiles;
      while (w <= last && stat * w / L.grid < end) {
        const double need = (stat * w / L.grid - acc) / uc;
        int64_t j = need <= 0.0 ? 0 : (int64_t)std::ceil(need);
        if (j > sp.ntiles) j = sp.ntiles;
        ranges[w] = WgRange{u + j, i, 0};
        ++w;
      }
      acc = end;
      u += sp.ntiles;
    }
  }
  for (; w <= L.grid; ++w) ranges[w] = WgRange{L.units, count - 1, 0};
  ranges[0] = WgRange{0, 0, 0};
  *dyn_begin = ranges[L.grid].begin;
  return ranges;
}

// The dynamic tail [dyn_begin, units) as claims, each followed by the next
// one's begin (the last entry only ends the tail): `chunk` units; a claim
// starting in a blocked matrix (tile-major units) takes chunk / nchunks
// whole tiles of it (at least one).  Blocked matrices lead the unit list,
// so a claim starting elsewhere never reaches one.
std::vector<DynClaim> tail_claims(const std::vector<DevMat>& mats, const PassLayout& L, int64_t dyn_begin,
                                  int chunk) {
  const int count = (int)mats.size();
  auto units_of = [&](int j) { return (int64_t)L.splits[j].nchunks * L.splits[j].ntiles; };
  auto tile_end = [&](int j, int64_t v) {  // first tile boundary of matrix j at or after unit v
    const int64_t nc = L.splits[j].nchunks;
    return mats[j].unit0 + std::min(ceil_div(v - mats[j].unit0, nc) * nc, units_of(j));
  };
  std::vector<DynClaim> claims;
  int i = 0;
  for (int64_t u = dyn_begin; u < L.units;) {
    while (i + 1 < count && mats[i + 1].unit0 <= u) ++i;
    int64_t e;
    if (L.splits[i].tb > 0) {
      const int64_t tiles = std::max<int64_t>(1, chunk / L.splits[i].nchunks);
      e = tile_end(i, u + tiles * L.splits[i].nchunks);
    } else {
      e = std::min<int64_t>(u + chunk, L.units);
    }
    claims.push_back(DynClaim{u, i, 0});
    u = e;
  }
  claims.push_back(DynClaim{L.units, count - 1, 0});
  return claims;
}

// Every static range and every claim starts at a tile boundary of any
// blocked matrix it starts in (what the kernel relies on).
bool blocks_whole(const std::vector<DevMat>& mats, const PassLayout& L, const std::vector<WgRange>& ranges,
                  const std::vector<DynClaim>& claims) {
  // v is in matrix j, or is the first unit after it
  auto whole = [&](int64_t v, int j) {
    if (j < 0 || j >= (int)mats.size()) return false;
    const int64_t local = v - mats[j].unit0;
    const int64_t units = (int64_t)L.splits[j].nchunks * L.splits[j].ntiles;
    if (local < 0 || local > units) return false;
    if (L.splits[j].tb == 0 || local == units) return true;
    return local % L.splits[j].nchunks == 0;
  };
  for (size_t w = 0; w + 1 < ranges.size(); ++w)
    if (!whole(ranges[w].begin, ranges[w].mat)) return false;
  for (const DynClaim& c : claims)
    if (!whole(c.begin, c.mat)) return false;
  return true;
}

// ---- chained MLP layers --------------------------------------------------------
// K split of a chain's down product (M = D rows, K = F), launched alone at 16
// waves per workgroup, whose waves stream all of the workgroup's units at
// once.  Candidates are scored by the busiest workgroup's units times steps
// per unit (fewer than 8 units leave the CU's memory pipeline part idle, so
// count as 8), plus half a step per chunk for the partial sums and their
// reduction.
Split chain_down_split(int D, int F, int cus) {
  const int sk = kTileStepK;
  const int64_t ntiles = ceil_div(D, kTileRows);
  const int nmin = (int)ceil_div(F, kKcMax);
  const int nmax = std::max(nmin, (int)std::min<int64_t>(32, ceil_div(F, sk)));
  Split best = verify_split(kFmtNvfp4Tiled, D, F);
  double best_cost = 1e300;
  for (int n = nmin; n <= nmax; ++n) {
    const int kc = (int)(ceil_div(ceil_div(F, n), sk) * sk);
    if ((int)ceil_div(F, kc) != n) continue;  // same split as a smaller n
    const int64_t units = ntiles * n;
    const int64_t grid = std::min<int64_t>(cus, units);
    // per workgroup, with the chunk-aligned runs of chunk_ranges
    const int64_t per = grid >= n ? ceil_div(ntiles, grid / n) : ceil_div(units, grid);
    const double cost = (double)std::max<int64_t>(per, 8) * (kc / sk) + 0.5 * n;
    if (cost < best_cost) {
      best_cost = cost;
      best = make_split(kFmtNvfp4Tiled, D, F, kc);
    }
  }
  return best;
}

struct ChainLayout {
  Split gate_up, down;
  int grid_gate_up = 0, grid_down = 0, parts = 0;
  size_t table_bytes = 0, ranges_gu_bytes = 0, ranges_down_bytes = 0, ctl_bytes = 0, part_bytes = 0, ssp_bytes = 0,
         total = 0;
};

wq_status check_chain_shape(int layers, int D, int F, int N) {
  if (layers < 1 || layers > (1 << 20) || N < 1 || N > 8 || D < 1 || F < 1) return WQ_ERROR_INVALID_VALUE;
  if (D % 32 != 0 || F % 32 != 0 || D > kKcMax || F > (1 << 24)) return WQ_ERROR_UNSUPPORTED_SHAPE;
  wq_status st = check_shape(kFmtNvfp4Tiled, 2 * F, D, N);
  if (st != WQ_SUCCESS) return st;
  return check_shape(kFmtNvfp4Tiled, D, F, N);
}

ChainLayout chain_layout(int layers, int D, int F, int N, int cus) {
  ChainLayout L;
  L.gate_up = verify_split(kFmtNvfp4Tiled, 2 * F, D);  // one chunk: D <= kKcMax
  L.down = chain_down_split(D, F, cus);
  L.grid_gate_up = (int)std::min<int64_t>(cus, L.gate_up.ntiles);
  L.grid_down = (int)std::min<int64_t>(cus, (int64_t)L.down.ntiles * L.down.nchunks);
  L.parts = (int)ceil_div(D, kChainThreads);
  L.table_bytes = align_up((size_t)2 * layers * sizeof(DevMat), kAlign);
  L.ranges_gu_bytes = align_up((size_t)(L.grid_gate_up + 1) * sizeof(WgRange), kAlign);
  L.ranges_down_bytes = align_up((size_t)(L.grid_down + 1) * sizeof(WgRange), kAlign);
  L.ctl_bytes = align_up(sizeof(ChainCtl), kAlign);
  L.part_bytes = align_up((size_t)L.down.nchunks * N * D * sizeof(float), kAlign);
  L.ssp_bytes = align_up((size_t)N * L.parts * sizeof(float), kAlign);
  L.total = L.table_bytes + L.ranges_gu_bytes + L.ranges_down_bytes + L.ctl_bytes + L.part_bytes + L.ssp_bytes;
  return L;
}

// grid runs of (nearly) equal unit counts over one matrix
void equal_ranges(int64_t units, int grid, WgRange* out) {
  for (int w = 0; w <= grid; ++w) out[w] = WgRange{units * w / grid, 0, 0};
}

// Runs that never cross a K chunk (each crossing costs a workgroup a second
// staging and ring ramp, which in a short launch showed as a tail of late
// workgroups): chunk c gets workgroups [c grid / C, (c + 1) grid / C) and
// splits its tiles equally among them.  Needs grid >= nchunks.
void chunk_ranges(int64_t ntiles, int nchunks, int grid, WgRange* out) {
  if (grid < nchunks) {
    equal_ranges(ntiles * nchunks, grid, out);
    return;
  }
  for (int c = 0; c < nchunks; ++c) {
    const int w0 = (int)((int64_t)c * grid / nchunks), w1 = (int)((int64_t)(c + 1) * grid / nchunks);
    for (int w = w0; w < w1; ++w) out[w] = WgRange{c * ntiles + ntiles * (w - w0) / (w1 - w0), 0, 0};
  }
  out[grid] = WgRange{ntiles * nchunks, 0, 0};
}

}  // namespace

wq_status check_gemm_args(int fmt, const void* w, const void* s, const void* x, const void* y, int M, int K, int N) {
  wq_status st = check_shape(fmt, M, K, N);
  if (st != WQ_SUCCESS) return st;
  return check_ptrs(fmt, w, s, x, y);
}

}  // namespace wq

using namespace wq;

extern "C" {

const char* wq_status_string(wq_status s) {
  switch (s) {
    case WQ_SUCCESS: return "success";
    case WQ_ERROR_INVALID_VALUE: return "invalid value";
    case WQ_ERROR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case WQ_ERROR_MISALIGNED: return "misaligned pointer";
    case WQ_ERROR_WORKSPACE: return "workspace missing or too small";
    case WQ_ERROR_LAUNCH: return "launch failed";
    case WQ_ERROR_DEVICE: return "no usable gfx950 device";
    case WQ_ERROR_SCRATCH_LIMIT: return "the shape needs more scratch than the library's static buffer holds";
  }
  return "unknown status";
}

size_t wq_gemm_workspace_bytes(int fmt, int M, int K, int N) {
  if (check_shape(fmt, M, K, N) != WQ_SUCCESS) return 0;
  const int cus = current_cus();
  if (cus <= 0) return 0;
  return gemm_workspace(fmt, M, K, N, cus);
}

wq_status wq_gemm_split(int fmt, int M, int K, int in_verify_pass, int* k_chunk, int* n_chunks) {
  if (!k_chunk || !n_chunks) return WQ_ERROR_INVALID_VALUE;
  wq_status st = check_shape(fmt, M, K, 1);
  if (st != WQ_SUCCESS) return st;
  Split sp;
  if (in_verify_pass == 2) {
    sp = is_tiled(fmt) ? blocked_split(fmt, M, K) : verify_split(fmt, M, K);
  } else if (in_verify_pass) {
    sp = verify_split(fmt, M, K);
  } else {
    const int cus = current_cus();
    if (cus <= 0) return WQ_ERROR_DEVICE;
    const TileSplit ts = tile_split_plan(fmt, M, K, cus);
    if (ts.ok) {
      // tiles split across waves and workgroups: reported as k_chunk 0
      *k_chunk = 0;
      *n_chunks = ts.chunks.nchunks;
      return WQ_SUCCESS;
    }
    sp = gemm_split(fmt, M, K, cus);
  }
  *k_chunk = sp.kc;
  *n_chunks = sp.nchunks;
  return WQ_SUCCESS;
}

wq_status wq_gemm_nvfp4(const uint8_t* codes, const uint8_t* scales, float global_scale, const uint16_t* x,
                        float* y, int M, int K, int N, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm(kFmtNvfp4, codes, scales, global_scale, x, y, M, K, N, workspace, workspace_bytes, stream);
}

wq_status wq_gemm_nvfp4_tiled(const uint8_t* tiled, float global_scale, const uint16_t* x, float* y, int M, int K,
                              int N, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm(kFmtNvfp4Tiled, tiled, nullptr, global_scale, x, y, M, K, N, workspace, workspace_bytes, stream);
}

wq_status wq_gemm_fp8row(const uint8_t* w, const float* row_scale, const uint16_t* x, float* y, int M, int K,
                         int N, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm(kFmtFp8Row, w, row_scale, 1.0f, x, y, M, K, N, workspace, workspace_bytes, stream);
}

wq_status wq_gemm_fp8row_tiled(const uint8_t* tiled, const float* row_scale, const uint16_t* x, float* y, int M,
                               int K, int N, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm(kFmtFp8RowTiled, tiled, row_scale, 1.0f, x, y, M, K, N, workspace, workspace_bytes, stream);
}

size_t wq_head_accept_workspace_bytes(int fmt, int M, int K, int N) {
  if (!is_tiled(fmt) || check_shape(fmt, M, K, N) != WQ_SUCCESS) return 0;
  if (verify_split(fmt, M, K).nchunks != 1) return 0;
  const int cus = current_cus();
  if (cus <= 0) return 0;
  return align_up((size_t)cus * 8 * sizeof(uint64_t), kAlign);
}

wq_status wq_head_accept(int fmt, const uint8_t* w, const float* row_scale, float global_scale, const uint16_t* x,
                         int M, int K, int N, const int32_t* drafts, float* logits, int32_t* tokens,
                         int32_t* accepted, void* workspace, size_t workspace_bytes, void* stream) {
  if (!is_tiled(fmt)) return WQ_ERROR_INVALID_VALUE;
  wq_status st = check_shape(fmt, M, K, N);
  if (st != WQ_SUCCESS) return st;
  if (!w || !x || !tokens || !accepted || (fmt == kFmtFp8RowTiled && !row_scale) || (N > 1 && !drafts))
    return WQ_ERROR_INVALID_VALUE;
  if (!aligned16(w) || !aligned16(x) || (row_scale && !aligned16(row_scale)) || (logits && !aligned16(logits)) ||
      ((uintptr_t)tokens & 3u) || ((uintptr_t)accepted & 3u) || ((uintptr_t)drafts & 3u))
    return WQ_ERROR_MISALIGNED;
  const Split sp = verify_split(fmt, M, K);
  if (sp.nchunks != 1) return WQ_ERROR_UNSUPPORTED_SHAPE;
  const int cus = current_cus();
  if (cus <= 0) return WQ_ERROR_DEVICE;
  const int grid = (int)std::min<int64_t>(cus, sp.ntiles);
  if (!workspace || !aligned16(workspace) || workspace_bytes < (size_t)grid * 8 * sizeof(uint64_t))
    return WQ_ERROR_WORKSPACE;
  DevMat one = dev_mat(fmt, w, row_scale, global_scale, x, logits, M, K, sp, nullptr, N, 0);
  one.best = static_cast<uint64_t*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_stream(N, kModeTiledArgmax, nullptr, nullptr, one, grid, lds_bytes_for(N) + kArgLdsBytes, s);
  if (e == hipSuccess) e = launch_accept(one.best, grid, N, drafts, tokens, accepted, s);
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

size_t wq_verify_workspace_bytes(const wq_matrix* descs, int count, int N) {
  if (check_descs(descs, count, N) != WQ_SUCCESS) return 0;
  const int cus = current_cus();
  if (cus <= 0) return 0;
  return pass_layout(descs, count, N, cus).total;
}

wq_status wq_verify_prepare(const wq_matrix* descs, int count, int N, void* workspace, size_t workspace_bytes,
                            void* stream, wq_verify_plan* plan) {
  if (!plan) return WQ_ERROR_INVALID_VALUE;
  wq_status st = check_descs(descs, count, N);
  if (st != WQ_SUCCESS) return st;
  if (!workspace) return WQ_ERROR_WORKSPACE;
  if (!aligned16(workspace)) return WQ_ERROR_MISALIGNED;
  const int cus = current_cus();
  if (cus <= 0) return WQ_ERROR_DEVICE;
  const PassLayout L = pass_layout(descs, count, N, cus);
  if (workspace_bytes < L.total) return WQ_ERROR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  char* scratch = ws + L.table_bytes + L.ranges_bytes + L.tasks_bytes;

  // host staging of the table, the ranges and the reduction runs;
  // thread-local so concurrent calls on different threads do not share it
  thread_local std::vector<char> host;
  host.assign(L.table_bytes + L.ranges_bytes + L.tasks_bytes, 0);
  std::vector<DevMat> mats(count);
  int64_t unit0 = 0;
  bool any_nv = false, any_fp8 = false, any_tiled = false, all_aligned = true;
  for (int i = 0; i < count; ++i) {
    const wq_matrix& d = L.descs[i];
    mats[i] = dev_mat(d.fmt, d.w, d.scales, d.global_scale, d.x, d.y, d.M, d.K, L.splits[i],
                      scratch + L.scratch_off[i], N, unit0);
    unit0 += (int64_t)L.splits[i].nchunks * L.splits[i].ntiles;
    if (d.fmt == kFmtNvfp4) {
      any_nv = true;
      all_aligned = all_aligned && d.K % 64 == 0;
    } else if (is_tiled(d.fmt)) {
      any_tiled = true;
    } else {
      any_fp8 = true;
    }
  }
  int64_t dyn_begin = L.units;
  const std::vector<WgRange> ranges =
      balance(L.descs.data(), count, L, any_tiled && !any_nv && !any_fp8, &dyn_begin);
  std::memcpy(host.data(), mats.data(), sizeof(DevMat) * count);
  std::memcpy(host.data() + L.table_bytes, ranges.data(), sizeof(WgRange) * ranges.size());
  // the dynamic tail: its bounds, zeroed counters and each chunk's matrix
  DynSched dyn{};
  dyn.begin = dyn_begin;
  dyn.end = L.units;
  dyn.chunk = dyn_chunk_units(L.units, L.grid);
  const std::vector<DynClaim> claims = tail_claims(mats, L, dyn_begin, dyn.chunk);
  if ((int64_t)claims.size() > L.dyn_chunks || !blocks_whole(mats, L, ranges, claims)) return WQ_ERROR_INVALID_VALUE;
  dyn.count = (int32_t)claims.size() - 1;
  char* dyn_host = host.data() + L.table_bytes + sizeof(WgRange) * ranges.size();
  std::memcpy(dyn_host, &dyn, sizeof(DynSched));
  std::memcpy(dyn_host + sizeof(DynSched), claims.data(), sizeof(DynClaim) * claims.size());
  if (!L.tasks.empty())
    std::memcpy(host.data() + L.table_bytes + L.ranges_bytes, L.tasks.data(), sizeof(ReduceTask) * L.tasks.size());
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, s) != hipSuccess)
    return WQ_ERROR_LAUNCH;
  plan->workspace = workspace;
  plan->workspace_bytes = workspace_bytes;
  plan->count = count;
  plan->N = N;
  const int kinds = (int)any_nv + (int)any_fp8 + (int)any_tiled;
  plan->mode = kinds > 1 ? kModeMixed
               : any_fp8 ? kModeFp8
               : any_tiled ? kModeTiled
               : all_aligned ? kModeNvfp4Aligned : kModeNvfp4;
  plan->grid = L.grid;
  plan->ranges_offset = L.table_bytes;
  plan->reduce_offset = L.table_bytes + L.ranges_bytes;
  plan->reduce_runs = (int32_t)L.tasks.size();
  plan->lds_extra = (int32_t)L.lds_extra;
  return WQ_SUCCESS;
}

// LDS past the X chunk and the zero block: the blocked chunk sums of an
// all-tiled pass, or nothing
static bool lds_extra_ok(const wq_verify_plan& p) {
  return p.lds_extra == 0 || (p.mode == kModeTiled && lds_bytes_for(p.N) + (uint32_t)p.lds_extra == kLdsLimit);
}

wq_status wq_verify_launch(const wq_verify_plan* plan, void* stream) {
  if (!plan || !plan->workspace || plan->N < 1 || plan->N > 8 || plan->grid < 1 || plan->count < 1 ||
      plan->mode < kModeNvfp4Aligned || plan->mode > kModeTiled || plan->ranges_offset >= plan->workspace_bytes ||
      plan->reduce_runs < 0 || (plan->reduce_runs > 0 && plan->reduce_offset >= plan->workspace_bytes) ||
      !lds_extra_ok(*plan))
    return WQ_ERROR_INVALID_VALUE;
  const char* ws = static_cast<const char*>(plan->workspace);
  const DevMat none{};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_stream(plan->N, plan->mode, reinterpret_cast<const DevMat*>(ws),
                               reinterpret_cast<const WgRange*>(ws + plan->ranges_offset), none, plan->grid,
                               lds_bytes_for(plan->N) + (size_t)plan->lds_extra, s);
  if (e == hipSuccess && plan->reduce_runs > 0)
    e = launch_reduce(reinterpret_cast<const DevMat*>(ws), reinterpret_cast<const ReduceTask*>(ws + plan->reduce_offset),
                      none, plan->reduce_runs, plan->N, s);
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_verify_launch_valu(const wq_verify_plan* plan, void* stream) {
  if (!plan || !plan->workspace || plan->N < 1 || plan->N > 8 || plan->grid < 1 || plan->count < 1 ||
      plan->mode != kModeTiled || plan->ranges_offset >= plan->workspace_bytes || plan->reduce_runs < 0 ||
      (plan->reduce_runs > 0 && plan->reduce_offset >= plan->workspace_bytes) || !lds_extra_ok(*plan))
    return WQ_ERROR_INVALID_VALUE;
  const char* ws = static_cast<const char*>(plan->workspace);
  const DevMat none{};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_stream(plan->N, kModeTiledValu, reinterpret_cast<const DevMat*>(ws),
                               reinterpret_cast<const WgRange*>(ws + plan->ranges_offset), none, plan->grid,
                               lds_bytes_for(plan->N) + (size_t)plan->lds_extra, s);
  if (e == hipSuccess && plan->reduce_runs > 0)
    e = launch_reduce(reinterpret_cast<const DevMat*>(ws), reinterpret_cast<const ReduceTask*>(ws + plan->reduce_offset),
                      none, plan->reduce_runs, plan->N, s);
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_verify_launch_n(const wq_verify_plan* plan, const int32_t* n_device, void* stream) {
  if (!plan || !plan->workspace || !n_device || ((uintptr_t)n_device & 3u) || plan->N != 8 || plan->grid < 1 ||
      plan->count < 1 || plan->mode != kModeTiled || plan->ranges_offset >= plan->workspace_bytes ||
      plan->reduce_runs < 0 || (plan->reduce_runs > 0 && plan->reduce_offset >= plan->workspace_bytes) ||
      !lds_extra_ok(*plan))
    return WQ_ERROR_INVALID_VALUE;
  const char* ws = static_cast<const char*>(plan->workspace);
  const DevMat none{};
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = launch_stream_dyn(reinterpret_cast<const DevMat*>(ws),
                                   reinterpret_cast<const WgRange*>(ws + plan->ranges_offset), n_device, plan->grid,
                                   lds_bytes_for(8) + (size_t)plan->lds_extra, s);
  if (e == hipSuccess && plan->reduce_runs > 0)
    e = launch_reduce(reinterpret_cast<const DevMat*>(ws), reinterpret_cast<const ReduceTask*>(ws + plan->reduce_offset),
                      none, plan->reduce_runs, 8, s, n_device);
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_verify_pass(const wq_matrix* descs, int count, int N, void* workspace, size_t workspace_bytes,
                         void* stream) {
  wq_verify_plan plan;
  wq_status st = wq_verify_prepare(descs, count, N, workspace, workspace_bytes, stream, &plan);
  if (st != WQ_SUCCESS) return st;
  return wq_verify_launch(&plan, stream);
}

size_t wq_mlp_chain_workspace_bytes(int layers, int D, int F, int N) {
  if (check_chain_shape(layers, D, F, N) != WQ_SUCCESS) return 0;
  const int cus = current_cus();
  if (cus <= 0) return 0;
  return chain_layout(layers, D, F, N, cus).total;
}

wq_status wq_mlp_chain_split(int D, int F, int* k_chunk, int* n_chunks) {
  if (!k_chunk || !n_chunks) return WQ_ERROR_INVALID_VALUE;
  wq_status st = check_chain_shape(1, D, F, 1);
  if (st != WQ_SUCCESS) return st;
  const int cus = current_cus();
  if (cus <= 0) return WQ_ERROR_DEVICE;
  const Split sp = chain_down_split(D, F, cus);
  *k_chunk = sp.kc;
  *n_chunks = sp.nchunks;
  return WQ_SUCCESS;
}

wq_status wq_mlp_chain_prepare(const wq_mlp_layer* layers, int count, int D, int F, int N, float eps, float* h,
                               uint16_t* a, uint16_t* s, void* workspace, size_t workspace_bytes, void* stream,
                               wq_mlp_plan* plan) {
  if (!plan || !layers) return WQ_ERROR_INVALID_VALUE;
  wq_status st = check_chain_shape(count, D, F, N);
  if (st != WQ_SUCCESS) return st;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return WQ_ERROR_INVALID_VALUE;
  if (!h || !a || !s) return WQ_ERROR_INVALID_VALUE;
  if (!aligned16(h) || !aligned16(a) || !aligned16(s)) return WQ_ERROR_MISALIGNED;
  for (int l = 0; l < count; ++l) {
    const wq_mlp_layer& y = layers[l];
    if (!y.gate_up || !y.down || !y.gamma) return WQ_ERROR_INVALID_VALUE;
    if (!aligned16(y.gate_up) || !aligned16(y.down) || !aligned16(y.gamma)) return WQ_ERROR_MISALIGNED;
  }
  if (!workspace) return WQ_ERROR_WORKSPACE;
  if (!aligned16(workspace)) return WQ_ERROR_MISALIGNED;
  const int cus = current_cus();
  if (cus <= 0) return WQ_ERROR_DEVICE;
  const ChainLayout L = chain_layout(count, D, F, N, cus);
  if (workspace_bytes < L.total) return WQ_ERROR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  const size_t off_rgu = L.table_bytes;
  const size_t off_rdn = off_rgu + L.ranges_gu_bytes;
  const size_t off_ctl = off_rdn + L.ranges_down_bytes;
  const size_t off_part = off_ctl + L.ctl_bytes;
  const size_t off_ssp = off_part + L.part_bytes;
  float* part = reinterpret_cast<float*>(ws + off_part);
  float* ssp = reinterpret_cast<float*>(ws + off_ssp);

  thread_local std::vector<char> host;
  host.assign(off_part, 0);
  DevMat* mats = reinterpret_cast<DevMat*>(host.data());
  for (int l = 0; l < count; ++l) {
    const wq_mlp_layer& y = layers[l];
    DevMat g{};
    g.w = static_cast<const uint8_t*>(y.gate_up);
    g.fmt = kFmtNvfp4Tiled;
    g.M = 2 * F;
    g.K = D;
    g.kc = L.gate_up.kc;
    g.nchunks = 1;
    g.ntiles = L.gate_up.ntiles;
    g.g = y.gate_scale;
    g.g2 = y.up_scale;
    g.eps = eps;
    g.h = h;
    g.ssp = ssp;
    g.nparts = L.parts;
    g.gamma = y.gamma;
    g.aout = a;
    g.sout = s;
    mats[2 * l] = g;
    // one chunk: the tile epilogue writes g * sum to plane 0 as y
    mats[2 * l + 1] = dev_mat(kFmtNvfp4Tiled, y.down, nullptr, y.down_scale, s, L.down.nchunks > 1 ? nullptr : part,
                              D, F, L.down, reinterpret_cast<char*>(part), N, 0);
  }
  equal_ranges(L.gate_up.ntiles, L.grid_gate_up, reinterpret_cast<WgRange*>(host.data() + off_rgu));
  chunk_ranges(L.down.ntiles, L.down.nchunks, L.grid_down, reinterpret_cast<WgRange*>(host.data() + off_rdn));
  if (hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return WQ_ERROR_LAUNCH;
  plan->workspace = workspace;
  plan->workspace_bytes = workspace_bytes;
  plan->h = h;
  plan->layers = count;
  plan->D = D;
  plan->F = F;
  plan->N = N;
  plan->grid_gate_up = L.grid_gate_up;
  plan->grid_down = L.grid_down;
  plan->down_chunks = L.down.nchunks;
  // the single-launch chain: as many workgroups as stay resident (all CUs)
  const int per_cu = chain_persistent_blocks_per_cu(N);
  plan->grid_chain = per_cu > 0 ? cus * std::min(per_cu, 1) : 0;
  plan->ranges_gate_up_offset = off_rgu;
  plan->ranges_down_offset = off_rdn;
  plan->ssp_offset = off_ssp;
  plan->ctl_offset = off_ctl;
  return WQ_SUCCESS;
}

wq_status wq_mlp_chain_launch(const wq_mlp_plan* plan, void* stream) {
  if (!plan || !plan->workspace || !plan->h || plan->layers < 1 || plan->N < 1 || plan->N > 8 ||
      plan->grid_gate_up < 1 || plan->grid_down < 1 || plan->D < 1 ||
      plan->ranges_gate_up_offset >= plan->workspace_bytes || plan->ranges_down_offset >= plan->workspace_bytes ||
      plan->ssp_offset >= plan->workspace_bytes)
    return WQ_ERROR_INVALID_VALUE;
  const char* ws = static_cast<const char*>(plan->workspace);
  const DevMat* mats = reinterpret_cast<const DevMat*>(ws);
  const WgRange* rgu = reinterpret_cast<const WgRange*>(ws + plan->ranges_gate_up_offset);
  const WgRange* rdn = reinterpret_cast<const WgRange*>(ws + plan->ranges_down_offset);
  float* ssp = reinterpret_cast<float*>(static_cast<char*>(plan->workspace) + plan->ssp_offset);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const DevMat none{};
  const int N = plan->N;
  hipError_t e = launch_chain_reduce(plan->h, nullptr, plan->D, N, ssp, s);
  for (int l = 0; l < plan->layers && e == hipSuccess; ++l) {
    e = launch_stream(N, kModeTiledGlu, mats + 2 * l, rgu, none, plan->grid_gate_up, lds_bytes_for(N) + kArgLdsBytes,
                      s);
    if (e == hipSuccess)
      e = launch_stream(N, kModeTiledWide, mats + 2 * l + 1, rdn, none, plan->grid_down, lds_bytes_for(N), s);
    if (e == hipSuccess) e = launch_chain_reduce(plan->h, mats + 2 * l + 1, plan->D, N, ssp, s);
  }
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

wq_status wq_mlp_chain_launch_persistent(const wq_mlp_plan* plan, void* stream) {
  if (!plan || !plan->workspace || !plan->h || plan->layers < 1 || plan->N < 1 || plan->N > 8 || plan->D < 1 ||
      plan->grid_chain < 0 || plan->ssp_offset >= plan->workspace_bytes || plan->ctl_offset >= plan->workspace_bytes ||
      ((plan->ctl_offset | plan->ssp_offset) & 15u))
    return WQ_ERROR_INVALID_VALUE;
  if (plan->grid_chain == 0) return WQ_ERROR_UNSUPPORTED_SHAPE;
  char* ws = static_cast<char*>(plan->workspace);
  // the launches' range tables (down's aligned to its K chunks) when they
  // were built for as many workgroups as the single launch has, else equal
  // splits
  const bool same_grid = plan->grid_gate_up == plan->grid_chain && plan->grid_down == plan->grid_chain &&
                         plan->ranges_gate_up_offset < plan->workspace_bytes &&
                         plan->ranges_down_offset < plan->workspace_bytes;
  const WgRange* rgu = same_grid ? reinterpret_cast<const WgRange*>(ws + plan->ranges_gate_up_offset) : nullptr;
  const WgRange* rdn = same_grid ? reinterpret_cast<const WgRange*>(ws + plan->ranges_down_offset) : nullptr;
  const hipError_t e = launch_chain_persistent(plan->N, reinterpret_cast<const DevMat*>(ws),
                                               reinterpret_cast<ChainCtl*>(ws + plan->ctl_offset), plan->h,
                                               reinterpret_cast<float*>(ws + plan->ssp_offset), plan->layers, plan->D,
                                               plan->grid_chain, rgu, rdn, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? WQ_SUCCESS : WQ_ERROR_LAUNCH;
}

}  // extern "C"
