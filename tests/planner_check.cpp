// Host check of the verify-pass planner (no GPU): for the dense 64-layer
// pass and a few hundred random passes, it builds the plan as
// wq_verify_prepare does, replays the persistent kernel's walk over every
// workgroup's static range and every claim of the dynamic tail (the same
// segment arithmetic as stream_body), and checks what the kernel relies on:
//  - every (matrix, chunk, tile) is computed exactly once;
//  - a blocked split matrix is walked in whole tiles, each block's chunks
//    back to back and in order in one walk, no block longer than its LDS
//    slots, and its slots lie between its X chunk and the zero block or
//    past the zero block, inside the launch's LDS;
//  - ranges and claims start on tile boundaries of blocked matrices, the
//    claim table fits its space, and the dense pass's tail avoids them.
// Exit status 0 and a last line "all ok" when every check holds.
#include "wq_api.cpp"

#include <cstdio>
#include <random>

// The dynamic tail's 64-bit claim counter is 8-byte aligned in the
// workspace: DynSched follows the 16-byte WgRange entries.
static_assert(sizeof(wq::WgRange) == 16 && offsetof(wq::DynSched, next) % 8 == 0, "claim counter alignment");

using namespace wq;

struct Seg {
  int mat, chunk, t0, t1, ptile0;
};

static int g_N = 1;
static int btiles(int kc) {
  const int na = (int)((2u * (uint32_t)(kKcMax - kc) * (uint32_t)g_N) / kPartTileBytes);
  return std::min(kPartTilesMax, na + part_tiles_for(g_N));
}
static bool walk(const std::vector<DevMat>& mats, int64_t u, int64_t u_end, int mi, std::vector<Seg>& out) {
  int bchunk = 0;
  while (u < u_end) {
    if (mi >= (int)mats.size()) return false;
    const DevMat& mt = mats[mi];
    const int64_t mend = mt.unit0 + (int64_t)mt.nchunks * mt.ntiles;
    if (u >= mend) { ++mi; continue; }
    if (u < mt.unit0) return false;
    const int64_t local = u - mt.unit0;
    int chunk, ptile0 = -1;
    int64_t first, run_end, ubase;
    if (mt.tb > 0) {
      const int nc = mt.nchunks;
      if (local % nc) return false;
      const int t0 = (int)(local / nc);
      const int t1 = std::min(t0 + btiles(mt.kc), (int)((std::min(u_end, mend) - mt.unit0) / nc));
      if ((std::min(u_end, mend) - mt.unit0) % nc) return false;
      chunk = bchunk; first = t0; run_end = t1; ubase = 0; ptile0 = t0;
      if (++bchunk == nc) { bchunk = 0; u = mt.unit0 + (int64_t)t1 * nc; }
    } else {
      chunk = (int)(local / mt.ntiles);
      ubase = mt.unit0 + (int64_t)chunk * mt.ntiles;
      first = u;
      run_end = std::min(u_end, ubase + mt.ntiles);
      u = run_end;
    }
    out.push_back(Seg{mi, chunk, (int)(first - ubase), (int)(run_end - ubase), ptile0});
  }
  return bchunk == 0;
}

static int check(const std::vector<wq_matrix>& descs, int N, int cus, const char* name) {
  g_N = N;
  const int count = (int)descs.size();
  const PassLayout L = pass_layout(descs.data(), count, N, cus);
  std::vector<DevMat> mats(count);
  int64_t unit0 = 0;
  bool tiled_only = true;
  for (int i = 0; i < count; ++i) {
    const wq_matrix& d = L.descs[i];
    mats[i] = dev_mat(d.fmt, d.w, d.scales, d.global_scale, d.x, d.y, d.M, d.K, L.splits[i], nullptr, N, unit0);
    unit0 += (int64_t)L.splits[i].nchunks * L.splits[i].ntiles;
    tiled_only = tiled_only && is_tiled(d.fmt);
  }
  int64_t dyn_begin = L.units;
  const std::vector<WgRange> ranges = balance(L.descs.data(), count, L, tiled_only, &dyn_begin);
  const int chunk = dyn_chunk_units(L.units, L.grid);
  const std::vector<DynClaim> claims = tail_claims(mats, L, dyn_begin, chunk);
  int bad = 0;
  if ((int64_t)claims.size() > L.dyn_chunks) { printf("%s: %zu claims > %lld\n", name, claims.size(), (long long)L.dyn_chunks); ++bad; }
  if (!blocks_whole(mats, L, ranges, claims)) { printf("%s: blocks_whole false\n", name); ++bad; }
  if (claims.front().begin != dyn_begin || claims.back().begin != L.units) { printf("%s: claim bounds\n", name); ++bad; }
  // coverage
  std::vector<std::vector<int>> cov(count);
  for (int i = 0; i < count; ++i) cov[i].assign((size_t)mats[i].nchunks * mats[i].ntiles, 0);
  std::vector<std::vector<Seg>> walks;
  for (int w = 0; w < L.grid; ++w) {
    std::vector<Seg> s;
    if (!walk(mats, ranges[w].begin, ranges[w + 1].begin, ranges[w].mat, s)) { printf("%s: walk wg %d\n", name, w); ++bad; }
    walks.push_back(s);
  }
  for (size_t k = 0; k + 1 < claims.size(); ++k) {
    std::vector<Seg> s;
    if (!walk(mats, claims[k].begin, claims[k + 1].begin, claims[k].mat, s)) { printf("%s: walk claim %zu\n", name, k); ++bad; }
    walks.push_back(s);
  }
  for (const auto& s : walks) {
    for (size_t j = 0; j < s.size(); ++j) {
      const Seg& g = s[j];
      const DevMat& mt = mats[g.mat];
      for (int t = g.t0; t < g.t1; ++t) {
        if (t < 0 || t >= mt.ntiles) { ++bad; continue; }
        cov[g.mat][(size_t)g.chunk * mt.ntiles + t]++;
      }
      if (mt.tb > 0) {
        if (g.t0 != g.ptile0 || g.t1 - g.t0 > btiles(mt.kc) || g.t1 <= g.t0) { printf("%s: bad block seg\n", name); ++bad; }
        // chunks of a block follow each other in the same walk, in order
        if (g.chunk > 0) {
          if (j == 0 || s[j - 1].mat != g.mat || s[j - 1].chunk != g.chunk - 1 || s[j - 1].ptile0 != g.ptile0 ||
              s[j - 1].t1 != g.t1) {
            printf("%s: chunk %d of block %d not after chunk %d\n", name, g.chunk, g.ptile0, g.chunk - 1);
            ++bad;
          }
        }
        if (g.chunk < mt.nchunks - 1) {
          if (j + 1 >= s.size() || s[j + 1].mat != g.mat || s[j + 1].chunk != g.chunk + 1 || s[j + 1].ptile0 != g.ptile0) {
            printf("%s: chunk %d of block %d not followed\n", name, g.chunk, g.ptile0);
            ++bad;
          }
        }
      }
    }
  }
  for (int i = 0; i < count; ++i)
    for (size_t k = 0; k < cov[i].size(); ++k)
      if (cov[i][k] != 1) { if (bad < 20) printf("%s: mat %d unit %zu covered %d\n", name, i, k, cov[i][k]); ++bad; }
  // the tail holds no blocked unit
  // LDS of the blocked slots: region A inside [2 kc N, zero block), region B
  // past the zero block and inside the allocation
  for (int i = 0; i < count; ++i) {
    const DevMat& mt = mats[i];
    if (mt.tb == 0) continue;
    const uint32_t xbytes = 2u * mt.kc * N, zoff = 2u * kKcMax * N, zb = 512u * N;
    const uint32_t alloc = 2u * kKcMax * N + 512u * N + L.lds_extra;
    const int na = (int)((2u * (uint32_t)(kKcMax - mt.kc) * (uint32_t)N) / kPartTileBytes);
    const int nb = std::max(0, btiles(mt.kc) - na);
    if (xbytes + 512u * na > zoff || zoff + zb + 512u * nb > alloc || alloc > kLdsLimit || btiles(mt.kc) < 1) {
      printf("%s: LDS slots of mat %d out of place\n", name, i);
      ++bad;
    }
  }
  int tail_blocked = 0;
  for (size_t k = 0; k + 1 < claims.size(); ++k) tail_blocked += mats[claims[k].mat].tb > 0;
  if (tail_blocked && strncmp(name, "dense64", 7) == 0) { printf("%s: tail claim in a blocked matrix\n", name); ++bad; }
  // balance report
  int64_t blocked = 0;
  for (int i = 0; i < count; ++i) blocked += L.splits[i].tb > 0;
  printf("%-28s N=%d cus=%3d units=%7lld grid=%3d tail=%6lld claims=%5zu blocked mats=%lld lds_extra=%u tasks=%zu tb=%d tailblk=%d %s\n",
         name, N, cus, (long long)L.units, L.grid, (long long)(L.units - dyn_begin), claims.size() - 1,
         (long long)blocked, L.lds_extra, L.tasks.size(), count && mats[0].tb ? btiles(mats[0].kc) : 0, tail_blocked, bad ? "FAIL" : "ok");
  return bad;
}

static wq_matrix mk(int fmt, int M, int K) {
  static char dummy[64];
  wq_matrix d{};
  d.fmt = fmt;
  d.M = M;
  d.K = K;
  d.global_scale = 1.0f;
  d.w = dummy;
  d.scales = dummy;
  d.x = reinterpret_cast<const uint16_t*>(dummy);
  d.y = reinterpret_cast<float*>(dummy);
  return d;
}

// The single-product split plan (tile_split_plan) replayed as split_kernel
// walks it: workgroups shared out among the chunks, each an equal share of
// its chunk's tiles, wave pieces, the tiles each piece touches (its LDS
// slots), the parts each workgroup writes and the arrivals per tile.
// Checks: every (tile, step) once; slots and arrivals within their bounds;
// the launch's LDS at N = 8 within the limit; with several chunks, every
// tile-chunk's part written once (C arrivals per tile), with one chunk, none.
static int check_tile_split(int fmt, int M, int K, int cus) {
  const TileSplit ts = tile_split_plan(fmt, M, K, cus);
  if (!ts.ok) return 0;
  const int sk = seg_k(fmt);
  const int64_t T = ceil_div(M, 16), S = ceil_div(K, sk);
  const int64_t C = ts.chunks.nchunks;
  const int64_t sf = ts.chunks.kc / sk, sl = S - (C - 1) * sf;
  const int64_t U = T * S, G = ts.grid;
  const int W = kSplitThreads / 64;
  int bad = 0;
  if (ts.chunks.ntiles != T || sl < 1 || sl > sf || C > kSplitChunksMax) ++bad;
  if (lds_bytes_for(8) + (uint64_t)W * ts.slots * kSplitPartBytes + kSplitStaticLds > 160u * 1024u) ++bad;
  if (G < C || G > cus || T > kSplitMaxTiles || U >= (1ll << 31)) ++bad;
  std::vector<int> seen(U, 0), parts((size_t)(C * T), 0);
  for (int64_t g = 0; g < G; ++g) {
    const int64_t ch = (C * (g + 1) - 1) / G;
    const int64_t g0 = G * ch / C, gc = G * (ch + 1) / C - g0;
    if (g < g0 || g >= g0 + gc || ch >= C) { ++bad; continue; }
    const int64_t ta = T * (g - g0) / gc, tb = T * (g - g0 + 1) / gc;
    if (ta >= tb) continue;
    const int64_t n = ch == C - 1 ? sl : sf;
    const int64_t la = ta * n, lb = tb * n;
    for (int w = 0; w < W; ++w) {
      const int64_t e0 = la + (lb - la) * w / W, e1 = la + (lb - la) * (w + 1) / W;
      if (e0 < e1 && (e1 - 1) / n - e0 / n + 1 > ts.slots) ++bad;
      for (int64_t e = e0; e < e1; ++e) seen[(e / n) * S + ch * sf + e % n] += 1;
    }
    if (C > 1) {
      if (tb - ta > kSplitArrivalsMax) ++bad;
      for (int64_t t = ta; t < tb; ++t) parts[ch * T + t] += 1;
    }
  }
  for (int64_t i = 0; i < U; ++i)
    if (seen[i] != 1) { ++bad; break; }
  for (int64_t i = 0; i < C * T; ++i)
    if (parts[i] != (C > 1 ? 1 : 0)) { ++bad; break; }
  if (bad) printf("tile split fmt=%d M=%d K=%d cus=%d: %d problems\n", fmt, M, K, cus, bad);
  return bad;
}

int main() {
  int bad = 0;
  {
    // the single products of the benchmark, and random small ones
    int nsplit = 0;
    const int shapes[][3] = {{kFmtNvfp4Tiled, 1024, 1024}, {kFmtNvfp4Tiled, 17408, 5120},
                             {kFmtNvfp4Tiled, 5120, 17408}, {kFmtNvfp4Tiled, 1, 32},
                             {kFmtNvfp4Tiled, 96, 17408},   {kFmtFp8RowTiled, 40, 17424},
                             {kFmtNvfp4Tiled, 1000, 8736},  {kFmtFp8RowTiled, 1, 16}};
    for (const auto& sh : shapes)
      for (int cus : {256, 304, 80, 1}) {
        bad += check_tile_split(sh[0], sh[1], sh[2], cus);
        nsplit += tile_split_plan(sh[0], sh[1], sh[2], cus).ok;
      }
    std::mt19937 rng(7);
    for (int it = 0; it < 3000; ++it) {
      const bool fp8 = rng() % 3 == 0;
      int K = (fp8 ? 16 : 32) * (1 + (int)(rng() % 1100));
      const int M = 1 + (int)(rng() % 33000);
      const int cus = (int[]){1, 3, 64, 256, 304}[rng() % 5];
      bad += check_tile_split(fp8 ? kFmtFp8RowTiled : kFmtNvfp4Tiled, M, K, cus);
      nsplit += tile_split_plan(fp8 ? kFmtFp8RowTiled : kFmtNvfp4Tiled, M, K, cus).ok;
    }
    const TileSplit c1 = tile_split_plan(kFmtNvfp4Tiled, 17408, 5120, 256);
    const TileSplit c2 = tile_split_plan(kFmtNvfp4Tiled, 5120, 17408, 256);
    printf("tile split: %d plans checked; 17408x5120: ok=%d grid=%d chunks=%d kc=%d slots=%d; "
           "5120x17408: ok=%d grid=%d chunks=%d kc=%d slots=%d\n",
           nsplit, c1.ok, c1.grid, c1.chunks.nchunks, c1.chunks.kc, c1.slots, c2.ok, c2.grid, c2.chunks.nchunks,
           c2.chunks.kc, c2.slots);
    if (!c1.ok || !c2.ok) ++bad;
  }
  std::vector<wq_matrix> dense;
  for (int l = 0; l < 64; ++l) {
    dense.push_back(mk(kFmtNvfp4Tiled, 7168, 5120));
    dense.push_back(mk(kFmtNvfp4Tiled, 5120, 6144));
    dense.push_back(mk(kFmtNvfp4Tiled, 34816, 5120));
    dense.push_back(mk(kFmtNvfp4Tiled, 5120, 17408));
  }
  for (int N : {2, 4, 8})
    for (int cus : {256, 304, 80, 1}) bad += check(dense, N, cus, "dense64");
  std::vector<wq_matrix> plain_dense;
  for (auto d : dense) { d.fmt = kFmtNvfp4; plain_dense.push_back(d); }
  bad += check(plain_dense, 8, 256, "dense64 plain");
  std::vector<wq_matrix> layer(dense.begin(), dense.begin() + 4);
  for (int N = 1; N <= 8; ++N) bad += check(layer, N, 256, "one layer");
  std::vector<wq_matrix> inv = {mk(kFmtNvfp4Tiled, 96, 17408), mk(kFmtNvfp4Tiled, 40, 17440),
                                mk(kFmtNvfp4Tiled, 33, 8736), mk(kFmtNvfp4Tiled, 17, 544)};
  for (int N = 1; N <= 8; ++N) bad += check(inv, N, 256, "invariance");
  std::vector<wq_matrix> tail = {mk(kFmtNvfp4Tiled, 1100000, 256), mk(kFmtNvfp4Tiled, 8192, 17408)};
  bad += check(tail, 3, 256, "tail + blocked");
  std::vector<wq_matrix> tail2 = {mk(kFmtNvfp4Tiled, 8192, 17408), mk(kFmtNvfp4Tiled, 1100000, 256),
                                  mk(kFmtFp8RowTiled, 4000, 17424)};
  bad += check(tail2, 5, 256, "blocked + tail + fp8");
  std::mt19937 rng(12345);
  const int ks[] = {256, 512, 5120, 8704, 8736, 17408, 17440, 26112, 40000};
  for (int it = 0; it < 400; ++it) {
    std::vector<wq_matrix> v;
    const int cnt = 1 + rng() % 12;
    for (int i = 0; i < cnt; ++i) {
      const bool fp8 = rng() % 4 == 0;
      int K = ks[rng() % 9];
      if (!fp8) K = (K / 32) * 32;
      int M = 1 + rng() % (rng() % 3 == 0 ? 400000 : 3000);
      v.push_back(mk(fp8 ? kFmtFp8RowTiled : kFmtNvfp4Tiled, M, K));
    }
    const int N = 1 + rng() % 8;
    const int cus = (int[]){1, 3, 64, 256, 304}[rng() % 5];
    char nm[32];
    snprintf(nm, sizeof nm, "random %d", it);
    const int b = check(v, N, cus, nm);
    bad += b;
  }
  printf("%s (%d problems)\n", bad ? "FAILED" : "all ok", bad);
  return bad ? 1 : 0;
}
