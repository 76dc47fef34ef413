// Per-row top-k of fp32 scores, indices returned in ascending order.
//
// QUOKA write-up, section 2.3 listing: the BSA keys with the largest
// aggregated score per KV head.  Ties go to the lower position and -0.0
// equals +0.0, so the selected set is unique.
//
// One workgroup of 1024 threads per row.  Layout: wave w covers the span
// [w * 64 * ITEMS, (w + 1) * 64 * ITEMS) of the row in groups of 256
// elements; lane l holds elements 4l .. 4l + 3 of each group, so every load
// instruction of a wave reads 1 KiB contiguous and every store of selected
// positions lands in a narrow window.  The row stays in registers and the
// per-element work is kept to a few instructions per phase, because a single
// CU's issue rate bounds this kernel:
//   1. min / max of the row;
//   2. histogram over 2048 equal-width value bins between min and max (the
//      bin index is monotone in the value, so every bin above the one holding
//      the k-th largest value is selected whole); the bin of every element is
//      kept, packed, in registers; one wave finds the boundary bin;
//   3. the boundary bin's elements are appended to an LDS list (per-thread
//      bitmask, one wave prefix sum and one LDS atomic per wave);
//   4. the exact threshold among them: each candidate is ranked against the
//      others (an 8-bit radix select takes over for very large bins);
//   5. compaction in index order: every element above the threshold, plus the
//      first `need` elements equal to it.  Output offsets come from one wave
//      prefix sum per group of four elements and one block sum over waves.
// Rows longer than 16K scores, and rows longer than 4K when there are too few
// to fill the chip, take the split path below instead.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kTopkThreads = 1024;
static_assert(kL1Bins == kL1BinsHost, "one bin count for host and device");
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kCand = 4096;  // boundary-bin candidates kept in LDS

__device__ __forceinline__ uint32_t fkey(float x) { return order_key(x); }
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

constexpr int kHistWords = hist_words(kBins);

struct TopkShared {
  int hist[kHistWords];
  uint32_t cand[kCand];
  uint32_t wsum[kTopkWaves];
  int wtot[kTopkWaves];
  float red_min[kTopkWaves], red_max[kTopkWaves];
  int bin, above, nbin, cnt, need;
  uint32_t tau;
};

// Boundary bin of a histogram held two bins per thread (thread t: bins 2t and
// 2t + 1, counts c0 and c1): the bin b with count(bins > b) < need <=
// count(bins >= b), for 1 <= need <= total.  The whole block takes part: one
// wave prefix sum, the waves' totals through LDS, then the one thread whose
// bin it is writes (bin, above, its count).  Every thread calls this; the
// results are visible after the second barrier.
__device__ __forceinline__ void block_crossing(int c0, int c1, int need, int* wtot, int* bin,
                                               int* above, int* count) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = threadIdx.x;
  const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(c0 + c1)));
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int below = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int v = wtot[w];
    total += v;
    below += w < wave ? v : 0;
  }
  const int above1 = total - below - incl;  // bins > 2t + 1
  const int above0 = above1 + c1;           // bins > 2t
  if (above1 < need && need <= above1 + c1) {
    *bin = 2 * t + 1;
    *above = above1;
    *count = c1;
  } else if (above0 < need && need <= above0 + c0) {
    *bin = 2 * t;
    *above = above0;
    *count = c0;
  }
  __syncthreads();
}

// Exact threshold among the LDS candidate list: the need-th largest key.
// Writes sh.tau and sh.need (copies of the threshold still to take).
// `visit_bin(f)` calls f(x) for every real element of bin B of this thread
// (used only when the candidates overflow the list).
template <typename VisitBin>
__device__ void exact_threshold(TopkShared& sh, int need, VisitBin visit_bin) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const int ncand = sh.cnt;
  if (ncand <= kTopkThreads) {
    if (tid < ncand) {
      const uint32_t mine = sh.cand[tid];
      int gt = 0, eq = 0;
      for (int c = 0; c < ncand; ++c) {
        const uint32_t o = sh.cand[c];
        gt += o > mine;
        eq += o == mine;
      }
      if (gt < need && need <= gt + eq) {  // every holder of this key agrees
        sh.tau = mine;
        sh.need = need - gt;
      }
    }
    __syncthreads();
    return;
  }
  const bool in_lds = ncand <= kCand;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < hpad(256); i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    auto count = [&](uint32_t kx) {
      if ((kx & pmask) == prefix) atomicAdd(&sh.hist[hpad((kx >> shift) & 255u)], 1);
    };
    if (in_lds) {
      for (int c = tid; c < ncand; c += kTopkThreads) count(sh.cand[c]);
    } else {
      visit_bin([&](float x) { count(fkey(x)); });
    }
    __syncthreads();
    if (wave == 0) wave_crossing<4>(sh.hist, need, &sh.bin, &sh.above);
    __syncthreads();
    need -= sh.above;
    prefix |= static_cast<uint32_t>(min(max(sh.bin, 0), 255)) << shift;
    pmask |= 0xffu << shift;
    __syncthreads();
  }
  if (tid == 0) {
    sh.tau = prefix;
    sh.need = need;
  }
  __syncthreads();
}

// Position of element e (0 <= e < ITEMS) of this thread in a tile of
// 1024 * ITEMS elements starting at `base`.
template <int ITEMS>
__device__ __forceinline__ int tile_pos(int base, int e) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return base + wave * 64 * ITEMS + (e >> 2) * 256 + 4 * lane + (e & 3);
}

// Loads this thread's elements of the tile at `base` (-inf beyond n); the
// returned mask has bit e set for real elements.  Branch-free, so that all
// loads are in flight together: addresses past the row are clamped into it.
// VEC (rows 16-byte aligned, n a multiple of 4): one 16-byte load per group.
template <int ITEMS, bool VEC>
__device__ __forceinline__ uint32_t load_tile(const float* s, int base, int n, float* x) {
  uint32_t valid = 0;
#pragma unroll
  for (int m = 0; m < ITEMS / 4; ++m) {
    const int p = tile_pos<ITEMS>(base, 4 * m);
    if constexpr (VEC) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s + min(p, n - 4));
#pragma unroll
      for (int j = 0; j < 4; ++j) x[4 * m + j] = p < n ? v[j] : -INFINITY;
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = s[min(p + j, n - 1)];
        x[4 * m + j] = p + j < n ? v : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) valid |= static_cast<uint32_t>(p + j < n) << (4 * m + j);
  }
  return valid;
}

// Writes, in ascending position order, the positions of the tile's elements
// in gmask (above the threshold) and the first elements of emask (equal to
// it) while fewer than `need` equal elements have been taken in the whole row.
// (base_gt, base_eq) count the elements of earlier tiles and are advanced by
// this tile's totals.  Every thread of the block calls this, once, as the
// kernel's last step (wsum is not released for reuse).
template <int ITEMS>
__device__ void write_picks(uint32_t gmask, uint32_t emask, int base, int need, int k,
                            int32_t* out, uint32_t* wsum, int& base_gt, int& base_eq) {
  constexpr int M = ITEMS / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // packed (greater | equal << 16) counts; a tile holds at most 32768 elements
  uint32_t pre[M];
  uint32_t run = 0;
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t c = static_cast<uint32_t>(__popc((gmask >> (4 * m)) & 15u)) |
                       (static_cast<uint32_t>(__popc((emask >> (4 * m)) & 15u)) << 16);
    const uint32_t incl = wave_incl_scan(c);
    pre[m] = run + incl - c;
    run += lane63(incl);
  }
  if (lane == 0) wsum[wave] = run;
  __syncthreads();
  uint32_t woff = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t v = wsum[w];
    woff += w < wave ? v : 0u;
    tot += v;
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t ex = woff + pre[m];
    const int eq_before = base_eq + static_cast<int>(ex >> 16);
    const int gt_before = base_gt + static_cast<int>(ex & 0xffffu);
    const uint32_t g4 = (gmask >> (4 * m)) & 15u, e4 = (emask >> (4 * m)) & 15u;
    int take = need - eq_before;
    take = take < 0 ? 0 : min(take, __popc(e4));
    uint32_t keep = 0, rest = e4;
    for (int t = 0; t < take; ++t) {  // the lowest `take` equal elements
      keep |= rest & (0u - rest);
      rest &= rest - 1u;
    }
    const uint32_t pick = g4 | keep;
    if (pick) {
      int pos = gt_before + min(need, eq_before);
      const int p0 = tile_pos<ITEMS>(base, 4 * m);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((pick >> j) & 1u) {
          if (pos < k) out[pos] = p0 + j;
          ++pos;
        }
      }
    }
  }
  base_gt += static_cast<int>(tot & 0xffffu);
  base_eq += static_cast<int>(tot >> 16);
}

// Rows of n <= 1024 * ITEMS held in registers.
template <int ITEMS, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(const float* __restrict__ scores,
                                                                int n, int k, int ld_scores,
                                                                int32_t* __restrict__ idx,
                                                                int ld_idx) {
  static_assert(ITEMS % 4 == 0 && ITEMS <= 16, "items per thread");
  __shared__ TopkShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* s = scores + static_cast<size_t>(blockIdx.x) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(blockIdx.x) * ld_idx;
  if (k > n) k = n;
  if (k <= 0) return;
  if (k == n) {
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }

  float x[ITEMS];
  const uint32_t valid = load_tile<ITEMS, VEC>(s, 0, n, x);

  // 1. min / max (padding is -inf: it never lowers the max; the min skips it)
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    mx = fmaxf(mx, x[e]);
    mn = fminf(mn, ((valid >> e) & 1u) ? x[e] : INFINITY);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { sh.red_min[wave] = mn; sh.red_max[wave] = mx; }
  for (int i = tid; i < kHistWords; i += kTopkThreads) sh.hist[i] = 0;
  if (tid == 0) { sh.cnt = 0; sh.bin = 0; sh.above = 0; sh.need = 1; sh.tau = 0u; }
  __syncthreads();
  mn = sh.red_min[0];
  mx = sh.red_max[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) { mn = fminf(mn, sh.red_min[w]); mx = fmaxf(mx, sh.red_max[w]); }
  float bscale = static_cast<float>(kBins) / (mx - mn);
  if (!(bscale < INFINITY)) bscale = 0.f;  // degenerate range: one bin
  const float boff = -mn * bscale;

  // 2. histogram; bins kept packed two per register (padding lands in bin 0
  //    and is counted there, harmlessly: k < n)
  uint32_t bins[ITEMS / 2];
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    int b = static_cast<int>(__builtin_fmaf(x[e], bscale, boff));
    b = max(0, min(b, kBins - 1));
    atomicAdd(&sh.hist[hpad(b)], 1);
    if (e & 1) bins[e >> 1] |= static_cast<uint32_t>(b) << 16;
    else bins[e >> 1] = static_cast<uint32_t>(b);
  }
  __syncthreads();
  block_crossing(sh.hist[hpad(2 * tid)], sh.hist[hpad(2 * tid + 1)], k, sh.wtot, &sh.bin, &sh.above,
                 &sh.nbin);
  const uint32_t B = static_cast<uint32_t>(min(max(sh.bin, 0), kBins - 1));
  const int need0 = k - sh.above;

  // 3. boundary-bin elements -> LDS list
  uint32_t cmask = 0;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    const uint32_t b = (bins[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    cmask |= static_cast<uint32_t>(b == B) << e;
  }
  cmask &= valid;
  {
    const int cnt = __popc(cmask);
    const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(cnt)));
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&sh.cnt, incl);
    base = static_cast<int>(lane63(static_cast<uint32_t>(base))) + incl - cnt;
    if (cmask) {
#pragma unroll
      for (int e = 0; e < ITEMS; ++e) {
        if ((cmask >> e) & 1u) {
          if (base < kCand) sh.cand[base] = fkey(x[e]);
          ++base;
        }
      }
    }
  }
  __syncthreads();

  // 4. exact threshold
  exact_threshold(sh, need0, [&](auto f) {
#pragma unroll
    for (int e = 0; e < ITEMS; ++e)
      if ((cmask >> e) & 1u) f(x[e]);
  });
  const float tau = key_to_float(sh.tau);
  const int need = sh.need;

  // 5. compaction in index order
  uint32_t gmask = 0, emask = 0;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    gmask |= static_cast<uint32_t>(x[e] > tau) << e;
    emask |= static_cast<uint32_t>(x[e] == tau) << e;
  }
  int base_gt = 0, base_eq = 0;
  write_picks<ITEMS>(gmask, emask & valid, 0, need, k, out, sh.wsum, base_gt, base_eq);
}

// k >= n: every position, in order.
__global__ __launch_bounds__(256) void topk_all_kernel(int n, int32_t* __restrict__ idx, int ld_idx) {
  int32_t* out = idx + static_cast<size_t>(blockIdx.y) * ld_idx;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) out[i] = i;
}

// ---------------------------------------------------------------------------
// Split path, for rows that are few or long: one row is spread over `slices`
// workgroups of 1024 threads, each owning a tile of 1024 * IPT elements.  It
// starts from the row's histogram over the level-1 bins (l1_bin): one per
// row, filled by the scoring pass, or one per tile, written by
// topk_tilehist_kernel just before (then summed).
//   topk_cand_kernel, per tile: the boundary bin B of the row (where the k-th
//     largest key lies) and the keys above it, from the histogram; writes the
//     tile's keys of bin B with their positions (a few dozen at the cosine
//     workloads' sizes), its count of bin-B keys and of keys above bin B;
//   topk_pick_kernel, per tile: gathers the row's bin-B keys into LDS, finds
//     tau, the need-th largest of them (the row's k-th largest key): few keys
//     are ranked against the whole list, the work split over the block, more
//     take radix levels over bin B's key range; then counts the keys > tau and
//     == tau before its tile and writes its tile's picks.
// A workgroup never reads more of the row than its own tile: on this chip one
// CU pulls only some tens of GB/s from memory, so a tile per CU and a small
// exchange through the workspace beat a full read of the row per workgroup.
// Workspace, for W = rows * slices tiles (split_ws below): the W tile
// histograms unless the scoring pass filled the row's, then per row (B, need,
// count of bin B), per tile (bin-B count, count above bin B), and per tile
// room for all of its keys as (key, position) pairs.  Nothing needs
// initialising.
// ---------------------------------------------------------------------------
constexpr int kSplitCand = 6144;  // bin-B keys kept in LDS
constexpr int kMaxSlices = 1024;  // tiles per row (8M scores at 8 per thread)
// bin-B slots per thread fetched before the counts are known: about four
// times the count a tile of cosine scores holds at the workloads' sizes
template <int IPT> constexpr int spec_per() { return IPT >= 8 ? 2 : 1; }

struct SplitWs {
  int4* info;    // per row: (B, need, count of bin B in the row, 0)
  int2* meta;    // per tile: (its bin-B count, its count above bin B)
  uint2* slots;  // per tile: its bin-B keys and positions, tile-size slots
};

// Per-tile level-1 histograms (part[w * kL1Bins + b] for tile w of row
// w / slices) when the scoring pass has not filled the rows'.
template <int IPT, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_tilehist_kernel(const float* __restrict__ scores,
                                                                     int n, int ld_scores, int slices,
                                                                     int* __restrict__ part) {
  __shared__ int h[kL1Bins];
  static_assert(kL1Bins == 2 * kTopkThreads, "two bins per thread");
  const int tid = threadIdx.x;
  const int w = blockIdx.x, row = w / slices, sl = w - row * slices;
  const float* s = scores + static_cast<size_t>(row) * ld_scores;
  for (int i = tid; i < kL1Bins; i += kTopkThreads) h[i] = 0;
  float x[IPT];
  const uint32_t valid = load_tile<IPT, VEC>(s, sl * kTopkThreads * IPT, n, x);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < IPT; ++e)
    if ((valid >> e) & 1u) atomicAdd(&h[l1_bin(fkey(x[e]))], 1);
  __syncthreads();
  *reinterpret_cast<int2*>(part + static_cast<size_t>(w) * kL1Bins + 2 * tid) =
      int2{h[2 * tid], h[2 * tid + 1]};
}

struct CandShared {
  uint32_t wtot[kTopkWaves];
  int red[kTopkWaves];
  int bin, above, nb;
};

// hist: `hists` level-1 histograms per row (row r's at hist + r * hists *
// kL1Bins) whose sum counts every score of the row once.
template <int IPT, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_cand_kernel(const float* __restrict__ scores,
                                                                 int n, int k, int ld_scores,
                                                                 int slices,
                                                                 const int* __restrict__ hist,
                                                                 int hists, SplitWs ws) {
  __shared__ CandShared sh;
  constexpr int kTile = kTopkThreads * IPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x, row = w / slices, sl = w - row * slices;
  const float* s = scores + static_cast<size_t>(row) * ld_scores;
  const int p0 = sl * kTile;  // first position of this workgroup's tile
  const int* hrow = hist + static_cast<size_t>(row) * hists * kL1Bins;

  // Its tile and the row's histograms are requested together (batches of 8
  // histograms, addresses clamped so that a batch is branch-free); thread t
  // sums bins 2t and 2t + 1.
  float x[IPT];
  const uint32_t valid = load_tile<IPT, VEC>(s, p0, n, x);
  constexpr int kBatch = 8;
  int total[2] = {0, 0};
  if (hists == 1) {  // uniform: the row's histogram from the scoring pass
    const int2 v = *reinterpret_cast<const int2*>(hrow + 2 * tid);
    total[0] = v.x;
    total[1] = v.y;
  } else {
    for (int h0 = 0; h0 < hists; h0 += kBatch) {
      int2 v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        v[i] = *reinterpret_cast<const int2*>(hrow + static_cast<size_t>(min(h0 + i, hists - 1)) * kL1Bins +
                                              2 * tid);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        total[0] += h0 + i < hists ? v[i].x : 0;
        total[1] += h0 + i < hists ? v[i].y : 0;
      }
    }
  }
  if (tid == 0) {  // defaults, overwritten below (ordered by the crossing's barriers)
    sh.bin = 0;
    sh.above = 0;
    sh.nb = 0;
  }
  block_crossing(total[0], total[1], k, sh.red, &sh.bin, &sh.above, &sh.nb);
  const int B = min(max(sh.bin, 0), kL1Bins - 1);
  uint32_t lo, hi;
  l1_bin_range(B, &lo, &hi);
  const uint32_t span = hi - lo;  // key x is in bin B iff x - lo <= span (unsigned)

  // the tile's bin-B keys, and its count above bin B
  uint32_t cm = 0;
  int above = 0;
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const uint32_t kx = fkey(x[e]);
    const bool v = (valid >> e) & 1u;
    cm |= static_cast<uint32_t>(v && kx - lo <= span) << e;
    above += (v && kx > hi) ? 1 : 0;
  }
  // packed (bin-B | above << 16) counts: a tile holds at most 8192 elements
  const uint32_t mine = static_cast<uint32_t>(__popc(cm)) | (static_cast<uint32_t>(above) << 16);
  const uint32_t incl = wave_incl_scan(mine);
  if (lane == 63) sh.wtot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int v = 0; v < kTopkWaves; ++v) {
    const uint32_t t = sh.wtot[v];
    tot += t;
    before += v < wave ? t : 0u;
  }
  int at = static_cast<int>((before + incl - mine) & 0xffffu);
  uint2* slot = ws.slots + static_cast<size_t>(w) * kTile;
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    if ((cm >> e) & 1u) {
      slot[at] = uint2{fkey(x[e]), static_cast<uint32_t>(tile_pos<IPT>(p0, e))};
      ++at;
    }
  }
  if (tid == 0) {
    ws.meta[w] = int2{static_cast<int>(tot & 0xffffu), static_cast<int>(tot >> 16)};
    if (sl == 0) ws.info[row] = int4{B, k - sh.above, sh.nb, 0};
  }
}

// Sum over the block of (a, b); every thread gets the totals.
__device__ __forceinline__ void block_sum2(int& a, int& b, int (*red)[kTopkWaves]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  a = static_cast<int>(lane63(wave_incl_scan(static_cast<uint32_t>(a))));
  b = static_cast<int>(lane63(wave_incl_scan(static_cast<uint32_t>(b))));
  if (lane == 0) { red[0][wave] = a; red[1][wave] = b; }
  __syncthreads();
  a = 0;
  b = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) { a += red[0][w]; b += red[1][w]; }
  __syncthreads();
}

struct PickShared {
  int hist2[hist_words(1 << 11)];  // radix levels over bin B's key range
  uint32_t ckey[kSplitCand];
  int cpos[kSplitCand];
  int seg[kMaxSlices];  // tile t's bin-B keys start at list position seg[t]
  int cnt[kMaxSlices];  // ... and are cnt[t]
  uint32_t wsum[kTopkWaves];
  int red[2][kTopkWaves];
  int bin, above;
};

template <int IPT, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_pick_kernel(const float* __restrict__ scores,
                                                                 int n, int k, int ld_scores,
                                                                 int slices, SplitWs ws,
                                                                 int32_t* __restrict__ idx,
                                                                 int ld_idx) {
  __shared__ PickShared sh;
  constexpr int kTile = kTopkThreads * IPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x, row = w / slices, sl = w - row * slices;
  const float* s = scores + static_cast<size_t>(row) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(row) * ld_idx;
  const int p0 = sl * kTile;
  const uint2* srow = ws.slots + static_cast<size_t>(row) * slices * kTile;

  // One trip to memory: the tile, the row's (B, need), every tile's counts,
  // and the first `cap` bin-B slots of every tile (before their counts are
  // known; clamped addresses keep the loads branch-free).
  // (B, need) through the vector path, issued first: as a scalar load (the
  // address is uniform) it would be issued late and waited on alone
  int row_v = row;
  asm volatile("" : "+v"(row_v));
  const int4 info = ws.info[row_v];
  float xo[IPT];
  const uint32_t vo = load_tile<IPT, VEC>(s, p0, n, xo);
  const int2 m = ws.meta[static_cast<size_t>(row) * slices + min(tid, slices - 1)];
  constexpr int kSpecPer = spec_per<IPT>();
  const int cap = max(1, kSpecPer * kTopkThreads / slices);
  uint2 sp[kSpecPer];
#pragma unroll
  for (int u = 0; u < kSpecPer; ++u) {
    const int r = tid + kTopkThreads * u;
    const int t = min(r / cap, slices - 1), j = min(r - (r / cap) * cap, kTile - 1);
    sp[u] = srow[static_cast<size_t>(t) * kTile + j];
  }

  // list offsets of the tiles (a block scan of their counts), the count
  // above bin B before this tile, and whether any tile holds more than `cap`
  const int cx = tid < slices ? m.x : 0;
  const int ax = tid < sl ? m.y : 0;
  const int ox = cx > cap ? 1 : 0;
  const uint32_t incl = wave_incl_scan(static_cast<uint32_t>(cx));
  const int aw = static_cast<int>(lane63(wave_incl_scan(static_cast<uint32_t>(ax))));
  const int ow = static_cast<int>(lane63(wave_incl_scan(static_cast<uint32_t>(ox))));
  if (lane == 63) {
    sh.red[0][wave] = static_cast<int>(incl);
    sh.red[1][wave] = aw | (ow << 24);  // above_before < 2^24: rows hold at most 8M scores
  }
  __syncthreads();
  int before = 0, nb = 0, above_before = 0, over = 0;
#pragma unroll
  for (int v = 0; v < kTopkWaves; ++v) {
    const int c = sh.red[0][v];
    nb += c;
    before += v < wave ? c : 0;
    above_before += sh.red[1][v] & 0xffffff;
    over += sh.red[1][v] >> 24;
  }
  if (tid < slices) {
    sh.seg[tid] = before + static_cast<int>(incl) - cx;
    sh.cnt[tid] = cx;
  }
  __syncthreads();
  const bool in_lds = nb <= kSplitCand;
  const int ncand = in_lds ? nb : 0;
  if (in_lds) {
#pragma unroll
    for (int u = 0; u < kSpecPer; ++u) {
      const int r = tid + kTopkThreads * u, t = r / cap, j = r - t * cap;
      if (t < slices && j < sh.cnt[t]) {
        const int at = sh.seg[t] + j;
        sh.ckey[at] = sp[u].x;
        sh.cpos[at] = static_cast<int>(sp[u].y);
      }
    }
    if (over) {  // uniform: tiles with more than `cap` bin-B keys
      for (int t = 0; t < slices; ++t) {
        for (int j = cap + tid; j < sh.cnt[t]; j += kTopkThreads) {
          const uint2 c = srow[static_cast<size_t>(t) * kTile + j];
          sh.ckey[sh.seg[t] + j] = c.x;
          sh.cpos[sh.seg[t] + j] = static_cast<int>(c.y);
        }
      }
    }
  }
  __syncthreads();

  // f(key, position) for every key of bin B (from the list, or the slots)
  auto visit = [&](auto f) __attribute__((always_inline)) {
    if (in_lds) {
      for (int i = tid; i < ncand; i += kTopkThreads) f(sh.ckey[i], sh.cpos[i]);
    } else {
      for (int t = 0; t < slices; ++t) {
        const int c = sh.cnt[t];
        for (int j = tid; j < c; j += kTopkThreads) {
          const uint2 p = srow[static_cast<size_t>(t) * kTile + j];
          f(p.x, static_cast<int>(p.y));
        }
      }
    }
  };

  // tau, and the copies of it still to take: radix levels over [base, base +
  // width], the keys of bin B, until one key is left -- 9-bit digits over
  // the LDS list (a small crossing per level; a bin's 2^17 keys take two
  // levels), 11-bit digits when every visit re-reads the slots.  (Measured
  // on a list of about 200 keys, the block-wide levels beat both a pairwise
  // ranking and levels run by one wave.)
  int need = info.y;
  uint32_t base, hi;
  l1_bin_range(min(max(info.x, 0), kL1Bins - 1), &base, &hi);
  uint32_t width = hi - base;
  auto levels = [&](auto dig) __attribute__((always_inline)) {
    constexpr int DIG = decltype(dig)::value, NBIN = 1 << DIG;
    while (width > 0) {  // uniform
      const int shift = max(0, 32 - DIG - __clz(static_cast<int>(width)));  // width >> shift < NBIN
      for (int i = tid; i < hist_words(NBIN); i += kTopkThreads) sh.hist2[i] = 0;
      if (tid == 0) {  // (kept should no bin hold the crossing: the counts are exact)
        sh.bin = 0;
        sh.above = 0;
      }
      __syncthreads();
      visit([&](uint32_t kx, int) {
        const uint32_t dx = kx - base;
        if (kx >= base && dx <= width) atomicAdd(&sh.hist2[hpad(static_cast<int>(dx >> shift))], 1);
      });
      __syncthreads();
      if (wave == 0) wave_crossing<NBIN / 64>(sh.hist2, need, &sh.bin, &sh.above);
      __syncthreads();
      need -= sh.above;
      const uint32_t dg = static_cast<uint32_t>(min(max(sh.bin, 0), NBIN - 1)) << shift;
      base += dg;
      width = min(width - dg, (1u << shift) - 1u);
      // bin / above are rewritten two barriers later, after every read
    }
  };
  if (in_lds) levels(std::integral_constant<int, 9>{});
  else levels(std::integral_constant<int, 11>{});
  const uint32_t tau = base;
  // `need` copies of tau are taken (lowest positions first)

  // what precedes this tile: greater keys and copies of tau
  int gt_before = 0, eq_before = 0;
  visit([&](uint32_t kx, int pos) {
    if (pos < p0) {
      gt_before += kx > tau;
      eq_before += kx == tau;
    }
  });
  block_sum2(gt_before, eq_before, sh.red);
  gt_before += above_before;

  // this tile's picks, in position order
  uint32_t gmask = 0, emask = 0;
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const uint32_t kx = fkey(xo[e]);
    gmask |= static_cast<uint32_t>(kx > tau) << e;
    emask |= static_cast<uint32_t>(kx == tau) << e;
  }
  write_picks<IPT>(gmask & vo, emask & vo, p0, need, k, out, sh.wsum, gt_before, eq_before);
}

// Tile elements per thread of the split path for rows of n scores.
int split_items(int n) { return n <= 65536 ? 4 : 8; }
int split_slices(int n) {
  const int tile = kTopkThreads * split_items(n);
  return (n + tile - 1) / tile;
}
// The split path serves rows longer than 16K scores, and rows of more than 4K
// when they are too few to fill the chip one per CU.
bool split_shape(int rows, int n) {
  return n > 16 * kTopkThreads || (n > 4 * kTopkThreads && rows < 128);
}

// The split path's workspace for `rows` rows of n scores: the tile histograms
// (unless the scoring pass fills one per row, row_hist; those then come
// first, rows * kL1Bins ints), then the SplitWs arrays, each 16-byte aligned.
struct SplitLayout {
  size_t hist, info, meta, slots, total;
};
SplitLayout split_layout(int rows, int n, bool row_hist) {
  auto up = [](size_t x) { return (x + 15) & ~static_cast<size_t>(15); };
  const size_t tiles = static_cast<size_t>(rows) * split_slices(n);
  SplitLayout l;
  l.hist = 0;
  l.info = up((row_hist ? static_cast<size_t>(rows) : tiles) * kL1Bins * sizeof(int));
  l.meta = l.info + up(static_cast<size_t>(rows) * sizeof(int4));
  l.slots = l.meta + up(tiles * sizeof(int2));
  l.total = l.slots + tiles * kTopkThreads * split_items(n) * sizeof(uint2);
  return l;
}

}  // namespace

size_t topk_workspace_bytes(int rows, int n, bool row_hist) {
  if (rows <= 0 || n <= 0 || !split_shape(rows, n)) return 0;
  return split_layout(rows, n, row_hist).total;
}

int topk_max_row() { return kMaxSlices * kTopkThreads * 8; }

bool topk_uses_row_hist(int rows, int n, int k) { return k < n && split_shape(rows, n); }

namespace {

template <int IPT, bool VEC>
void launch_split(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                  int ld_idx, char* ws, bool row_hist, hipStream_t st) {
  const int slices = split_slices(n);
  const dim3 grid(rows * slices), block(kTopkThreads);
  const SplitLayout l = split_layout(rows, n, row_hist);
  int* hist = reinterpret_cast<int*>(ws + l.hist);
  SplitWs sw;
  sw.info = reinterpret_cast<int4*>(ws + l.info);
  sw.meta = reinterpret_cast<int2*>(ws + l.meta);
  sw.slots = reinterpret_cast<uint2*>(ws + l.slots);
  if (!row_hist)
    hipLaunchKernelGGL((topk_tilehist_kernel<IPT, VEC>), grid, block, 0, st, scores, n, ld_scores, slices, hist);
  hipLaunchKernelGGL((topk_cand_kernel<IPT, VEC>), grid, block, 0, st, scores, n, k, ld_scores, slices,
                     hist, row_hist ? 1 : slices, sw);
  hipLaunchKernelGGL((topk_pick_kernel<IPT, VEC>), grid, block, 0, st, scores, n, k, ld_scores, slices,
                     sw, idx, ld_idx);
}

template <bool VEC>
void launch_rows(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                 int ld_idx, void* ws, bool row_hist, hipStream_t st) {
  const dim3 block(kTopkThreads);
  if (k < n && split_shape(rows, n)) {
    char* w = static_cast<char*>(ws);
    if (split_items(n) == 4) launch_split<4, VEC>(rows, n, k, scores, ld_scores, idx, ld_idx, w, row_hist, st);
    else launch_split<8, VEC>(rows, n, k, scores, ld_scores, idx, ld_idx, w, row_hist, st);
    return;
  }
  const dim3 grid(rows);
  if (n <= 4 * kTopkThreads)
    hipLaunchKernelGGL((topk_reg_kernel<4, VEC>), grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else if (n <= 8 * kTopkThreads)
    hipLaunchKernelGGL((topk_reg_kernel<8, VEC>), grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else if (n <= 16 * kTopkThreads)
    hipLaunchKernelGGL((topk_reg_kernel<16, VEC>), grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else  // k >= n
    hipLaunchKernelGGL(topk_all_kernel, dim3(min((n + 255) / 256, 64), rows), dim3(256), 0, st, n, idx,
                       ld_idx);
}

}  // namespace

hipError_t launch_topk(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                       int ld_idx, void* ws, bool row_hist, hipStream_t st) {
  if (rows == 0 || n == 0) return hipSuccess;
  // 16-byte loads need aligned rows and whole groups of four
  const bool vec = (ld_scores % 4 == 0) && (n % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  if (vec) launch_rows<true>(rows, n, k, scores, ld_scores, idx, ld_idx, ws, row_hist, st);
  else launch_rows<false>(rows, n, k, scores, ld_scores, idx, ld_idx, ws, row_hist, st);
  return hipGetLastError();
}

}  // namespace qk
