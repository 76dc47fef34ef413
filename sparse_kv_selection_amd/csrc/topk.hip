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
// Split path for rows that are few or long: one row is spread over `slices`
// workgroups of 1024 threads, each owning a tile of 1024 * IPT elements.
//   pass 1 (topk_hist_kernel): each workgroup counting-sorts its tile by the
//     level-1 bin of the order-preserving key (l1_bin below): it writes the
//     tile's histogram, its exclusive prefix, and the tile's (key, position)
//     pairs grouped by bin (workspace; nothing needs initialising);
//   pass 2 (topk_split_kernel): each workgroup sums the row's histograms and
//     finds the boundary bin B, reads bin B's pairs from every tile's groups
//     into LDS, finds the k-th largest key among them (each ranked against
//     the others when they are few, else radix levels over their key range),
//     counts what earlier tiles contribute, and writes the positions picked
//     in its own tile.
// Workspace, for W = rows * slices workgroups: W histograms, W prefixes
// (2048 ints each), then W tiles of (key, position) pairs.
// ---------------------------------------------------------------------------
constexpr int kSplitCand = 6144;   // bin-B pairs kept in LDS
constexpr int kCandPerThread = kSplitCand / kTopkThreads;
constexpr int kRankDirect = 64;  // bin B ranked pair by pair up to this size

// Level-1 bin of an order key (2048 bins), monotone in the key so that every
// bin above the boundary bin is selected whole.  Each sign gets 1024 bins:
// 64 per binade of |x| over [2^-8, 2^(1022/64 - 8)) (about 0.0039 to 250:
// cosine scores and dot products of unit-scale vectors), one bin for the
// smaller magnitudes next to zero and one for the larger ones (and NaN) at the
// end.  The top bits of the key alone would spend most bins on exponents that
// such scores never reach and put a tenth of a row into one bin.
constexpr int kL1Shift = 17;         // key bits below a bin: 23 - 6 mantissa bits
constexpr int kFineBase = 119 << 6;  // (exponent, top 6 mantissa bits) of 2^-8
__device__ __forceinline__ int l1_bin(uint32_t key) {
  const bool pos = key >= 0x80000000u;
  const uint32_t mag = pos ? (key & 0x7fffffffu) : (0x7fffffffu - key);  // bits of |x|
  const int v = static_cast<int>(mag >> kL1Shift) - kFineBase;
  const int i = v < 0 ? 0 : min(v + 1, 1023);
  return pos ? 1024 + i : 1023 - i;
}
// The keys of level-1 bin b: [*lo, *hi].
__device__ __forceinline__ void l1_bin_range(int b, uint32_t* lo, uint32_t* hi) {
  const bool pos = b >= 1024;
  const int i = pos ? b - 1024 : 1023 - b;
  const uint32_t mlo = i == 0 ? 0u : static_cast<uint32_t>(kFineBase + i - 1) << kL1Shift;
  const uint32_t mhi =
      i == 1023 ? 0x7fffffffu : (static_cast<uint32_t>(kFineBase + i) << kL1Shift) - 1u;
  *lo = pos ? (0x80000000u | mlo) : (0x7fffffffu - mhi);
  *hi = pos ? (0x80000000u | mhi) : (0x7fffffffu - mlo);
}

template <int IPT, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_hist_kernel(const float* __restrict__ scores,
                                                                 int n, int ld_scores, int slices,
                                                                 int* __restrict__ part) {
  constexpr int kTile = kTopkThreads * IPT;
  __shared__ int h[kBins];
  __shared__ int wtot[kTopkWaves];
  __shared__ uint4 stage[kTile / 2];  // the tile's pairs in bin order, two per entry
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x, nwg = gridDim.x;
  const int row = w / slices, sl = w - row * slices;
  const float* s = scores + static_cast<size_t>(row) * ld_scores;
  for (int i = tid; i < kBins; i += kTopkThreads) h[i] = 0;
  float x[IPT];
  const uint32_t valid = load_tile<IPT, VEC>(s, sl * kTile, n, x);
  uint32_t kx[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) kx[e] = fkey(x[e]);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < IPT; ++e)
    if ((valid >> e) & 1u) atomicAdd(&h[l1_bin(kx[e])], 1);
  __syncthreads();
  // exclusive prefix over the bins; thread t owns bins 2t and 2t + 1
  const int c0 = h[2 * tid], c1 = h[2 * tid + 1];
  const int incl = static_cast<int>(wave_incl_scan(static_cast<uint32_t>(c0 + c1)));
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int v = 0; v < kTopkWaves; ++v) off += v < wave ? wtot[v] : 0;
  const int ex = off + incl - c0 - c1;
  h[2 * tid] = ex;  // now the bins' write cursors (each thread rewrites only its own bins)
  h[2 * tid + 1] = ex + c0;
  __syncthreads();
  // The pairs are sorted into LDS and then written out contiguously: with
  // scores spread over many bins, direct scattered 8-byte stores would each
  // touch a line of their own.
  uint2* lp = reinterpret_cast<uint2*>(stage);
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    if ((valid >> e) & 1u) {
      const int slot = atomicAdd(&h[l1_bin(kx[e])], 1);
      if (slot < kTile)  // always: the slots of a bin end where the next bin's begin
        lp[slot] = uint2{kx[e], static_cast<uint32_t>(tile_pos<IPT>(sl * kTile, e))};
    }
  }
  __syncthreads();
  uint4* pairs = reinterpret_cast<uint4*>(part + 2 * static_cast<size_t>(nwg) * kBins) +
                 static_cast<size_t>(w) * (kTile / 2);
  const int nvalid = min(kTile, n - sl * kTile);  // slots [0, nvalid) are filled
  for (int i = tid; 2 * i < nvalid; i += kTopkThreads) pairs[i] = stage[i];
  // the tile's histogram and prefix, stored after the last barrier (a store
  // before a barrier holds the barrier until it completes)
  *reinterpret_cast<int2*>(part + static_cast<size_t>(w) * kBins + 2 * tid) = int2{c0, c1};
  *reinterpret_cast<int2*>(part + (static_cast<size_t>(nwg) + w) * kBins + 2 * tid) = int2{ex, ex + c0};
}

constexpr int kMaxSlices = 1024;

struct SplitShared {
  int hist2[kHistWords];      // radix levels over bin B's key range
  alignas(16) uint32_t ckey[kSplitCand];
  int cpos[kSplitCand];
  int seg_start[kMaxSlices + 1];  // bin B's pairs of tile t: [seg_start[t], seg_start[t + 1])
  int seg_off[kMaxSlices];        // ... found at this offset in tile t's sorted pairs
  uint32_t wsum[kTopkWaves];
  int red[2][kTopkWaves];
  int bin[2], above[2], nb;
  uint32_t tau;
  int need;
};


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


template <int IPT, bool VEC>
__global__ __launch_bounds__(kTopkThreads) void topk_split_kernel(const float* __restrict__ scores,
                                                                  int n, int k, int ld_scores,
                                                                  int slices,
                                                                  const int* __restrict__ part,
                                                                  int32_t* __restrict__ idx,
                                                                  int ld_idx) {
  __shared__ SplitShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x / slices, sl = blockIdx.x - row * slices;
  const float* s = scores + static_cast<size_t>(row) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(row) * ld_idx;
  const int p0 = sl * kTopkThreads * IPT;  // first position of this workgroup's tile
  const int* prow = part + static_cast<size_t>(row) * slices * kBins;

  // Its own tile and the row's tile histograms are requested together
  // (batches of 8 tiles, addresses clamped so that a batch is branch-free).
  // Thread t sums bins 2t and 2t + 1 over the tiles (all, and those before
  // its own).
  float xo[IPT];
  const uint32_t vo = load_tile<IPT, VEC>(s, p0, n, xo);
  static_assert(kBins == 2 * kTopkThreads, "two bins per thread");
  constexpr int kBatch = 8;
  int total[2] = {0, 0}, before[2] = {0, 0};
  for (int s0 = 0; s0 < slices; s0 += kBatch) {
    int2 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      v[i] = *reinterpret_cast<const int2*>(prow + static_cast<size_t>(min(s0 + i, slices - 1)) * kBins +
                                            2 * tid);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int c0 = s0 + i < slices ? v[i].x : 0, c1 = s0 + i < slices ? v[i].y : 0;
      total[0] += c0;
      total[1] += c1;
      before[0] += s0 + i < sl ? c0 : 0;
      before[1] += s0 + i < sl ? c1 : 0;
    }
  }

  // 1. boundary bin B of the row; bins above it in earlier tiles
  block_crossing(total[0], total[1], k, sh.red[0], &sh.bin[0], &sh.above[0],
                 &sh.nb);
  const uint32_t B = static_cast<uint32_t>(min(max(sh.bin[0], 0), kBins - 1));
  int need = k - sh.above[0];
  const int nb = sh.nb;
  int above_before = 0, unused = 0;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    above_before += static_cast<uint32_t>(2 * tid + u) > B ? before[u] : 0;

  // 2. bin B's pairs of every tile -> LDS when they fit (else every visit
  //    below reads them from the workspace)
  if (tid < slices) {
    const size_t t = static_cast<size_t>(row) * slices + tid;
    sh.seg_start[tid + 1] = part[t * kBins + B];
    sh.seg_off[tid] = part[(static_cast<size_t>(gridDim.x) + t) * kBins + B];
  }
  __syncthreads();
  if (wave == 0) {  // inclusive scan of the tiles' counts
    int carry = 0;
    for (int t0 = 0; t0 < slices; t0 += 64) {
      const int c = static_cast<int>(
          wave_incl_scan(static_cast<uint32_t>(t0 + lane < slices ? sh.seg_start[t0 + lane + 1] : 0)));
      if (t0 + lane < slices) sh.seg_start[t0 + lane + 1] = carry + c;
      carry += static_cast<int>(lane63(static_cast<uint32_t>(c)));
    }
    if (lane == 0) sh.seg_start[0] = 0;
  }
  __syncthreads();
  const uint2* pairs = reinterpret_cast<const uint2*>(part + 2 * static_cast<size_t>(gridDim.x) * kBins);
  constexpr int kTile = kTopkThreads * IPT;
  auto fetch = [&](int i) {  // the i-th pair of bin B, 0 <= i < nb
    int lo = 0, hi = slices - 1;  // the tile t with seg_start[t] <= i < seg_start[t + 1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.seg_start[mid] <= i) lo = mid;
      else hi = mid - 1;
    }
    const int at = min(max(sh.seg_off[lo] + (i - sh.seg_start[lo]), 0), kTile - 1);
    return pairs[(static_cast<size_t>(row) * slices + lo) * kTile + at];
  };
  const bool in_lds = nb <= kSplitCand;
  if (in_lds) {
    uint2 c[kCandPerThread];
#pragma unroll
    for (int r = 0; r < kCandPerThread; ++r) c[r] = fetch(min(tid + kTopkThreads * r, nb - 1));
#pragma unroll
    for (int r = 0; r < kCandPerThread; ++r) {
      const int i = tid + kTopkThreads * r;
      if (i < nb) {
        sh.ckey[i] = c[r].x;
        sh.cpos[i] = static_cast<int>(c[r].y);
      }
    }
  }
  block_sum2(above_before, unused, sh.red);  // also orders the LDS list before its reads
  auto visit = [&](auto f) {  // f(key, position) for every element of bin B
    if (in_lds) {
      for (int i = tid; i < nb; i += kTopkThreads) f(sh.ckey[i], sh.cpos[i]);
    } else {
      for (int i = tid; i < nb; i += kTopkThreads) {
        const uint2 c = fetch(i);
        f(c.x, static_cast<int>(c.y));
      }
    }
  };

  // 3. the k-th largest key tau of the row, the need-th largest of bin B
  uint32_t tau;
  if (in_lds && nb <= kRankDirect) {
    // few: each candidate counts the greater and equal keys among the others
    if (tid < nb) {
      const uint32_t mine = sh.ckey[tid];
      int gt = 0, eq = 0;
      for (int c = 0; c < nb; ++c) {
        const uint32_t o = sh.ckey[c];
        gt += o > mine;
        eq += o == mine;
      }
      if (gt < need && need <= gt + eq) {  // every holder of this key agrees
        sh.tau = mine;
        sh.need = need - gt;
      }
    }
    __syncthreads();
    tau = sh.tau;
    need = sh.need;
  } else {
    // radix levels over [lo, lo + span], the keys of bin B, until one key is
    // left: 9-bit digits over the LDS list (a small crossing per level; a fine
    // bin's 2^17 keys take two levels), 11-bit digits when every visit
    // re-reads the workspace
    uint32_t lo, hi;
    l1_bin_range(static_cast<int>(B), &lo, &hi);
    uint32_t span = hi - lo;
    auto levels = [&](auto dig) {
      constexpr int DIG = decltype(dig)::value, NBIN = 1 << DIG;
      while (span > 0) {  // uniform
        const int shift = max(0, 32 - DIG - __clz(static_cast<int>(span)));  // span >> shift < NBIN
        for (int i = tid; i < hist_words(NBIN); i += kTopkThreads) sh.hist2[i] = 0;
        __syncthreads();
        visit([&](uint32_t kx, int) {
          const uint32_t dx = kx - lo;
          if (kx >= lo && dx <= span) atomicAdd(&sh.hist2[hpad(static_cast<int>(dx >> shift))], 1);
        });
        __syncthreads();
        if (wave == 0) wave_crossing<NBIN / 64>(sh.hist2, need, &sh.bin[1], &sh.above[1]);
        __syncthreads();
        need -= sh.above[1];
        const uint32_t dg = static_cast<uint32_t>(min(max(sh.bin[1], 0), NBIN - 1)) << shift;
        lo += dg;
        span = min(span - dg, (1u << shift) - 1u);
        // bin / above are rewritten two barriers later, after every read
      }
    };
    if (in_lds) levels(std::integral_constant<int, 9>{});
    else levels(std::integral_constant<int, 11>{});
    tau = lo;
  }
  // `need` copies of tau are taken (lowest positions first)

  // 4. what earlier tiles contribute: greater keys and copies of tau
  int gt_before = 0, eq_before = 0;
  visit([&](uint32_t kx, int pos) {
    if (pos < p0) {
      gt_before += kx > tau;
      eq_before += kx == tau;
    }
  });
  block_sum2(gt_before, eq_before, sh.red);
  gt_before += above_before;

  // 5. this tile's picks, in position order
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

}  // namespace

size_t topk_workspace_bytes(int rows, int n) {
  if (rows <= 0 || n <= 0 || !split_shape(rows, n)) return 0;
  const size_t tiles = static_cast<size_t>(rows) * split_slices(n);
  return tiles * (2 * kBins * sizeof(int) + kTopkThreads * split_items(n) * sizeof(uint2));
}

int topk_max_row() { return kMaxSlices * kTopkThreads * 8; }

template <bool VEC>
void launch_rows(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                 int ld_idx, void* ws, hipStream_t st) {
  const dim3 block(kTopkThreads);
  if (k < n && split_shape(rows, n)) {
    const int slices = split_slices(n);
    const dim3 grid(rows * slices);
    int* part = static_cast<int*>(ws);
    if (split_items(n) == 4) {
      hipLaunchKernelGGL((topk_hist_kernel<4, VEC>), grid, block, 0, st, scores, n, ld_scores, slices, part);
      hipLaunchKernelGGL((topk_split_kernel<4, VEC>), grid, block, 0, st, scores, n, k, ld_scores, slices, part, idx, ld_idx);
    } else {
      hipLaunchKernelGGL((topk_hist_kernel<8, VEC>), grid, block, 0, st, scores, n, ld_scores, slices, part);
      hipLaunchKernelGGL((topk_split_kernel<8, VEC>), grid, block, 0, st, scores, n, k, ld_scores, slices, part, idx, ld_idx);
    }
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

hipError_t launch_topk(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                       int ld_idx, void* ws, hipStream_t st) {
  if (rows == 0 || n == 0) return hipSuccess;
  // 16-byte loads need aligned rows and whole groups of four
  const bool vec = (ld_scores % 4 == 0) && (n % 4 == 0) &&
                   (reinterpret_cast<uintptr_t>(scores) % 16 == 0);
  if (vec) launch_rows<true>(rows, n, k, scores, ld_scores, idx, ld_idx, ws, st);
  else launch_rows<false>(rows, n, k, scores, ld_scores, idx, ld_idx, ws, st);
  return hipGetLastError();
}

}  // namespace qk
