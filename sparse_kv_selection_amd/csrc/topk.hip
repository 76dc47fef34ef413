// Per-row top-k of fp32 scores, indices returned in ascending order.
//
// QUOKA write-up, section 2.3 listing: the BSA keys with the largest
// aggregated score per KV head.  Ties go to the lower position and -0.0
// equals +0.0, so the selected set is unique.
//
// One workgroup of 1024 threads per row; every thread owns contiguous runs of
// the row (so the index-order compaction needs one prefix sum per run):
//   1. min / max of the row;
//   2. histogram over 2048 equal-width value bins between min and max -- the
//      binning is monotone in the value, so every bin above the one holding
//      the k-th largest value is selected whole;
//   3. an exact 8-bit radix select over the order-preserving 32-bit keys of
//      that boundary bin's elements gives the threshold key and how many
//      elements equal to it are still needed;
//   4. compaction in index order: every element above the threshold, plus the
//      first `need` elements equal to it.
// Rows of up to 16K scores are read once into registers; longer rows are
// streamed in runs of 16 per thread with all loads of a run in flight (after
// the first pass the row is served from L2).
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kRun = 16;  // elements per thread per streamed run

// Order-preserving map of a float to uint32 (-0.0 maps like +0.0).
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive prefix sum over 1024 threads; *total gets the sum.
__device__ int block_excl_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kTopkWaves ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < kTopkWaves; o <<= 1) {
      const int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kTopkWaves) wsum[lane] = w;
  }
  __syncthreads();
  const int off = wave > 0 ? wsum[wave - 1] : 0;
  *total = wsum[kTopkWaves - 1];
  __syncthreads();
  return off + x - v;
}

// Given counts h[0..nb) (nb <= 2048) and 1 <= need <= sum(h), find the bin b
// with count(bins > b) < need <= count(bins >= b); writes (*bin, *above).
__device__ void find_crossing(const int* h, int nb, int need, int* wsum, int* bin, int* above) {
  const int t = threadIdx.x;
  const int b0 = nb - 1 - 2 * t, b1 = b0 - 1;
  const int h0 = b0 >= 0 ? h[b0] : 0, h1 = b1 >= 0 ? h[b1] : 0;
  int tot;
  const int ex = block_excl_scan(h0 + h1, wsum, &tot);
  if (b0 >= 0 && ex < need && need <= ex + h0) { *bin = b0; *above = ex; }
  if (b1 >= 0 && ex + h0 < need && need <= ex + h0 + h1) { *bin = b1; *above = ex + h0; }
  __syncthreads();
}

constexpr int kCand = 4096;  // boundary-bin candidates kept in LDS

struct TopkShared {
  int hist[kBins];
  uint32_t cand[kCand];
  int wsum[kTopkWaves];
  float red_min[kTopkWaves], red_max[kTopkWaves];
  int bin, above, cnt;
};

// Load `N` consecutive scores starting at i0 (-inf past the end).
template <int N>
__device__ __forceinline__ void load_run(const float* s, int n, int i0, bool vec, float* x) {
  if (vec && i0 + N <= n) {
#pragma unroll
    for (int m = 0; m < N / 4; ++m) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s + i0 + 4 * m);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * m + e] = v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < N; ++e) x[e] = (i0 + e < n) ? s[i0 + e] : -INFINITY;
  }
}

// Wave 0 finds the bin b of counts h[0..nb) (nb a multiple of 64) with
// count(bins > b) < need <= count(bins >= b); writes (*bin, *above).  Lane l
// owns the nb/64 bins counted downward from nb - 1 - l * nb/64.
__device__ void wave_crossing(const int* h, int nb, int need, int* bin, int* above) {
  const int lane = threadIdx.x & 63;
  const int per = nb / 64;
  const int top = nb - 1 - lane * per;
  int sum = 0;
  for (int q = 0; q < per; ++q) sum += h[top - q];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  int ex = incl - sum;  // count of bins above this lane's range
  if (ex < need && need <= incl) {
    for (int q = 0; q < per; ++q) {
      const int c = h[top - q];
      if (need <= ex + c) {
        *bin = top - q;
        *above = ex;
        break;
      }
      ex += c;
    }
  }
}

// Shared selection logic.  `visit(f)` calls f(value, index) for every slot of
// the row owned by this thread, including the -inf padding past the end
// (index >= n); `runs(g)` calls g(x, i0) for each owned run of RUN slots, in
// increasing run order (runs with the same number are consecutive in the row
// and ordered by thread id).  Padding is the smallest key: it may be counted
// in a histogram but is never selected, because k <= n.
template <int RUN, typename Visit, typename Runs>
__device__ void select_row(TopkShared& sh, int n, int k, int32_t* out, Visit visit, Runs runs) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // 1. min / max over the real elements
  float mn = INFINITY, mx = -INFINITY;
  visit([&](float x, int i) {
    mn = fminf(mn, i < n ? x : INFINITY);
    mx = fmaxf(mx, x);
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { sh.red_min[wave] = mn; sh.red_max[wave] = mx; }
  for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
  if (tid == 0) { sh.cnt = 0; sh.bin = 0; sh.above = 0; }
  __syncthreads();
  mn = sh.red_min[0];
  mx = sh.red_max[0];
  for (int w = 1; w < kTopkWaves; ++w) { mn = fminf(mn, sh.red_min[w]); mx = fmaxf(mx, sh.red_max[w]); }
  // equal-width bins between mn and mx (monotone in the value); a degenerate
  // range puts everything in bin 0 and leaves the decision to the exact stage
  float bscale = static_cast<float>(kBins) / (mx - mn);
  if (!(bscale < INFINITY)) bscale = 0.f;
  auto bin_of = [&](float x) {
    const int b = static_cast<int>((x - mn) * bscale);
    return max(0, min(b, kBins - 1));
  };

  // 2. value-bin histogram; wave 0 finds the boundary bin
  visit([&](float x, int) { atomicAdd(&sh.hist[bin_of(x)], 1); });
  __syncthreads();
  if (wave == 0) wave_crossing(sh.hist, kBins, k, &sh.bin, &sh.above);
  __syncthreads();
  const int B = min(max(sh.bin, 0), kBins - 1);
  int need = k - sh.above;  // elements still to take from bin B, >= 1

  // 3. compact the boundary bin's real elements into LDS (wave ballots)
  visit([&](float x, int i) {
    const bool c = (i < n) & (bin_of(x) == B);
    const unsigned long long bal = __ballot(c);
    if (bal == 0ull) return;
    const int before = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(bal >> 32),
                                                 __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(bal), 0));
    int base = 0;
    if (lane == 0) base = atomicAdd(&sh.cnt, __popcll(bal));
    base = __shfl(base, 0);
    const int slot = base + before;
    if (c && slot < kCand) sh.cand[slot] = fkey(x);
  });
  __syncthreads();
  const int ncand = sh.cnt;

  // 4. exact threshold key tau: the need-th largest candidate key.  Up to one
  //    candidate per thread: rank each against all; else 8-bit radix passes.
  uint32_t tau;
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
        sh.bin = static_cast<int>(mine);
        sh.above = gt;
      }
    }
    __syncthreads();
    tau = static_cast<uint32_t>(sh.bin);
    need -= sh.above;
  } else {
    const bool in_lds = ncand <= kCand;
    uint32_t prefix = 0, pmask = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < 256; i += kTopkThreads) sh.hist[i] = 0;
      __syncthreads();
      if (in_lds) {
        for (int c = tid; c < ncand; c += kTopkThreads) {
          const uint32_t kx = sh.cand[c];
          if ((kx & pmask) == prefix) atomicAdd(&sh.hist[(kx >> shift) & 255u], 1);
        }
      } else {
        visit([&](float x, int i) {
          if (i >= n || bin_of(x) != B) return;
          const uint32_t kx = fkey(x);
          if ((kx & pmask) == prefix) atomicAdd(&sh.hist[(kx >> shift) & 255u], 1);
        });
      }
      __syncthreads();
      if (wave == 0) wave_crossing(sh.hist, 256, need, &sh.bin, &sh.above);
      __syncthreads();
      need -= sh.above;
      prefix |= static_cast<uint32_t>(min(max(sh.bin, 0), 255)) << shift;
      pmask |= 0xffu << shift;
      __syncthreads();
    }
    tau = prefix;
  }

  // 5. compaction in index order.  One scan of packed (greater, equal) counts
  //    per run: the output position of a thread's first pick is
  //    GT_before + min(need, EQ_before).
  int base_gt = 0, base_eq = 0;
  runs([&](const float* x, int i0) {
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < RUN; ++e) {
      const uint32_t kx = fkey(x[e]);
      gt += kx > tau;
      eq += kx == tau;
    }
    int tot;
    const int ex = block_excl_scan(gt | (eq << 16), sh.wsum, &tot);
    const int gt_before = base_gt + (ex & 0xffff), eq_before = base_eq + (ex >> 16);
    int take = need - eq_before;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    if (gt + take > 0) {
      int pos = gt_before + min(need, eq_before);
      int eq_seen = 0;
#pragma unroll
      for (int e = 0; e < RUN; ++e) {
        const uint32_t kx = fkey(x[e]);
        bool pick = kx > tau;
        if (kx == tau) {
          pick = eq_seen < take;
          ++eq_seen;
        }
        if (pick) {
          if (pos < k) out[pos] = i0 + e;
          ++pos;
        }
      }
    }
    base_gt += tot & 0xffff;
    base_eq += tot >> 16;
  });
}

// Rows of n <= 1024 * ITEMS: thread t owns [t * ITEMS, (t + 1) * ITEMS) in registers.
template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(const float* __restrict__ scores,
                                                                int n, int k, int ld_scores,
                                                                int32_t* __restrict__ idx,
                                                                int ld_idx) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const float* s = scores + static_cast<size_t>(blockIdx.x) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(blockIdx.x) * ld_idx;
  if (k > n) k = n;
  if (k <= 0) return;
  if (k == n) {
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }
  const bool vec = ((ld_scores & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  const int i0 = tid * ITEMS;
  float x[ITEMS];
  load_run<ITEMS>(s, n, i0, vec, x);
  select_row<ITEMS>(
      sh, n, k, out,
      [&](auto f) {
#pragma unroll
        for (int e = 0; e < ITEMS; ++e) f(x[e], i0 + e);
      },
      [&](auto g) { g(x, i0); });
}

// Longer rows: runs of kRun elements per thread, super-tile r covering
// [r * 1024 * kRun, (r + 1) * 1024 * kRun), re-read from L2 for every pass.
__global__ __launch_bounds__(kTopkThreads) void topk_stream_kernel(const float* __restrict__ scores,
                                                                   int n, int k, int ld_scores,
                                                                   int32_t* __restrict__ idx,
                                                                   int ld_idx) {
  __shared__ TopkShared sh;
  const int tid = threadIdx.x;
  const float* s = scores + static_cast<size_t>(blockIdx.x) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(blockIdx.x) * ld_idx;
  if (k > n) k = n;
  if (k <= 0) return;
  if (k == n) {
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }
  const bool vec = ((ld_scores & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  constexpr int kSuper = kTopkThreads * kRun;
  auto runs = [&](auto g) {
    for (int base = 0; base < n; base += kSuper) {
      const int i0 = base + tid * kRun;
      float x[kRun];
      load_run<kRun>(s, n, i0, vec, x);
      g(x, i0);
    }
  };
  auto visit = [&](auto f) {
    runs([&](const float* x, int i0) {
#pragma unroll
      for (int e = 0; e < kRun; ++e) f(x[e], i0 + e);
    });
  };
  select_row<kRun>(sh, n, k, out, visit, runs);
}

}  // namespace

hipError_t launch_topk(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                       int ld_idx, hipStream_t st) {
  if (rows == 0 || n == 0) return hipSuccess;
  const dim3 grid(rows), block(kTopkThreads);
  if (n <= 4 * kTopkThreads)
    hipLaunchKernelGGL(topk_reg_kernel<4>, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else if (n <= 8 * kTopkThreads)
    hipLaunchKernelGGL(topk_reg_kernel<8>, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else if (n <= 16 * kTopkThreads)
    hipLaunchKernelGGL(topk_reg_kernel<16>, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else
    hipLaunchKernelGGL(topk_stream_kernel, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  return hipGetLastError();
}

}  // namespace qk
