// Per-row top-k of fp32 scores, indices returned in ascending order.
//
// QUOKA write-up, section 2.3 listing: the BSA keys with the largest
// aggregated score per KV head.  Ties go to the lower position and -0.0
// equals +0.0, so the selected set is unique.
//
// One workgroup of 1024 threads per row; the row stays in L2 between passes:
//   1. min / max of the row;
//   2. histogram over 2048 equal-width value bins between min and max (the
//      binning is monotone in the value, so every bin above the one that holds
//      the k-th largest value is selected whole);
//   3. the elements of that boundary bin are collected in LDS and an exact
//      8-bit radix select over their order-preserving 32-bit keys finds the
//      threshold key and how many elements equal to it are still needed (if
//      the bin holds more than the LDS capacity, the same radix select runs
//      over the row in global memory instead);
//   4. compaction in index order with block-wide prefix sums: every element
//      above the threshold, plus the first `need` elements equal to it.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kCand = 4096;

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

// Given counts h[0..nb) (nb <= 2 * 1024) and need >= 1, find the bin b with
// count(bins > b) < need <= count(bins >= b).  Writes (*bin, *above).
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

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int n, int k, int ld_scores,
                                                            int32_t* __restrict__ idx,
                                                            int ld_idx) {
  __shared__ int hist[kBins];
  __shared__ uint32_t ckey[kCand];
  __shared__ int wsum[kTopkWaves];
  __shared__ float red_min[kTopkWaves], red_max[kTopkWaves];
  __shared__ int s_bin, s_above, s_cnt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) { s_bin = 0; s_above = 0; }
  const float* s = scores + static_cast<size_t>(blockIdx.x) * ld_scores;
  int32_t* out = idx + static_cast<size_t>(blockIdx.x) * ld_idx;
  if (k > n) k = n;
  if (k <= 0) return;
  if (k == n) {
    for (int i = tid; i < n; i += kTopkThreads) out[i] = i;
    return;
  }

  // 1. min / max
  float mn = INFINITY, mx = -INFINITY;
  for (int i = tid; i < n; i += kTopkThreads) {
    const float x = s[i];
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { red_min[wave] = mn; red_max[wave] = mx; }
  __syncthreads();
  mn = red_min[0];
  mx = red_max[0];
  for (int w = 1; w < kTopkWaves; ++w) { mn = fminf(mn, red_min[w]); mx = fmaxf(mx, red_max[w]); }

  // bin width: value bins between mn and mx; a degenerate range puts every
  // element in bin 0 and leaves the exact work to the radix select
  float bscale = static_cast<float>(kBins) / (mx - mn);
  if (!(bscale < INFINITY)) bscale = 0.f;
  auto bin_of = [&](float x) {
    int b = static_cast<int>((x - mn) * bscale);
    return b < kBins - 1 ? b : kBins - 1;
  };

  // 2. histogram of value bins
  for (int i = tid; i < kBins; i += kTopkThreads) hist[i] = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kTopkThreads) atomicAdd(&hist[bin_of(s[i])], 1);
  __syncthreads();
  find_crossing(hist, kBins, k, wsum, &s_bin, &s_above);
  const int B = min(max(s_bin, 0), kBins - 1), above = s_above;
  const int in_b = hist[B];
  const int need0 = k - above;  // 1 .. in_b
  __syncthreads();

  // 3. exact threshold inside bin B
  const bool use_lds = in_b <= kCand;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  if (use_lds) {
    for (int i = tid; i < n; i += kTopkThreads) {
      const float x = s[i];
      if (bin_of(x) == B) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < kCand) ckey[slot] = fkey(x);
      }
    }
    __syncthreads();
  }
  uint32_t prefix = 0, pmask = 0;
  int need = need0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    if (use_lds) {
      for (int c = tid; c < in_b; c += kTopkThreads) {
        const uint32_t kx = ckey[c];
        if ((kx & pmask) == prefix) atomicAdd(&hist[(kx >> shift) & 255u], 1);
      }
    } else {
      for (int i = tid; i < n; i += kTopkThreads) {
        const float x = s[i];
        if (bin_of(x) != B) continue;
        const uint32_t kx = fkey(x);
        if ((kx & pmask) == prefix) atomicAdd(&hist[(kx >> shift) & 255u], 1);
      }
    }
    __syncthreads();
    find_crossing(hist, 256, need, wsum, &s_bin, &s_above);
    need -= s_above;
    prefix |= static_cast<uint32_t>(s_bin) << shift;
    pmask |= 0xffu << shift;
    __syncthreads();
  }
  const uint32_t tau = prefix;  // the threshold key; `need` elements equal to it are taken

  // 4. compaction in index order, 4 consecutive elements per thread per tile
  int base_sel = 0, base_eq = 0;
  for (int t0 = 0; t0 < n; t0 += 4 * kTopkThreads) {
    const int i0 = t0 + 4 * tid;
    uint32_t kx[4];
    int gt = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kx[e] = (i0 + e < n) ? fkey(s[i0 + e]) : 0u;
      const bool valid = i0 + e < n;
      gt += valid & (kx[e] > tau);
      eq += valid & (kx[e] == tau);
    }
    int tot_eq, tot_sel;
    const int eq_rank = base_eq + block_excl_scan(eq, wsum, &tot_eq);
    int take = need - eq_rank;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    const int pos0 = base_sel + block_excl_scan(gt + take, wsum, &tot_sel);
    int pos = pos0, eq_seen = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (i0 + e >= n) break;
      if (kx[e] > tau) {
        if (pos < k) out[pos] = i0 + e;
        ++pos;
      } else if (kx[e] == tau) {
        if (eq_seen < take) {
          if (pos < k) out[pos] = i0 + e;
          ++pos;
        }
        ++eq_seen;
      }
    }
    base_eq += tot_eq;
    base_sel += tot_sel;
  }
}

}  // namespace

hipError_t launch_topk(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                       int ld_idx, hipStream_t st) {
  if (rows == 0 || n == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kTopkThreads), 0, st, scores, n, k, ld_scores,
                     idx, ld_idx);
  return hipGetLastError();
}

}  // namespace qk
