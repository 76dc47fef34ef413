// Per-row top-k of fp32 scores, indices returned in ascending order.
//
// QUOKA write-up, section 2.3 listing: the BSA keys with the largest
// aggregated score per KV head.  Ties go to the lower position and -0.0
// equals +0.0, so the selected set is unique.
//
// One workgroup of 1024 threads per row; thread t owns the contiguous run
// [t * ITEMS, (t + 1) * ITEMS) so that the output, in index order, needs one
// block prefix sum.  The row stays in registers and the per-element work is
// kept to a few instructions per phase, because a single CU's vector issue
// rate bounds this kernel:
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
//      first `need` elements equal to it, from one block prefix sum of packed
//      (greater, equal) counts.
// Rows longer than 32K scores are streamed from L2 in runs of 16 per pass.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kBins = 2048;
constexpr int kCand = 4096;  // boundary-bin candidates kept in LDS
constexpr int kRun = 16;     // elements per thread per streamed run

// Order-preserving map of a float to uint32 (-0.0 maps like +0.0).
__device__ __forceinline__ uint32_t fkey(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

struct TopkShared {
  int hist[kBins];
  uint32_t cand[kCand];
  int wsum[kTopkWaves];
  float red_min[kTopkWaves], red_max[kTopkWaves];
  int bin, above, cnt, need;
  uint32_t tau;
};

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

// Wave 0 only: the bin b of counts h[0..64 * PER) with
// count(bins > b) < need <= count(bins >= b); writes (*bin, *above) from the
// lane that holds it.  Each lane keeps its PER bins in registers, so the search
// is one batch of LDS reads, one wave scan and a register walk.
template <int PER>
__device__ void wave_crossing(const int* h, int need, int* bin, int* above) {
  const int lane = threadIdx.x & 63;
  const int top = 64 * PER - 1 - lane * PER;  // lane 0 holds the highest bins
  int c[PER];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    c[q] = h[top - q];
    sum += c[q];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  const int ex = incl - sum;
  if (ex < need && need <= incl) {
    int b = top, a = ex;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      if (a + c[q] >= need) { b = top - q; break; }
      a += c[q];
    }
    *bin = b;
    *above = a;
  }
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
    for (int i = tid; i < 256; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    auto count = [&](uint32_t kx) {
      if ((kx & pmask) == prefix) atomicAdd(&sh.hist[(kx >> shift) & 255u], 1);
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

// Rows of n <= 1024 * ITEMS held in registers.
template <int ITEMS>
__global__ __launch_bounds__(kTopkThreads) void topk_reg_kernel(const float* __restrict__ scores,
                                                                int n, int k, int ld_scores,
                                                                int32_t* __restrict__ idx,
                                                                int ld_idx) {
  static_assert(ITEMS % 4 == 0 && ITEMS <= 32, "items per thread");
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
  const int i0 = tid * ITEMS;
  const int nv = max(0, min(ITEMS, n - i0));  // real elements of this thread
  const bool vec = ((ld_scores & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);

  float x[ITEMS];
  if (vec && nv == ITEMS) {
#pragma unroll
    for (int m = 0; m < ITEMS / 4; ++m) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(s + i0 + 4 * m);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * m + e] = v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) x[e] = e < nv ? s[i0 + e] : -INFINITY;
  }

  // 1. min / max (padding is -inf: it never lowers the max; the min skips it)
  float mn = INFINITY, mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    mx = fmaxf(mx, x[e]);
    mn = fminf(mn, e < nv ? x[e] : INFINITY);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { sh.red_min[wave] = mn; sh.red_max[wave] = mx; }
  for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
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
  //    and is counted there, harmlessly: k <= n)
  uint32_t bins[ITEMS / 2];
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    int b = static_cast<int>(__builtin_fmaf(x[e], bscale, boff));
    b = max(0, min(b, kBins - 1));
    atomicAdd(&sh.hist[b], 1);
    if (e & 1) bins[e >> 1] |= static_cast<uint32_t>(b) << 16;
    else bins[e >> 1] = static_cast<uint32_t>(b);
  }
  __syncthreads();
  if (wave == 0) wave_crossing<kBins / 64>(sh.hist, k, &sh.bin, &sh.above);
  __syncthreads();
  const uint32_t B = static_cast<uint32_t>(min(max(sh.bin, 0), kBins - 1));
  const int need0 = k - sh.above;

  // 3. boundary-bin elements -> LDS list
  uint32_t cmask = 0;
#pragma unroll
  for (int e = 0; e < ITEMS; ++e) {
    const uint32_t b = (bins[e >> 1] >> (16 * (e & 1))) & 0xffffu;
    cmask |= static_cast<uint32_t>((b == B) & (e < nv)) << e;
  }
  {
    const int cnt = __popc(cmask);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&sh.cnt, incl);
    base = __shfl(base, 63) + incl - cnt;
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
    emask |= static_cast<uint32_t>((x[e] == tau) & (e < nv)) << e;
  }
  const int gt = __popc(gmask), eq = __popc(emask);
  int tot;
  const int ex = block_excl_scan(gt | (eq << 16), sh.wsum, &tot);
  const int eq_before = ex >> 16;
  int take = need - eq_before;
  take = take < 0 ? 0 : (take > eq ? eq : take);
  if (gt + take > 0) {
    int pos = (ex & 0xffff) + min(need, eq_before);
    // keep the first `take` equal elements of this thread
    uint32_t keep = emask;
    for (int drop = eq - take; drop > 0; --drop) keep &= ~(0x80000000u >> __clz(keep));
    const uint32_t pick = gmask | keep;
#pragma unroll
    for (int e = 0; e < ITEMS; ++e) {
      if ((pick >> e) & 1u) {
        if (pos < k) out[pos] = i0 + e;
        ++pos;
      }
    }
  }
}

// Longer rows: runs of kRun elements per thread, super-tile r covering
// [r * 1024 * kRun, (r + 1) * 1024 * kRun), re-read (from L2) for each pass.
__global__ __launch_bounds__(kTopkThreads) void topk_stream_kernel(const float* __restrict__ scores,
                                                                   int n, int k, int ld_scores,
                                                                   int32_t* __restrict__ idx,
                                                                   int ld_idx) {
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
  const bool vec = ((ld_scores & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  constexpr int kSuper = kTopkThreads * kRun;
  // calls g(x, i0, nv) for each run of this thread, in row order
  auto runs = [&](auto g) {
    for (int base = 0; base < n; base += kSuper) {
      const int i0 = base + tid * kRun;
      const int nv = max(0, min(kRun, n - i0));
      float x[kRun];
      if (vec && nv == kRun) {
#pragma unroll
        for (int m = 0; m < kRun / 4; ++m) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(s + i0 + 4 * m);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * m + e] = v[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < kRun; ++e) x[e] = e < nv ? s[i0 + e] : -INFINITY;
      }
      g(x, i0, nv);
    }
  };

  float mn = INFINITY, mx = -INFINITY;
  runs([&](const float* x, int, int nv) {
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      mx = fmaxf(mx, x[e]);
      mn = fminf(mn, e < nv ? x[e] : INFINITY);
    }
  });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, o));
    mx = fmaxf(mx, __shfl_xor(mx, o));
  }
  if (lane == 0) { sh.red_min[wave] = mn; sh.red_max[wave] = mx; }
  for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
  if (tid == 0) { sh.cnt = 0; sh.bin = 0; sh.above = 0; sh.need = 1; sh.tau = 0u; }
  __syncthreads();
  mn = sh.red_min[0];
  mx = sh.red_max[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) { mn = fminf(mn, sh.red_min[w]); mx = fmaxf(mx, sh.red_max[w]); }
  float bscale = static_cast<float>(kBins) / (mx - mn);
  if (!(bscale < INFINITY)) bscale = 0.f;
  const float boff = -mn * bscale;
  auto bin_of = [&](float v) {
    const int b = static_cast<int>(__builtin_fmaf(v, bscale, boff));
    return static_cast<uint32_t>(max(0, min(b, kBins - 1)));
  };

  runs([&](const float* x, int, int) {
#pragma unroll
    for (int e = 0; e < kRun; ++e) atomicAdd(&sh.hist[bin_of(x[e])], 1);
  });
  __syncthreads();
  if (wave == 0) wave_crossing<kBins / 64>(sh.hist, k, &sh.bin, &sh.above);
  __syncthreads();
  const uint32_t B = static_cast<uint32_t>(min(max(sh.bin, 0), kBins - 1));
  const int need0 = k - sh.above;

  runs([&](const float* x, int, int nv) {
    uint32_t cmask = 0;
#pragma unroll
    for (int e = 0; e < kRun; ++e) cmask |= static_cast<uint32_t>((bin_of(x[e]) == B) & (e < nv)) << e;
    const int cnt = __popc(cmask);
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    int base = 0;
    if (lane == 63 && incl > 0) base = atomicAdd(&sh.cnt, incl);
    base = __shfl(base, 63) + incl - cnt;
    if (cmask) {
#pragma unroll
      for (int e = 0; e < kRun; ++e) {
        if ((cmask >> e) & 1u) {
          if (base < kCand) sh.cand[base] = fkey(x[e]);
          ++base;
        }
      }
    }
  });
  __syncthreads();

  exact_threshold(sh, need0, [&](auto f) {
    runs([&](const float* x, int, int nv) {
#pragma unroll
      for (int e = 0; e < kRun; ++e)
        if (e < nv && bin_of(x[e]) == B) f(x[e]);
    });
  });
  const float tau = key_to_float(sh.tau);
  const int need = sh.need;

  int base_gt = 0, base_eq = 0;
  runs([&](const float* x, int i0, int nv) {
    uint32_t gmask = 0, emask = 0;
#pragma unroll
    for (int e = 0; e < kRun; ++e) {
      gmask |= static_cast<uint32_t>(x[e] > tau) << e;
      emask |= static_cast<uint32_t>((x[e] == tau) & (e < nv)) << e;
    }
    const int gt = __popc(gmask), eq = __popc(emask);
    int tot;
    const int ex = block_excl_scan(gt | (eq << 16), sh.wsum, &tot);
    const int eq_before = base_eq + (ex >> 16);
    int take = need - eq_before;
    take = take < 0 ? 0 : (take > eq ? eq : take);
    if (gt + take > 0) {
      int pos = base_gt + (ex & 0xffff) + min(need, eq_before);
      uint32_t keep = emask;
      for (int drop = eq - take; drop > 0; --drop) keep &= ~(0x80000000u >> __clz(keep));
      const uint32_t pick = gmask | keep;
#pragma unroll
      for (int e = 0; e < kRun; ++e) {
        if ((pick >> e) & 1u) {
          if (pos < k) out[pos] = i0 + e;
          ++pos;
        }
      }
    }
    base_gt += tot & 0xffff;
    base_eq += tot >> 16;
  });
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
  else if (n <= 32 * kTopkThreads)
    hipLaunchKernelGGL(topk_reg_kernel<32>, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  else
    hipLaunchKernelGGL(topk_stream_kernel, grid, block, 0, st, scores, n, k, ld_scores, idx, ld_idx);
  return hipGetLastError();
}

}  // namespace qk
