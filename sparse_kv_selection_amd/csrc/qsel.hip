// Query sub-selection and group-aware aggregation.
//
// QUOKA write-up, section 2.1 Algorithm 1: per query head, the mean query MQ
// over the chunk, the negated cosine SQ of every chunk query to MQ, and the NQ
// queries with the largest SQ.  Section 2.3 listing: those queries are
// L2-normalised and averaged over the G query heads that share a KV head.
//
// Two kernels, both latency-bound (the chunk is a few MiB at most):
//   1. one workgroup per query head: every thread owns one 16-byte column
//      chunk of a strided set of rows, held in registers so all row loads are
//      in flight at once; the mean is a column sum reduced through LDS, the
//      per-row dot products and norms are reduced across the lanes that share
//      a row, and one wave sorts the (score, position) keys with a bitonic
//      network -- exact, deterministic, ties to the lower position;
//   2. (when the group queries are asked for) one wave per (sequence, KV
//      head, slot n): the n-th kept query of each of the G heads is normalised
//      and the G unit vectors are averaged in a fixed order.  The scoring pass
//      can form the same means itself from the kept positions instead.
#include <algorithm>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

// Raw 8-element chunk kept in registers between passes.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld16(p); }
  __device__ __forceinline__ void get(float* x) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(w[e]); x[2 * e + 1] = bf16hi(w[e]); }
  }
  // sum of squares of the 8 values: packed bf16 dot products (exact products,
  // fp32 sums; pairs taken by shuffles, not by a bit cast of one element)
  __device__ __forceinline__ float sumsq() const {
    const bf16x8 v = as_bf16x8(w);
    float n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1),
                                               __builtin_shufflevector(v, v, 0, 1), 0.f, false);
    n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3),
                                         __builtin_shufflevector(v, v, 2, 3), n2, false);
    n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5),
                                         __builtin_shufflevector(v, v, 4, 5), n2, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7),
                                           __builtin_shufflevector(v, v, 6, 7), n2, false);
  }
  __device__ __forceinline__ void zero() { w = u32x4{}; }
  __device__ __forceinline__ void store(uint16_t* p) const { st16(p, w); }
};
template <> struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void get(float* x) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  }
  __device__ __forceinline__ float sumsq() const {
    float n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) n2 += a[e] * a[e] + b[e] * b[e];
    return n2;
  }
  __device__ __forceinline__ void zero() { a = f32x4{}; b = f32x4{}; }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<f32x4*>(p) = a;
    *reinterpret_cast<f32x4*>(p + 4) = b;
  }
};

__device__ __forceinline__ uint32_t okey(float x) { return order_key(x); }

// Bins of the selection histogram (equal width between the chunk's smallest and
// largest SQ; NQ-th key found by one wave's crossing search over them).
constexpr int kQselBins = 512;

// Sum over the lanes of a wave that share lane % CH (CH = 8, 16 or 32): DPP
// rotation by 8 inside each 16-lane row, then the gfx950 lane swaps between
// 16-lane rows and between the 32-lane halves.  Every lane gets the sum.
template <int CH>
__device__ __forceinline__ float rowgroup_sum(float x) {
  static_assert(CH == 8 || CH == 16 || CH == 32, "row group width");
  if constexpr (CH <= 8) x += dpp_f<0x128>(x);  // row_ror:8
  if constexpr (CH <= 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One wave sorts P = 64 * E packed keys descending (bitonic network); lane l
// holds positions [l * E, (l + 1) * E).  Key = (score key << 32) | ~position,
// so larger scores come first and equal scores keep the lower position first.
template <int E>
__device__ __forceinline__ void wave_sort_desc(uint64_t* v) {
  const int lane = threadIdx.x & 63;
  constexpr int P = 64 * E;
#pragma unroll
  for (int kk = 2; kk <= P; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int pe = e ^ j;
          if (pe > e) {
            const int i = lane * E + e;
            const bool desc_block = (i & kk) == 0;  // this block sorts descending
            const uint64_t a = v[e], c = v[pe];
            const bool swap = desc_block ? (a < c) : (a > c);
            v[e] = swap ? c : a;
            v[pe] = swap ? a : c;
          }
        }
      } else {
        const int lx = j / E;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = lane * E + e;
          const uint64_t o = __shfl_xor(v[e], lx);
          const bool lower = (i & j) == 0;
          const bool desc_block = (i & kk) == 0;
          // the lower position of a descending block keeps the larger key
          const bool keep_max = lower == desc_block;
          v[e] = keep_max ? (v[e] > o ? v[e] : o) : (v[e] < o ? v[e] : o);
        }
      }
    }
  }
}

// Wave 0 of the block: top-NQ positions of sq[0..bcp) by decreasing score.
template <int E>
__device__ __forceinline__ void top_positions(const float* sq, int bcp, int nq_keep, int32_t* out,
                                              int* kmap) {
  const int lane = threadIdx.x & 63;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane * E + e;
    v[e] = i < bcp ? (static_cast<uint64_t>(okey(sq[i])) << 32) | static_cast<uint32_t>(~i) : 0ull;
  }
  wave_sort_desc<E>(v);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = lane * E + e;
    if (p < nq_keep) {
      const int32_t i = static_cast<int32_t>(~static_cast<uint32_t>(v[e]));
      out[p] = i;
      kmap[i] = p;
      kmap[bcp + p] = i;
    }
  }
}

// Top-NQ positions of sq[0..bcp) by decreasing key K(i) = (order key of
// sq[i] << 32) | ~i: larger scores first, equal scores at the lower position
// first (keys are unique, so the result is exact and deterministic).
//   1. histogram over kQselBins equal-width bins between the smallest and the
//      largest score (the bin is monotone in the score); the boundary bin B
//      holds the NQ-th largest key, `above` keys lie in higher bins;
//   2. the positions of the higher bins (list A, fewer than NQ) and of bin B
//      (list C) are appended to LDS;
//   3. each entry of A is ranked among A and each of C among C by counting
//      larger keys, 16 threads per entry; A's ranks are final, C's are offset
//      by |A| and kept while below NQ - |A|.
// scratch: hist_words(kQselBins) + 256 + bcp + 4 ints, its histogram and
// counters cleared by select_clear before the barrier that precedes this call;
// red: each wave's smallest and largest SQ, written before that barrier.
// Every thread of the block calls this.  (Inlined: as a called function it
// needed a scratch slot per lane, and a kernel with scratch waits for its
// allocation at launch.)
template <int NT>
__device__ __forceinline__ void select_clear(int* scratch, int bcp) {
  for (int i = threadIdx.x; i < hist_words(kQselBins); i += NT) scratch[i] = 0;
  if (threadIdx.x < 2) scratch[hist_words(kQselBins) + 256 + bcp + threadIdx.x] = 0;
}
template <int NT>
__device__ __forceinline__ void top_positions_select(const float* sq, int* scratch, int bcp, int nq_keep,
                                                     int32_t* out, int* kmap,
                                                     const float (*red)[NT / 64]) {
  constexpr int kB = kQselBins, kWaves = NT / 64, TPP = 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* hist = scratch;
  int* la = hist + hist_words(kB);
  int* lc = la + 256;
  int* cnt = lc + bcp;  // |A|, |C|, B, above
  auto key = [&](int i) {
    return (static_cast<uint64_t>(okey(sq[i])) << 32) | static_cast<uint32_t>(~i);
  };
  float mn = red[0][0], mx = red[1][0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) { mn = fminf(mn, red[0][w]); mx = fmaxf(mx, red[1][w]); }
  float scale = static_cast<float>(kB) / (mx - mn);
  if (!(scale < INFINITY)) scale = 0.f;  // all scores equal: one bin
  auto bin = [&](int i) { return min(max(static_cast<int>((sq[i] - mn) * scale), 0), kB - 1); };
  for (int i = tid; i < bcp; i += NT) atomicAdd(&hist[hpad(bin(i))], 1);
  __syncthreads();
  if (wave == 0) wave_crossing<kB / 64>(hist, nq_keep, &cnt[2], &cnt[3]);
  __syncthreads();
  const int B = cnt[2];
  for (int i0 = 0; i0 < bcp; i0 += NT) {  // uniform trip count (wave scans below)
    const int i = i0 + tid;
    const int bi = i < bcp ? bin(i) : -1;
    const bool in_a = bi > B, in_c = bi == B;
    const uint32_t flag = static_cast<uint32_t>(in_a) | (static_cast<uint32_t>(in_c) << 16);
    const uint32_t incl = wave_incl_scan(flag);
    uint32_t base = 0;
    if (lane == 63) {
      const int na = static_cast<int>(incl & 0xffffu), nc = static_cast<int>(incl >> 16);
      base = static_cast<uint32_t>(na > 0 ? atomicAdd(&cnt[0], na) : 0) |
             (static_cast<uint32_t>(nc > 0 ? atomicAdd(&cnt[1], nc) : 0) << 16);
    }
    base = lane63(base);
    const uint32_t ex = incl - flag;
    if (in_a) la[(base & 0xffffu) + (ex & 0xffffu)] = i;
    if (in_c) lc[(base >> 16) + (ex >> 16)] = i;
  }
  __syncthreads();
  const int na = cnt[0], nc = cnt[1], need = nq_keep - cnt[3];
  const int part = tid % TPP, slot = tid / TPP;
  for (int t0 = 0; t0 < na + nc; t0 += NT / TPP) {  // uniform trip count (group sums)
    const int t = t0 + slot;
    const bool a = t < na;
    const int* list = a ? la : lc;
    const int n = t < na + nc ? (a ? na : nc) : 0;
    const int i = n > 0 ? list[a ? t : t - na] : 0;
    const uint64_t ki = key(i);
    int r = 0;
    for (int j = part; j < n; j += TPP) r += key(list[j]) > ki;
    r = group_sum<TPP>(r);
    if (part == 0 && n > 0) {
      if (a) {
        out[r] = i;
        kmap[i] = r;
        kmap[bcp + r] = i;
      } else if (r < need) {
        out[na + r] = i;
        kmap[i] = na + r;
        kmap[bcp + na + r] = i;
      }
    }
  }
}

// One workgroup of NT threads per query head.  Thread (row lane r, chunk c)
// owns the 8-element chunk c of rows r, r + NT / CH, ...; RPT > 0: all of
// them held in registers (one memory trip); RPT == 0: two passes over memory.
// E > 0: wave 0 sorts 64 * E >= bcp keys; E == 0: histogram selection
// (its scratch reuses the column-sum partials).
template <typename T, int D, int NT, int RPT, int E>
__global__ __launch_bounds__(NT) void qsel_head_kernel(const T* __restrict__ q,
                                                       int32_t* __restrict__ q_idx,
                                                       float* __restrict__ sq_out, int bcp,
                                                       int nq_keep, u32x4* __restrict__ zero,
                                                       int zero16, T* __restrict__ q_kept) {
  constexpr int CH = D / 8;          // chunks per row (CH divides 64)
  constexpr int NRL = NT / CH;       // rows handled at once
  constexpr int S = NT / D > 0 ? NT / D : 1;  // lanes per column in the column sum
  extern __shared__ float smem[];
  float* part = smem;                // [NT / 64][D] column partials, one row per wave (room for
                                     // NRL rows), then the selection scratch
  float* mq = part + (E > 0 ? NRL * D : max(NRL * D, hist_words(kQselBins) + 256 + bcp + 4));  // [D]
  float* sq = mq + D;                // [bcp]
  // [bcp] rank of a kept position, else -1; then [NQ] the kept positions by rank
  int* kmap = reinterpret_cast<int*>(sq + bcp);
  const int tid = threadIdx.x;
  const int c = tid % CH, rl = tid / CH;
  const int bh = blockIdx.x;
  const T* qh = q + static_cast<size_t>(bh) * bcp * D;
  // clears the buffer (zero16 16-byte words) that the scoring pass after this
  // one accumulates into
  for (int i = bh * NT + tid; i < zero16; i += static_cast<int>(gridDim.x) * NT) zero[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = tid; i < bcp; i += NT) kmap[i] = -1;  // (ordered by the barriers below)

  Raw8<T> rows[RPT > 0 ? RPT : 1];
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (RPT > 0) {
#pragma unroll
    for (int u = 0; u < RPT; ++u)  // rows past the chunk re-read its last row (branch-free)
      rows[u].load(qh + static_cast<size_t>(min(u * NRL + rl, bcp - 1)) * D + 8 * c);
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      const bool ok = u * NRL + rl < bcp;
      float x[8];
      rows[u].get(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += ok ? x[e] : 0.f;
    }
  } else {
    for (int i = rl; i < bcp; i += NRL) {
      Raw8<T> r;
      r.load(qh + static_cast<size_t>(i) * D + 8 * c);
      float x[8];
      r.get(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[e];
    }
  }
  // column sums of the wave's rows in registers, one partial row per wave
  constexpr int W = NT / 64;
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = rowgroup_sum<CH>(acc[e]);
  if (lane < CH)
#pragma unroll
    for (int e = 0; e < 8; ++e) part[wave * D + 8 * c + e] = acc[e];
  __syncthreads();
  // mean query: S lanes per column, W / S partials each, then a shuffle sum
  for (int col = tid / S; col < D; col += NT / S) {
    float sum = 0.f;
    for (int r = tid % S; r < W; r += S) sum += part[r * D + col];
    sum = group_sum<S>(sum);
    if (tid % S == 0) mq[col] = sum / static_cast<float>(bcp);
  }
  __syncthreads();
  // |MQ|: the CH lanes of a row group hold all of MQ between them
  float m8[8], m2 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    m8[e] = mq[8 * c + e];
    m2 += m8[e] * m8[e];
  }
  const float mq_norm = fmaxf(sqrtf(group_sum<CH>(m2)), kEps);

  // SQ per row: the CH lanes of a row sit in one wave.  mn / mx: the
  // smallest and largest SQ this lane wrote (for the selection histogram)
  float mn = INFINITY, mx = -INFINITY;
  auto sq_of = [&](float dot, float n2) {
    const float v = -dot / (fmaxf(sqrtf(n2), kEps) * mq_norm);
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
    return v;
  };
  auto score_row = [&](int i, const float* x) {
    float dot = 0.f, n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { dot += x[e] * m8[e]; n2 += x[e] * x[e]; }
    dot = group_sum<CH>(dot);
    n2 = group_sum<CH>(n2);
    if (c == 0 && i < bcp) sq[i] = sq_of(dot, n2);
  };
  if constexpr (RPT > 0) {
    // the row sums of all RPT rows first; then lane c of the row group
    // finishes row u = c (+ CH, ...): one square root and one division per
    // lane instead of RPT (the VALU is the bound of this phase)
    float dots[RPT], n2s[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
      float x[8];
      rows[u].get(x);
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += x[e] * m8[e];
      const float n2 = rows[u].sumsq();
      dots[u] = group_sum<CH>(dot);
      n2s[u] = group_sum<CH>(n2);
    }
#pragma unroll
    for (int u0 = 0; u0 < RPT; u0 += CH) {
      const int u = u0 + c;
      float dot = 0.f, n2 = 1.f;
#pragma unroll
      for (int v = 0; v < RPT; ++v)
        if (v == u) { dot = dots[v]; n2 = n2s[v]; }
      const int i = u * NRL + rl;
      if (u < RPT && i < bcp) sq[i] = sq_of(dot, n2);
    }
  } else {
    for (int i0 = 0; i0 < bcp; i0 += NRL) {
      const int i = i0 + rl;
      float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (i < bcp) {
        Raw8<T> r;
        r.load(qh + static_cast<size_t>(i) * D + 8 * c);
        r.get(x);
      }
      score_row(i, x);
    }
  }
  __shared__ float red[2][W];
  if constexpr (E == 0) {
    mn = group_reduce<64>(mn, [](float a, float b) { return fminf(a, b); });
    mx = group_reduce<64>(mx, [](float a, float b) { return fmaxf(a, b); });
    if (lane == 0) { red[0][wave] = mn; red[1][wave] = mx; }
    select_clear<NT>(reinterpret_cast<int*>(part), bcp);  // the partials are consumed
  }
  __syncthreads();
  int32_t* out = q_idx + static_cast<size_t>(bh) * nq_keep;
  if constexpr (E > 0) {
    if (tid < 64) top_positions<E>(sq, bcp, nq_keep, out, kmap);
  } else {
    top_positions_select<NT>(sq, reinterpret_cast<int*>(part), bcp, nq_keep, out, kmap, red);
  }
  // The kept rows themselves, by rank (q_kept: (b, nq, NQ, d), the chunk's
  // dtype), for a scoring pass that then needs no kept position to find them:
  // rows held in registers go out from there, others are read again.
  if (q_kept) {  // uniform
    __syncthreads();
    T* kh = q_kept + static_cast<size_t>(bh) * nq_keep * D + 8 * c;
    if constexpr (RPT > 0) {
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        const int i = u * NRL + rl;
        const int r = i < bcp ? kmap[i] : -1;
        if (r >= 0) rows[u].store(kh + static_cast<size_t>(r) * D);
      }
    } else {
      for (int r = rl; r < nq_keep; r += NRL) {
        Raw8<T> x;
        x.load(qh + static_cast<size_t>(kmap[bcp + r]) * D + 8 * c);
        x.store(kh + static_cast<size_t>(r) * D);
      }
    }
  }
  // SQ goes out last, coalesced from LDS (unchanged since the barrier above):
  // a global store issued before a barrier would hold that barrier until the
  // store completes
  if (sq_out)
    for (int i = tid; i < bcp; i += NT) sq_out[static_cast<size_t>(bh) * bcp + i] = sq[i];
}

// One wave per (b, j, n): mean over the group's heads of the unit n-th kept query.
template <typename T, int D>
__global__ __launch_bounds__(64) void qgroup_kernel(const T* __restrict__ q,
                                                    const int32_t* __restrict__ q_idx,
                                                    float* __restrict__ q_group, int nq, int nkv,
                                                    int bcp, int nq_keep) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int n = blockIdx.x % nq_keep;
  const int bj = blockIdx.x / nq_keep;
  const int b = bj / nkv, j = bj % nkv;
  const int G = nq / nkv;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  // lane g fetches head g's n-th kept position (G <= 64); rows are then
  // loaded kGBatch heads at a time, all loads in flight before any reduction
  const int myrow = lane < G ? q_idx[(static_cast<size_t>(b) * nq + j * G + lane) * nq_keep + n] : 0;
  constexpr int kGBatch = 8;
  for (int g0 = 0; g0 < G; g0 += kGBatch) {
    float x[kGBatch][PER];
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) {
      const int g = g0 + u;
      const int row = __shfl(myrow, g < G ? g : 0);
      const T* qr = q + ((static_cast<size_t>(b) * nq + j * G + (g < G ? g : 0)) * bcp + row) * D;
#pragma unroll
      for (int e = 0; e < PER; ++e) x[u][e] = g < G ? Elem<T>::load(qr + lane + 64 * e) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kGBatch; ++u) {
      float n2 = 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) n2 += x[u][e] * x[u][e];
      n2 = wave_sum(n2);
      const float inv = g0 + u < G ? 1.0f / fmaxf(sqrtf(n2), kEps) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += x[u][e] * inv;
    }
  }
  const float inv_g = 1.0f / static_cast<float>(G);
  float* out = q_group + (static_cast<size_t>(bj) * nq_keep + n) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) out[lane + 64 * e] = acc[e] * inv_g;
}

template <typename T, int D, int NT, int RPT>
void launch_head(const void* q, int32_t* q_idx, float* sq, int b, int nq, int bcp, int nq_keep,
                 u32x4* zero, int zero16, void* q_kept, hipStream_t st) {
  constexpr int NRL = NT / (D / 8);
  const dim3 grid(b * nq), block(NT);
  const T* qq = static_cast<const T*>(q);
  // up to 64 positions: one-wave sort; beyond: histogram selection
  if (bcp <= 64) {
    const size_t shm = sizeof(float) * (static_cast<size_t>(NRL) * D + D + 2 * bcp + 256);
    hipLaunchKernelGGL((qsel_head_kernel<T, D, NT, RPT, 1>), grid, block, shm, st, qq, q_idx, sq, bcp, nq_keep, zero, zero16, static_cast<T*>(q_kept));
  } else {
    const size_t part = std::max<size_t>(static_cast<size_t>(NRL) * D, hist_words(kQselBins) + 256 + bcp + 4);
    const size_t shm = sizeof(float) * (part + D + 2 * bcp + 256);
    hipLaunchKernelGGL((qsel_head_kernel<T, D, NT, RPT, 0>), grid, block, shm, st, qq, q_idx, sq, bcp, nq_keep, zero, zero16, static_cast<T*>(q_kept));
  }
}

template <typename T, int D>
hipError_t run(const void* q, int32_t* q_idx, float* sq, float* q_group, int b, int nq, int nkv,
               int bcp, int nq_keep, u32x4* zero, int zero16, void* q_kept, hipStream_t st) {
  constexpr int CH = D / 8;
  if (bcp * CH <= 64) {
    launch_head<T, D, 64, 1>(q, q_idx, sq, b, nq, bcp, nq_keep, zero, zero16, q_kept, st);   // decode-sized chunks
  } else if (bcp * CH <= 256) {
    launch_head<T, D, 256, 1>(q, q_idx, sq, b, nq, bcp, nq_keep, zero, zero16, q_kept, st);  // short chunks
  } else {
    constexpr int NRL = 1024 / CH;
    const int rpt = (bcp + NRL - 1) / NRL;
    if (rpt <= 4) launch_head<T, D, 1024, 4>(q, q_idx, sq, b, nq, bcp, nq_keep, zero, zero16, q_kept, st);
    else if (rpt <= 8) launch_head<T, D, 1024, 8>(q, q_idx, sq, b, nq, bcp, nq_keep, zero, zero16, q_kept, st);
    else launch_head<T, D, 1024, 0>(q, q_idx, sq, b, nq, bcp, nq_keep, zero, zero16, q_kept, st);
  }
  if (q_group)
    hipLaunchKernelGGL((qgroup_kernel<T, D>), dim3(b * nkv * nq_keep), dim3(64), 0, st,
                       static_cast<const T*>(q), q_idx, q_group, nq, nkv, bcp, nq_keep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qsel(bool bf16, const void* q, int32_t* q_idx, float* sq, float* q_group, int b,
                       int nq, int nkv, int d, int bcp, int nq_keep, int* zero, size_t zero_bytes,
                       void* q_kept, hipStream_t st) {
  u32x4* z = reinterpret_cast<u32x4*>(zero);
  const int z16 = zero ? static_cast<int>(zero_bytes / 16) : 0;
  if (bf16) {
    if (d == 64) return run<uint16_t, 64>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
    if (d == 128) return run<uint16_t, 128>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
    if (d == 256) return run<uint16_t, 256>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
  } else {
    if (d == 64) return run<float, 64>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
    if (d == 128) return run<float, 128>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
    if (d == 256) return run<float, 256>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, z, z16, q_kept, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qk
