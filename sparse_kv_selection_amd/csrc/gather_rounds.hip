// Row gather of the selected keys/values, and the round-granular selection.
//
// Gather: the selected KV is the attention's KV input (QUOKA write-up,
// section 4.2 question 3).  Each row is d elements; a thread moves 16 bytes,
// so a wave moves 1 KiB of consecutive row data per instruction.
//
// Rounds: Round Attention press release (Moore Threads), sections 01-02: the
// KV cache is cut at dialogue-round boundaries and the most relevant rounds are
// kept as whole blocks.  A round's score is the max of the aggregated key score
// over its positions; the latest round is always kept.  One workgroup of 1024
// threads per (sequence, KV head): each thread scans runs of consecutive scores
// and merges per-round maxima with integer atomics on order-preserving keys in
// LDS; a rank count picks the top rounds (ties: lower round id); a block prefix
// sum places them, and their positions are written out in ascending order.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

__global__ __launch_bounds__(256) void gather_kernel(const uint8_t* __restrict__ k,
                                                     const uint8_t* __restrict__ v,
                                                     const int32_t* __restrict__ idx, int ld_idx,
                                                     const int32_t* __restrict__ sel_len,
                                                     int n_sel, uint8_t* __restrict__ k_sel,
                                                     uint8_t* __restrict__ v_sel, int row_bytes,
                                                     int kv_cap) {
  const int bj = blockIdx.y;
  const int units = row_bytes / 16;
  const int nsel = min(sel_len ? sel_len[bj] : n_sel, ld_idx);
  const long long u = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int r = static_cast<int>(u / units), c = static_cast<int>(u % units);
  if (r >= nsel) return;
  const int row = min(max(idx[static_cast<size_t>(bj) * ld_idx + r], 0), kv_cap - 1);
  const size_t src = (static_cast<size_t>(bj) * kv_cap + row) * row_bytes + 16 * c;
  const size_t dst = (static_cast<size_t>(bj) * ld_idx + r) * row_bytes + 16 * c;
  st16(k_sel + dst, ld16(k + src));
  st16(v_sel + dst, ld16(v + src));
}

constexpr int kRoundThreads = 1024;
constexpr int kRoundWaves = kRoundThreads / 64;
constexpr int kRun = 16;        // consecutive scores per thread per pass (short rounds)
constexpr int kWaveBatch = 8;   // loads in flight per lane (long rounds)
constexpr int kRankThreads = 16;  // threads ranking one round

// Order-preserving float <-> uint32 maps (for integer atomic max in LDS).
__device__ __forceinline__ uint32_t okey(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ofloat(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Block-wide exclusive prefix sum over kRoundThreads threads.
__device__ int round_excl_scan(int v, int* wsum, int* total) {
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
    int w = lane < kRoundWaves ? wsum[lane] : 0;
#pragma unroll
    for (int o = 1; o < kRoundWaves; o <<= 1) {
      const int y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kRoundWaves) wsum[lane] = w;
  }
  __syncthreads();
  const int off = wave > 0 ? wsum[wave - 1] : 0;
  *total = wsum[kRoundWaves - 1];
  __syncthreads();
  return off + x - v;
}

// Phases 2-4 of the round selection from the rounds' maxima rkey (order keys,
// 0 = empty round) and the clamped bounds so: the chosen rounds, their output
// offsets, their positions, then the per-round outputs.  Every thread of the
// block calls this.
__device__ void choose_rounds(const int* so, const uint32_t* rkey, int* base, int* wsum,
                              int n_rounds, int top_r, int keep_latest, int bj,
                              int32_t* __restrict__ idx, int ld_idx, int32_t* __restrict__ sel_len,
                              float* __restrict__ s_round_out, uint8_t* __restrict__ chosen_out) {
  const int tid = threadIdx.x;
  // 2. chosen rounds by rank (ties: lower round id); the latest is always
  //    kept.  kRankThreads threads count the better rounds of one round.
  const int n_cand = keep_latest ? n_rounds - 1 : n_rounds;
  for (int r0 = 0; r0 < n_rounds; r0 += kRoundThreads / kRankThreads) {
    const int r = r0 + tid / kRankThreads, part = tid % kRankThreads;
    const int rr = r < n_rounds ? r : n_rounds - 1;
    const float sr = rkey[rr] ? ofloat(rkey[rr]) : -INFINITY;
    int better = 0;
    if (rr < n_cand)
      for (int r2 = part; r2 < n_cand; r2 += kRankThreads) {
        const float s2 = rkey[r2] ? ofloat(rkey[r2]) : -INFINITY;
        better += (s2 > sr) | ((s2 == sr) & (r2 < rr));
      }
    better = group_sum<kRankThreads>(better);
    if (r < n_rounds && part == 0) base[r] = (rr >= n_cand || better < top_r) ? 1 : -1;
  }
  __syncthreads();

  // 3. output offsets of the chosen rounds, in round order
  int running = 0;
  for (int r0 = 0; r0 < n_rounds; r0 += kRoundThreads) {
    const int r = r0 + tid;
    const int len = (r < n_rounds && base[r] > 0) ? so[r + 1] - so[r] : 0;
    int tot;
    const int ex = round_excl_scan(len, wsum, &tot);
    if (r < n_rounds) base[r] = base[r] > 0 ? running + ex : -1;
    running += tot;
  }
  __syncthreads();

  // 4. positions of the chosen rounds, ascending: the waves take the rounds
  //    round-robin, and a chosen round's positions go out in coalesced stores
  int32_t* out = idx + static_cast<size_t>(bj) * ld_idx;
  {
    const int lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < n_rounds; r += kRoundWaves) {
      const int b0 = base[r];
      if (b0 < 0) continue;
      for (int t = so[r] + lane; t < so[r + 1]; t += 64) {
        const int o = b0 + (t - so[r]);
        if (o < ld_idx) out[o] = t;
      }
    }
  }
  __syncthreads();
  // per-round outputs last (a global store issued before a barrier holds the
  // barrier until it completes); base[r] >= 0 marks a chosen round
  for (int r = tid; r < n_rounds; r += kRoundThreads) {
    if (s_round_out) s_round_out[static_cast<size_t>(bj) * n_rounds + r] = rkey[r] ? ofloat(rkey[r]) : -INFINITY;
    if (chosen_out) chosen_out[static_cast<size_t>(bj) * n_rounds + r] = base[r] >= 0 ? 1 : 0;
  }
  if (tid == 0) sel_len[bj] = min(running, ld_idx);
}

__global__ __launch_bounds__(kRoundThreads) void round_select_kernel(
    const float* __restrict__ s_agg, int t_past, int n_rounds, const int32_t* __restrict__ off,
    int top_r, int keep_latest, int32_t* __restrict__ idx, int ld_idx,
    int32_t* __restrict__ sel_len, float* __restrict__ s_round_out, uint8_t* __restrict__ chosen_out) {
  extern __shared__ int sm[];
  int* so = sm;                                           // [n_rounds + 1] clamped offsets
  uint32_t* rkey = reinterpret_cast<uint32_t*>(so + n_rounds + 1);  // [n_rounds] max keys
  int* base = reinterpret_cast<int*>(rkey + n_rounds);    // [n_rounds] output offset, -1 = dropped
  __shared__ int wsum[kRoundWaves];
  const int tid = threadIdx.x;
  const int bj = blockIdx.x;
  const float* row = s_agg + static_cast<size_t>(bj) * t_past;

  // round bounds, clamped into [0, t_past] (valid offsets are unaffected)
  for (int r = tid; r <= n_rounds; r += kRoundThreads) so[r] = min(max(off[r], 0), t_past);
  for (int r = tid; r < n_rounds; r += kRoundThreads) rkey[r] = 0u;
  __syncthreads();

  // 1. round maxima.  Long rounds (at least 256 scores on average): one wave
  //    per round, round-robin over the waves, coalesced loads (kWaveBatch x 64
  //    consecutive scores in flight), a wave maximum and a plain store.  Short
  //    rounds: each thread scans runs of kRun consecutive scores, tracking the
  //    round it is in, with integer atomic maxima in LDS.
  if (t_past >= 256 * n_rounds) {
    const int lane = tid & 63, wave = tid >> 6;
    for (int r = wave; r < n_rounds; r += kRoundWaves) {
      const int lo = so[r], hi = so[r + 1];
      float m = -INFINITY;
      for (int base = lo; base < hi; base += 64 * kWaveBatch) {
        float x[kWaveBatch];
#pragma unroll
        for (int u = 0; u < kWaveBatch; ++u) x[u] = row[min(base + 64 * u + lane, t_past - 1)];
#pragma unroll
        for (int u = 0; u < kWaveBatch; ++u)
          if (base + 64 * u + lane < hi) m = fmaxf(m, x[u]);
      }
      m = wave_max(m);
      if (lane == 0) rkey[r] = m == -INFINITY ? 0u : okey(m);
    }
  } else {
    for (int i0 = tid * kRun; i0 < t_past; i0 += kRoundThreads * kRun) {
      float x[kRun];
#pragma unroll
      for (int e = 0; e < kRun; ++e) x[e] = i0 + e < t_past ? row[i0 + e] : -INFINITY;
      int lo = 0, hi = n_rounds - 1;  // round holding i0: largest r with so[r] <= i0
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (so[mid] <= i0) lo = mid; else hi = mid - 1;
      }
      int r = lo;
      float m = -INFINITY;
#pragma unroll
      for (int e = 0; e < kRun; ++e) {
        if (i0 + e >= t_past) break;
        while (r + 1 < n_rounds && i0 + e >= so[r + 1]) {
          if (m != -INFINITY) atomicMax(&rkey[r], okey(m));
          m = -INFINITY;
          ++r;
        }
        m = fmaxf(m, x[e]);
      }
      if (m != -INFINITY) atomicMax(&rkey[r], okey(m));
    }
  }
  __syncthreads();
  choose_rounds(so, rkey, base, wsum, n_rounds, top_r, keep_latest, bj, idx, ld_idx, sel_len,
                s_round_out, chosen_out);
}

// Round choice shared by the KV heads of a sequence: the round maxima of all
// of the sequence's heads (written by round_select_kernel to s_round) meet in
// one maximum per round, and every head gets the rounds chosen by it.  One
// workgroup per (sequence, KV head), rewriting that head's index list,
// length and chosen mask; s_round keeps the heads' own round scores.
__global__ __launch_bounds__(kRoundThreads) void round_share_kernel(
    int nkv, int t_past, int n_rounds, const int32_t* __restrict__ off, int top_r, int keep_latest,
    int32_t* __restrict__ idx, int ld_idx, int32_t* __restrict__ sel_len,
    const float* __restrict__ s_round, uint8_t* __restrict__ chosen_out) {
  extern __shared__ int sm[];
  int* so = sm;
  uint32_t* rkey = reinterpret_cast<uint32_t*>(so + n_rounds + 1);
  int* base = reinterpret_cast<int*>(rkey + n_rounds);
  __shared__ int wsum[kRoundWaves];
  const int tid = threadIdx.x;
  const int bj = blockIdx.x, b = bj / nkv;
  for (int r = tid; r <= n_rounds; r += kRoundThreads) so[r] = min(max(off[r], 0), t_past);
  for (int r = tid; r < n_rounds; r += kRoundThreads) {
    float m = -INFINITY;
    for (int j = 0; j < nkv; ++j) m = fmaxf(m, s_round[(static_cast<size_t>(b) * nkv + j) * n_rounds + r]);
    rkey[r] = m == -INFINITY ? 0u : okey(m);
  }
  __syncthreads();
  choose_rounds(so, rkey, base, wsum, n_rounds, top_r, keep_latest, bj, idx, ld_idx, sel_len,
                nullptr, chosen_out);
}

}  // namespace

hipError_t launch_gather(int esz, const void* k, const void* v, const int32_t* idx, int ld_idx,
                         const int32_t* sel_len, int n_sel, void* k_sel, void* v_sel, int bnkv,
                         int d, int kv_cap, hipStream_t st) {
  const int row_bytes = d * esz;
  const int max_rows = sel_len ? ld_idx : n_sel;
  if (max_rows == 0) return hipSuccess;
  const long long units = static_cast<long long>(max_rows) * (row_bytes / 16);
  dim3 grid(static_cast<unsigned>((units + 255) / 256), bnkv);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, st, static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(v), idx, ld_idx, sel_len, n_sel,
                     static_cast<uint8_t*>(k_sel), static_cast<uint8_t*>(v_sel), row_bytes,
                     kv_cap);
  return hipGetLastError();
}

hipError_t launch_round_select(const float* s_agg, int bnkv, int t_past, int n_rounds,
                               const int32_t* off, int top_r, int keep_latest, int32_t* idx,
                               int ld_idx, int32_t* sel_len, float* s_round, uint8_t* chosen,
                               int shared_nkv, hipStream_t st) {
  const size_t shm = sizeof(int) * (3 * static_cast<size_t>(n_rounds) + 1);
  hipLaunchKernelGGL(round_select_kernel, dim3(bnkv), dim3(kRoundThreads), shm, st, s_agg, t_past,
                     n_rounds, off, top_r, keep_latest, idx, ld_idx, sel_len, s_round, chosen);
  if (shared_nkv > 0)
    hipLaunchKernelGGL(round_share_kernel, dim3(bnkv), dim3(kRoundThreads), shm, st, shared_nkv,
                       t_past, n_rounds, off, top_r, keep_latest, idx, ld_idx, sel_len, s_round,
                       chosen);
  return hipGetLastError();
}

}  // namespace qk
