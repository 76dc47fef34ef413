// Query sub-selection and group-aware aggregation.
//
// QUOKA write-up, section 2.1 Algorithm 1: per query head, the mean query MQ
// over the chunk, the negated cosine SQ of every chunk query to MQ, and the NQ
// queries with the largest SQ.  Section 2.3 listing: those queries are
// L2-normalised and averaged over the G query heads that share a KV head.
//
// Two kernels, both latency-bound (the chunk is a few MiB at most):
//   1. one workgroup per query head: every thread owns one 16-byte column
//      chunk of a strided set of rows, so all row loads of a pass are in flight
//      at once; the mean is a column sum reduced through LDS, the per-row dot
//      products and norms are reduced across the lanes that share a row, and
//      the top-NQ is a rank count in LDS (number of queries that beat query i,
//      ties going to the lower position) -- exact and deterministic;
//   2. one wave per (sequence, KV head, slot n): the n-th kept query of each of
//      the G heads is normalised and the G unit vectors are averaged in a fixed
//      order.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kHeadThreads = 1024;
constexpr int kRankSplit = 4;  // lanes sharing one row's rank count

template <typename T> struct Chunk8;  // 8 consecutive elements as fp32
template <> struct Chunk8<uint16_t> {
  __device__ __forceinline__ static void load(const uint16_t* p, float* x) {
    const u32x4 w = ld16(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(w[e]); x[2 * e + 1] = bf16hi(w[e]); }
  }
};
template <> struct Chunk8<float> {
  __device__ __forceinline__ static void load(const float* p, float* x) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
  }
};

// Raw 8-element chunk kept in registers between passes.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = ld16(p); }
  __device__ __forceinline__ void get(float* x) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[2 * e] = bf16lo(w[e]); x[2 * e + 1] = bf16hi(w[e]); }
  }
  __device__ __forceinline__ void zero() { w = u32x4{}; }
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
  __device__ __forceinline__ void zero() { a = f32x4{}; b = f32x4{}; }
};

// rank of position i among the scores sq[0..n4*4) (padded with -inf): the
// number of entries larger than s, or equal to it at a lower position
__device__ __forceinline__ int rank_of(const float* sq, int n4, int i, float s) {
  const f32x4* sq4 = reinterpret_cast<const f32x4*>(sq);
  int rank = 0;
#pragma unroll 4
  for (int i4 = 0; i4 < n4; ++i4) {
    const f32x4 v = sq4[i4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rank += (v[e] > s) | ((v[e] == s) & (4 * i4 + e < i));
  }
  return rank;
}

// mq[e] = (sum over r < NRL of part[r][e]) / bcp: S = 1024 / D consecutive
// lanes share column e, each summing NRL / S partials, then a shuffle sum.
template <int D, int NRL>
__device__ __forceinline__ void column_mean(const float* part, float* mq, int bcp) {
  constexpr int S = kHeadThreads / D;
  static_assert(NRL % S == 0 && 64 % S == 0, "column split");
  const int tid = threadIdx.x;
  const int e = tid / S, j = tid % S;
  float sum = 0.f;
#pragma unroll 4
  for (int r = j; r < NRL; r += S) sum += part[r * D + e];
#pragma unroll
  for (int o = 1; o < S; o <<= 1) sum += __shfl_xor(sum, o);
  if (j == 0) mq[e] = sum / static_cast<float>(bcp);
}

// Top-NQ by rank, kRankSplit consecutive lanes per position: each counts over
// a quarter of the scores and the partial counts are summed with shuffles.
__device__ __forceinline__ void rank_and_store(const float* sq, int n4, int bcp, int nq_keep,
                                               int32_t* out) {
  const int tid = threadIdx.x;
  const int part = tid % kRankSplit;
  const int per4 = (n4 + kRankSplit - 1) / kRankSplit;
  const int lo4 = part * per4, hi4 = min(n4, lo4 + per4);
  for (int i0 = 0; i0 < bcp; i0 += kHeadThreads / kRankSplit) {
    const int i = i0 + tid / kRankSplit;
    const float s = i < bcp ? sq[i] : -INFINITY;
    const f32x4* sq4 = reinterpret_cast<const f32x4*>(sq);
    int rank = 0;
#pragma unroll 4
    for (int i4 = lo4; i4 < hi4; ++i4) {
      const f32x4 v = sq4[i4];
#pragma unroll
      for (int e = 0; e < 4; ++e) rank += (v[e] > s) | ((v[e] == s) & (4 * i4 + e < i));
    }
#pragma unroll
    for (int o = 1; o < kRankSplit; o <<= 1) rank += __shfl_xor(rank, o);
    if (part == 0 && i < bcp && rank < nq_keep) out[rank] = i;
  }
}

// Every row of the head is read once into registers (RPT rows per thread).
template <typename T, int D, int RPT>
__global__ __launch_bounds__(kHeadThreads) void qsel_head_reg_kernel(const T* __restrict__ q,
                                                                     int32_t* __restrict__ q_idx,
                                                                     float* __restrict__ sq_out,
                                                                     int bcp, int nq_keep) {
  constexpr int CH = D / 8;
  constexpr int NRL = kHeadThreads / CH;
  extern __shared__ float smem[];
  float* part = smem;                        // [NRL][D]
  float* mq = part + NRL * D;                // [D]
  float* sq = mq + D;                        // [bcp rounded up to 4]
  __shared__ float s_mq2;
  const int tid = threadIdx.x;
  const int c = tid % CH, rl = tid / CH;
  const int bh = blockIdx.x;
  const T* qh = q + static_cast<size_t>(bh) * bcp * D;
  const int n4 = (bcp + 3) / 4;

  Raw8<T> rows[RPT];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = u * NRL + rl;
    if (i < bcp) rows[u].load(qh + static_cast<size_t>(i) * D + 8 * c);
    else rows[u].zero();
  }
  for (int i = bcp + tid; i < 4 * n4; i += kHeadThreads) sq[i] = -INFINITY;

  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    float x[8];
    rows[u].get(x);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += x[e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rl * D + 8 * c + e] = acc[e];
  __syncthreads();
  column_mean<D, NRL>(part, mq, bcp);
  __syncthreads();
  if (tid < 64) {
    float m2 = 0.f;
    for (int e = tid; e < D; e += 64) m2 += mq[e] * mq[e];
    m2 = wave_sum(m2);
    if (tid == 0) s_mq2 = m2;
  }
  __syncthreads();
  const float mq_norm = fmaxf(sqrtf(s_mq2), kEps);
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = mq[8 * c + e];
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int i = u * NRL + rl;
    float x[8];
    rows[u].get(x);
    float dot = 0.f, n2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) { dot += x[e] * m8[e]; n2 += x[e] * x[e]; }
#pragma unroll
    for (int o = CH / 2; o > 0; o >>= 1) {
      dot += __shfl_xor(dot, o);
      n2 += __shfl_xor(n2, o);
    }
    if (c == 0 && i < bcp) {
      const float sc = -dot / (fmaxf(sqrtf(n2), kEps) * mq_norm);
      sq[i] = sc;
      if (sq_out) sq_out[static_cast<size_t>(bh) * bcp + i] = sc;
    }
  }
  __syncthreads();
  rank_and_store(sq, n4, bcp, nq_keep, q_idx + static_cast<size_t>(bh) * nq_keep);
}

// Chunks too long for registers: two passes over global memory (L2).
template <typename T, int D>
__global__ __launch_bounds__(kHeadThreads) void qsel_head_kernel(const T* __restrict__ q,
                                                                 int32_t* __restrict__ q_idx,
                                                                 float* __restrict__ sq_out,
                                                                 int bcp, int nq_keep) {
  constexpr int CH = D / 8;                  // 8-element chunks per row
  constexpr int NRL = kHeadThreads / CH;     // rows handled at once
  extern __shared__ float smem[];
  float* part = smem;                        // [NRL][D] column partial sums
  float* mq = part + NRL * D;                // [D]
  float* sq = mq + D;                        // [bcp]
  __shared__ float s_mq2;

  const int tid = threadIdx.x;
  const int c = tid % CH, rl = tid / CH;
  const int bh = blockIdx.x;                 // (b, h)
  const T* qh = q + static_cast<size_t>(bh) * bcp * D;
  const int n4 = (bcp + 3) / 4;
  for (int i = bcp + tid; i < 4 * n4; i += kHeadThreads) sq[i] = -INFINITY;

  // mean query: column sums over strided rows (kBatch rows' loads in flight
  // per thread), then over the NRL partials
  constexpr int kBatch = 8;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int i0 = 0; i0 < bcp; i0 += kBatch * NRL) {
    float x[kBatch][8];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * NRL + rl;
      if (i < bcp) {
        Chunk8<T>::load(qh + static_cast<size_t>(i) * D + 8 * c, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += x[u][e];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rl * D + 8 * c + e] = acc[e];
  __syncthreads();
  column_mean<D, NRL>(part, mq, bcp);
  __syncthreads();
  if (tid < 64) {
    float m2 = 0.f;
    for (int e = tid; e < D; e += 64) m2 += mq[e] * mq[e];
    m2 = wave_sum(m2);
    if (tid == 0) s_mq2 = m2;
  }
  __syncthreads();
  const float mq_norm = fmaxf(sqrtf(s_mq2), kEps);
  float m8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) m8[e] = mq[8 * c + e];

  // SQ per row: CH lanes share a row (CH divides 64, so they share a wave)
  for (int i0 = 0; i0 < bcp; i0 += kBatch * NRL) {
    float x[kBatch][8];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * NRL + rl;
      if (i < bcp) {
        Chunk8<T>::load(qh + static_cast<size_t>(i) * D + 8 * c, x[u]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = i0 + u * NRL + rl;
      float dot = 0.f, n2 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) { dot += x[u][e] * m8[e]; n2 += x[u][e] * x[u][e]; }
#pragma unroll
      for (int o = CH / 2; o > 0; o >>= 1) {
        dot += __shfl_xor(dot, o);
        n2 += __shfl_xor(n2, o);
      }
      if (c == 0 && i < bcp) {
        const float s = -dot / (fmaxf(sqrtf(n2), kEps) * mq_norm);
        sq[i] = s;
        if (sq_out) sq_out[static_cast<size_t>(bh) * bcp + i] = s;
      }
    }
  }
  __syncthreads();

  // top-NQ by rank
  rank_and_store(sq, n4, bcp, nq_keep, q_idx + static_cast<size_t>(bh) * nq_keep);
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

template <typename T, int D>
hipError_t run(const void* q, int32_t* q_idx, float* sq, float* q_group, int b, int nq, int nkv,
               int bcp, int nq_keep, hipStream_t st) {
  constexpr int NRL = kHeadThreads / (D / 8);
  const size_t shm = sizeof(float) * (static_cast<size_t>(NRL) * D + D + 4 * ((bcp + 3) / 4));
  const int rpt = (bcp + NRL - 1) / NRL;
  const T* qq = static_cast<const T*>(q);
  const dim3 grid(b * nq), block(kHeadThreads);
  if (rpt <= 2)
    hipLaunchKernelGGL((qsel_head_reg_kernel<T, D, 2>), grid, block, shm, st, qq, q_idx, sq, bcp, nq_keep);
  else if (rpt <= 8)
    hipLaunchKernelGGL((qsel_head_reg_kernel<T, D, 8>), grid, block, shm, st, qq, q_idx, sq, bcp, nq_keep);
  else
    hipLaunchKernelGGL((qsel_head_kernel<T, D>), grid, block, shm, st, qq, q_idx, sq, bcp, nq_keep);
  hipLaunchKernelGGL((qgroup_kernel<T, D>), dim3(b * nkv * nq_keep), dim3(64), 0, st,
                     static_cast<const T*>(q), q_idx, q_group, nq, nkv, bcp, nq_keep);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qsel(bool bf16, const void* q, int32_t* q_idx, float* sq, float* q_group, int b,
                       int nq, int nkv, int d, int bcp, int nq_keep, hipStream_t st) {
  if (bf16) {
    if (d == 64) return run<uint16_t, 64>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
    if (d == 128) return run<uint16_t, 128>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
    if (d == 256) return run<uint16_t, 256>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
  } else {
    if (d == 64) return run<float, 64>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
    if (d == 128) return run<float, 128>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
    if (d == 256) return run<float, 256>(q, q_idx, sq, q_group, b, nq, nkv, bcp, nq_keep, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qk
