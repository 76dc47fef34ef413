// Query sub-selection and group-aware aggregation.
//
// QUOKA write-up, section 2.1 Algorithm 1: per query head, the mean query MQ
// over the chunk, the negated cosine SQ of every chunk query to MQ, and the NQ
// queries with the largest SQ.  Section 2.3 listing: those queries are
// L2-normalised and averaged over the G query heads that share a KV head.
//
// One workgroup per (sequence, KV head); its G query heads are processed in
// turn.  Dot products and norms are wavefront reductions over the head dim;
// the top-NQ is a rank count (number of queries that beat query i, ties going
// to the lower position), which is exact, deterministic and cheap for chunk
// sizes up to a few thousand.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kQselThreads = 256;

template <typename T>
__global__ __launch_bounds__(kQselThreads) void qsel_kernel(const T* __restrict__ q,
                                                            int32_t* __restrict__ q_idx,
                                                            float* __restrict__ sq_out,
                                                            float* __restrict__ q_group, int nq,
                                                            int nkv, int d, int bcp, int nq_keep) {
  extern __shared__ float smem[];
  float* mq = smem;                  // [d]
  float* sq = mq + d;                // [bcp]
  float* qn2 = sq + bcp;             // [bcp] squared norms
  int* sel = reinterpret_cast<int*>(qn2 + bcp);  // [nq_keep]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = kQselThreads / 64;
  const int bj = blockIdx.x;
  const int b = bj / nkv, j = bj % nkv;
  const int G = nq / nkv;
  const float inv_g = 1.0f / static_cast<float>(G);
  float* qg = q_group + static_cast<size_t>(bj) * nq_keep * d;

  for (int g = 0; g < G; ++g) {
    const int h = j * G + g;
    const T* qh = q + static_cast<size_t>(b * nq + h) * bcp * d;

    // mean query over the chunk's token axis
    for (int e = tid; e < d; e += kQselThreads) {
      float s = 0.f;
      for (int i = 0; i < bcp; ++i) s += Elem<T>::load(qh + static_cast<size_t>(i) * d + e);
      mq[e] = s / static_cast<float>(bcp);
    }
    __syncthreads();

    float mq2 = 0.f;
    for (int e = lane; e < d; e += 64) mq2 += mq[e] * mq[e];
    mq2 = wave_sum(mq2);
    const float mq_norm = fmaxf(sqrtf(mq2), kEps);

    // negated cosine of every chunk query to the mean query
    for (int i = wave; i < bcp; i += nwaves) {
      float dot = 0.f, n2 = 0.f;
      for (int e = lane; e < d; e += 64) {
        const float x = Elem<T>::load(qh + static_cast<size_t>(i) * d + e);
        dot += x * mq[e];
        n2 += x * x;
      }
      dot = wave_sum(dot);
      n2 = wave_sum(n2);
      if (lane == 0) {
        const float s = -dot / (fmaxf(sqrtf(n2), kEps) * mq_norm);
        sq[i] = s;
        qn2[i] = n2;
        if (sq_out) sq_out[static_cast<size_t>(b * nq + h) * bcp + i] = s;
      }
    }
    __syncthreads();

    // top-NQ by rank: queries that beat i are larger, or equal at a lower position
    for (int i = tid; i < bcp; i += kQselThreads) {
      const float s = sq[i];
      int rank = 0;
      for (int i2 = 0; i2 < bcp; ++i2) {
        const float s2 = sq[i2];
        rank += (s2 > s) | ((s2 == s) & (i2 < i));
      }
      if (rank < nq_keep) {
        sel[rank] = i;
        q_idx[static_cast<size_t>(b * nq + h) * nq_keep + rank] = i;
      }
    }
    __syncthreads();

    // accumulate the unit kept queries, slot by slot, over the group's heads;
    // each element is owned by one thread across the g loop
    for (int e = tid; e < nq_keep * d; e += kQselThreads) {
      const int n = e / d, c = e - n * d;
      const int row = sel[n];
      const float inv = 1.0f / fmaxf(sqrtf(qn2[row]), kEps);
      const float val = Elem<T>::load(qh + static_cast<size_t>(row) * d + c) * inv;
      float acc = (g == 0) ? 0.f : qg[e];
      acc += val;
      qg[e] = (g == G - 1) ? acc * inv_g : acc;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_qsel(bool bf16, const void* q, int32_t* q_idx, float* sq, float* q_group, int b,
                       int nq, int nkv, int d, int bcp, int nq_keep, hipStream_t st) {
  const size_t shm = sizeof(float) * (d + 2 * static_cast<size_t>(bcp)) + sizeof(int) * nq_keep;
  dim3 grid(b * nkv), block(kQselThreads);
  if (bf16)
    hipLaunchKernelGGL(qsel_kernel<uint16_t>, grid, block, shm, st,
                       static_cast<const uint16_t*>(q), q_idx, sq, q_group, nq, nkv, d, bcp,
                       nq_keep);
  else
    hipLaunchKernelGGL(qsel_kernel<float>, grid, block, shm, st, static_cast<const float*>(q),
                       q_idx, sq, q_group, nq, nkv, d, bcp, nq_keep);
  return hipGetLastError();
}

}  // namespace qk
