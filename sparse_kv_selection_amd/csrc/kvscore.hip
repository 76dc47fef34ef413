// Key scoring pass: s_agg[b,j,t] = max_n q_group[b,j,n] . k[b,j,t] / |k[b,j,t]|.
//
// QUOKA write-up, section 2.2 (cosine score S_ij) and section 2.3 listing
// (matmul of the group queries with the normalised keys, then max over the
// kept queries).  Dividing the max by |k| equals normalising k first, since
// |k| > 0 (a zero key scores 0 on both readings).
//
// The pass is bound by HBM: every past key (d bf16) is read once and 4 bytes
// are written per key.  Layout of the bf16 kernel (d = 64/128/256):
//   * a workgroup of 4 waves streams tiles of 128 keys of one (b, KV head);
//     each tile is fetched with coalesced 16-byte loads into registers one tile
//     ahead (prefetch), then written to LDS with a 16-byte row pad;
//   * wave w takes keys [32w, 32w + 32) of the tile and multiplies them with the
//     group queries on the matrix cores (32x32x16 bf16, queries as rows, keys
//     as columns), so the max over queries is a max over one lane's 16
//     accumulators plus one exchange with the other lane half;
//   * the fp32 group queries are split into bf16 high and low parts and both
//     are multiplied (error about 2^-16 relative instead of 2^-8); the matrix
//     cores stay far below their roofline either way;
//   * |k|^2 is summed in fp32 from the same fragments.
// Query rows beyond NQ in the last 32-row block repeat query 0, which leaves
// the max unchanged.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kScoreThreads = 256;
constexpr int kScoreTile = 128;  // keys per tile (32 per wave)

template <int D, int NQB>
__global__ __launch_bounds__(kScoreThreads, 2) void kvscore_bf16_kernel(
    const float* __restrict__ q_group, const uint16_t* __restrict__ k, float* __restrict__ s_agg,
    int t_past, int kv_cap, int nq_keep, int tiles_per_bj, int tiles_per_wg) {
  constexpr int kRowElems = D + 8;                 // 16-byte pad per row
  constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  constexpr int kUnits = kScoreTile * kChunks;     // 16-byte units per tile
  constexpr int kPer = kUnits / kScoreThreads;     // units per thread
  static_assert(kUnits % kScoreThreads == 0, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t sk[kScoreTile * kRowElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int wgs_per_bj = (tiles_per_bj + tiles_per_wg - 1) / tiles_per_wg;
  const int bj = blockIdx.x / wgs_per_bj;
  const int tile0 = (blockIdx.x % wgs_per_bj) * tiles_per_wg;
  const int tile1 = min(tile0 + tiles_per_wg, tiles_per_bj);
  if (tile0 >= tile1) return;

  const uint16_t* kb = k + static_cast<size_t>(bj) * kv_cap * D;
  float* out = s_agg + static_cast<size_t>(bj) * t_past;

  // group-query fragments, hi and lo bf16 parts
  bf16x8 qhi[NQB][D / 16], qlo[NQB][D / 16];
  {
    const float* qg = q_group + static_cast<size_t>(bj) * nq_keep * D;
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      int row = mb * 32 + col;
      if (row >= nq_keep) row = 0;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const float* src = qg + static_cast<size_t>(row) * D + 16 * s + 8 * half;
        f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
        f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
        float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        u32x4 hi, lo;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint16_t h0 = f32_to_bf16(x[2 * p]), h1 = f32_to_bf16(x[2 * p + 1]);
          const float r0 = x[2 * p] - bf16_to_f32(h0), r1 = x[2 * p + 1] - bf16_to_f32(h1);
          hi[p] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
          lo[p] = pack_bf16x2(r0, r1);
        }
        qhi[mb][s] = as_bf16x8(hi);
        qlo[mb][s] = as_bf16x8(lo);
      }
    }
  }

  u32x4 pre[kPer];
  auto fetch = [&](int tile) {
    const int key0 = tile * kScoreTile;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kScoreThreads;
      const int r = u / kChunks, c = u - r * kChunks;
      const int row = min(key0 + r, kv_cap - 1);
      pre[p] = ld16(kb + static_cast<size_t>(row) * D + 8 * c);
    }
  };

  fetch(tile0);
  for (int tile = tile0; tile < tile1; ++tile) {
    __syncthreads();  // previous tile's LDS reads are done
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int u = tid + p * kScoreThreads;
      const int r = u / kChunks, c = u - r * kChunks;
      st16(sk + r * kRowElems + 8 * c, pre[p]);
    }
    __syncthreads();
    if (tile + 1 < tile1) fetch(tile + 1);

    f32x16 acc[NQB];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) acc[mb] = f32x16{};
    float n2 = 0.f;
    const uint16_t* krow = sk + (wave * 32 + col) * kRowElems + 8 * half;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(krow + 16 * s);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float a = bf16lo(w[p]), bb = bf16hi(w[p]);
        n2 += a * a + bb * bb;
      }
      const bf16x8 kf = as_bf16x8(w);
#pragma unroll
      for (int mb = 0; mb < NQB; ++mb) {
        acc[mb] = mfma32(qhi[mb][s], kf, acc[mb]);
        acc[mb] = mfma32(qlo[mb][s], kf, acc[mb]);
      }
    }
    float m = acc[0][0];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[mb][r]);
    m = fmaxf(m, __shfl_xor(m, 32));
    n2 += __shfl_xor(n2, 32);
    const int key = tile * kScoreTile + wave * 32 + col;
    if (half == 0 && key < t_past) out[key] = m / fmaxf(sqrtf(n2), kEps);
  }
}

// fp32 path: one thread per key, group queries staged in LDS.
__global__ __launch_bounds__(256) void kvscore_f32_kernel(const float* __restrict__ q_group,
                                                          const float* __restrict__ k,
                                                          float* __restrict__ s_agg, int d,
                                                          int t_past, int kv_cap, int nq_keep) {
  extern __shared__ float sq[];  // [nq_keep * d]
  const int bj = blockIdx.y;
  const float* qg = q_group + static_cast<size_t>(bj) * nq_keep * d;
  for (int e = threadIdx.x; e < nq_keep * d; e += blockDim.x) sq[e] = qg[e];
  __syncthreads();
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= t_past) return;
  const float* kr = k + (static_cast<size_t>(bj) * kv_cap + t) * d;
  float n2 = 0.f;
  for (int e = 0; e < d; ++e) n2 += kr[e] * kr[e];
  float m = -INFINITY;
  for (int n = 0; n < nq_keep; ++n) {
    float dot = 0.f;
    for (int e = 0; e < d; ++e) dot += sq[n * d + e] * kr[e];
    m = fmaxf(m, dot);
  }
  s_agg[static_cast<size_t>(bj) * t_past + t] = m / fmaxf(sqrtf(n2), kEps);
}

template <int D, int NQB>
void launch_bf16(const float* qg, const uint16_t* k, float* s, int bnkv, int t_past, int kv_cap,
                 int nq_keep, hipStream_t st) {
  const int tiles_per_bj = (t_past + kScoreTile - 1) / kScoreTile;
  const long long total = static_cast<long long>(tiles_per_bj) * bnkv;
  int tpw = static_cast<int>(total / 2048);
  tpw = tpw < 1 ? 1 : (tpw > 16 ? 16 : tpw);
  const int wgs_per_bj = (tiles_per_bj + tpw - 1) / tpw;
  hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB>), dim3(wgs_per_bj * bnkv), dim3(kScoreThreads),
                     0, st, qg, k, s, t_past, kv_cap, nq_keep, tiles_per_bj, tpw);
}

}  // namespace

hipError_t launch_kvscore(bool bf16, const float* q_group, const void* k, float* s_agg, int b,
                          int nkv, int d, int t_past, int kv_cap, int nq_keep, hipStream_t st) {
  const int bnkv = b * nkv;
  if (t_past == 0) return hipSuccess;
  if (!bf16) {
    dim3 grid((t_past + 255) / 256, bnkv);
    hipLaunchKernelGGL(kvscore_f32_kernel, grid, dim3(256), sizeof(float) * nq_keep * d, st,
                       q_group, static_cast<const float*>(k), s_agg, d, t_past, kv_cap, nq_keep);
    return hipGetLastError();
  }
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const int nqb = (nq_keep + 31) / 32;
  if (d == 128 && nqb == 1) launch_bf16<128, 1>(q_group, kk, s_agg, bnkv, t_past, kv_cap, nq_keep, st);
  else if (d == 128 && nqb == 2) launch_bf16<128, 2>(q_group, kk, s_agg, bnkv, t_past, kv_cap, nq_keep, st);
  else if (d == 64 && nqb == 1) launch_bf16<64, 1>(q_group, kk, s_agg, bnkv, t_past, kv_cap, nq_keep, st);
  else if (d == 64 && nqb == 2) launch_bf16<64, 2>(q_group, kk, s_agg, bnkv, t_past, kv_cap, nq_keep, st);
  else if (d == 256 && nqb == 1) launch_bf16<256, 1>(q_group, kk, s_agg, bnkv, t_past, kv_cap, nq_keep, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qk
