// Key scoring pass: s_agg[b,j,t] = max_n q_group[b,j,n] . k[b,j,t] / |k[b,j,t]|.
//
// QUOKA write-up, section 2.2 (cosine score S_ij) and section 2.3 listing
// (matmul of the group queries with the normalised keys, then max over the
// kept queries).  Dividing the max by |k| equals normalising k first, since
// |k| > 0 (a zero key scores 0 on both readings).
//
// The pass is bound by HBM: every past key (d bf16) is read once and 4 bytes
// are written per key.  bf16 kernel (d = 64/128/256):
//   * every wave streams its own share of 32-key blocks -- no LDS, no
//     barriers; the waves of one KV head interleave their blocks so that the
//     concurrent streams spread over the HBM channels.
//     Lane (c, h) loads key c's d-slots [16s + 8h, 16s + 8h + 8) as one
//     16-byte load per step s, which is exactly the matrix-core operand
//     layout (keys as the 32 columns of a 32x32x16 bf16 tile); every load
//     instruction covers 32 B of each of 32 rows and four consecutive steps
//     consume whole 128-byte lines;
//   * blocks are kept STAGES - 1 ahead in registers (unrolled ring), so each
//     wave has that many 8 KiB blocks (d = 128) in flight;
//   * queries are the 32 rows of the tile, so the max over queries is a max
//     over one lane's 16 accumulators plus one exchange with the other half;
//   * the fp32 group queries are split into bf16 high and low parts and both
//     are multiplied (error about 2^-16 relative instead of 2^-8); the matrix
//     cores stay far below their roofline either way;
//   * |k|^2 is summed in fp32 from the same registers (packed bf16 dot
//     products).
// Query rows beyond NQ in the last 32-row block repeat query 0, which leaves
// the max unchanged.
#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

constexpr int kScoreWaves = 4;     // independent waves per workgroup
constexpr int kBlock = 32;         // keys per block (one tile column set)

template <int D, int NQB, int STAGES>
__global__ __launch_bounds__(64 * kScoreWaves, 1) void kvscore_bf16_kernel(
    const float* __restrict__ q_group, const uint16_t* __restrict__ k, float* __restrict__ s_agg,
    int bnkv, int t_past, int kv_cap, int nq_keep, int blocks_per_bj, int blocks_per_wave) {
  constexpr int NS = D / 16;  // k-steps per key
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int waves_per_bj = (blocks_per_bj + blocks_per_wave - 1) / blocks_per_wave;
  const int gw = blockIdx.x * kScoreWaves + wave;
  const int bj = gw / waves_per_bj;
  // Wave wi of this (b, KV head) takes blocks wi, wi + W, wi + 2W, ... (W the
  // waves per head): at any moment the head's waves read neighbouring blocks,
  // so the concurrent streams spread over the HBM channels instead of every
  // wave sitting at the same offset of an equally aligned private run.
  const int wi = gw % waves_per_bj;
  const int nblk = wi < blocks_per_bj ? (blocks_per_bj - wi + waves_per_bj - 1) / waves_per_bj : 0;
  if (bj >= bnkv || nblk == 0) return;
  auto block_of = [&](int m) { return wi + m * waves_per_bj; };

  const uint16_t* kb = k + static_cast<size_t>(bj) * kv_cap * D + 8 * half;
  float* out = s_agg + static_cast<size_t>(bj) * t_past;

  u32x4 buf[STAGES][NS];
  auto load_block = [&](int blk, u32x4* dst) {
    const int row = min(blk * kBlock + col, kv_cap - 1);
    const uint16_t* src = kb + static_cast<size_t>(row) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) dst[s] = ld16(src + 16 * s);
  };
  // first blocks in flight before the query fragments are built
#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i)
    if (i < nblk) load_block(block_of(i), buf[i]);

  bf16x8 qhi[NQB][NS], qlo[NQB][NS];
  {
    const float* qg = q_group + static_cast<size_t>(bj) * nq_keep * D;
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      int row = mb * 32 + col;
      if (row >= nq_keep) row = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const float* src = qg + static_cast<size_t>(row) * D + 16 * s + 8 * half;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
        const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        u32x4 hi, lo;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint16_t h0 = f32_to_bf16(x[2 * p]), h1 = f32_to_bf16(x[2 * p + 1]);
          hi[p] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
          lo[p] = pack_bf16x2(x[2 * p] - bf16_to_f32(h0), x[2 * p + 1] - bf16_to_f32(h1));
        }
        qhi[mb][s] = as_bf16x8(hi);
        qlo[mb][s] = as_bf16x8(lo);
      }
    }
  }

  auto score_block = [&](int blk, const u32x4* w) {
    f32x16 acc[NQB];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) acc[mb] = f32x16{};
    float n2 = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 kf = as_bf16x8(w[s]);
      // |k|^2: one packed bf16 dot product per pair (the products are exact in
      // fp32, accumulation in fp32).  The pairs are taken from the bf16x8
      // operand by shuffles: a bit cast of a single 32-bit vector element was
      // observed to read the wrong register at -O3.
      n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 0, 1),
                                           __builtin_shufflevector(kf, kf, 0, 1), n2, false);
      n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 2, 3),
                                           __builtin_shufflevector(kf, kf, 2, 3), n2, false);
      n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 4, 5),
                                           __builtin_shufflevector(kf, kf, 4, 5), n2, false);
      n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 6, 7),
                                           __builtin_shufflevector(kf, kf, 6, 7), n2, false);
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
    const int key = blk * kBlock + col;
    // m / max(|k|, eps) as m * rsqrt(max(|k|^2, eps^2))
    if (half == 0 && key < t_past) out[key] = m * __builtin_amdgcn_rsqf(fmaxf(n2, kEps * kEps));
  };

  // unrolled ring: this wave's m-th block lives in buf[m % STAGES]
  for (int base = 0; base < nblk; base += STAGES) {
#pragma unroll
    for (int i = 0; i < STAGES; ++i) {
      const int m = base + i;
      if (m >= nblk) break;
      const int nxt = m + STAGES - 1;
      if (nxt < nblk) load_block(block_of(nxt), buf[(i + STAGES - 1) % STAGES]);
      score_block(block_of(m), buf[i]);
    }
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
  constexpr int STAGES = 4;
  const int blocks_per_bj = (t_past + kBlock - 1) / kBlock;
  // about as many waves as are resident (two per SIMD where the registers
  // allow, else one), each streaming its share of blocks
  constexpr long long kResident = (D == 256 || NQB > 1) ? 1024 : 2048;
  const long long total = static_cast<long long>(blocks_per_bj) * bnkv;
  long long bpw = (total + kResident - 1) / kResident;
  if (bpw < 2) bpw = 2;
  if (bpw > blocks_per_bj) bpw = blocks_per_bj;
  const long long waves = ((blocks_per_bj + bpw - 1) / bpw) * static_cast<long long>(bnkv);
  const int wgs = static_cast<int>((waves + kScoreWaves - 1) / kScoreWaves);
  hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES>), dim3(wgs), dim3(64 * kScoreWaves), 0,
                     st, qg, k, s, bnkv, t_past, kv_cap, nq_keep, blocks_per_bj, static_cast<int>(bpw));
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
