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

struct ScoreArgs {
  const float* q_group;    // (b, nkv, nq_keep, d) fp32, or nullptr: formed from q / q_idx
  const uint16_t* q;       // (b, nq, bcp, d) the chunk's queries
  const int32_t* q_idx;    // (b, nq, nq_keep) kept positions
  const uint16_t* q_kept;  // (b, nq, nq_keep, d) the kept rows by rank, or nullptr
  const void* k;           // (b, nkv, kv_cap, d) bf16, or E4M3 bytes
  float* s_agg;
  int* hist;               // (b * nkv, kL1Bins) zeroed level-1 histograms, or nullptr
  const uint16_t* conv_src;  // bf16 cache whose chunk rows are stored as E4M3 codes, or nullptr
  uint8_t* conv_dst;         // ... into this 8-bit copy (same element positions)
  int conv_total;            // (b, KV head, chunk row, 16 elements) units to convert
  int nkv, group, bcp, t_past, kv_cap, nq_keep;
  int blocks_per_bj, wgs_per_bj;
};

// Group queries of one (b, KV head) formed by the whole workgroup (section 2.3
// listing: the kept queries are L2-normalised, then averaged over the G heads
// of the group), split into bf16 high and low parts in LDS.  Thread pair p =
// (row n, 8-element chunk c); the CH threads of a row are adjacent lanes of
// one wave, so a row norm is a shuffle sum.
//
// Order of the memory trips: the kept positions, then the kept rows of the
// first GB heads (issue), and only then the caller's first key blocks.  Loads
// retire in issue order, so rows requested after the key blocks could not be
// used before every one of those blocks had arrived (several microseconds at
// the start of the pass, when every wave has its ring in flight).  Heads
// beyond the first GB are loaded in build, behind the key blocks.
template <int D, int NQB, int GB>
struct GroupBuild {
  static constexpr int CH = D / 8;
  static constexpr int ROWS = NQB * 32;
  static constexpr int U = ROWS * CH / (64 * kScoreWaves);  // pairs per thread
  static constexpr int LD = D + 8;                           // padded LDS row (bf16)
  static_assert(U >= 1 && (64 * kScoreWaves) % CH == 0, "pair layout");

  u32x4 x[U][GB];

  // kept rows of heads g0 .. g0 + GB - 1 (clamped to the last head: the loads
  // are unconditional, so the wait before their use counts exactly them)
  __device__ __forceinline__ void issue(const ScoreArgs& a, int bj, int g0) {
    const int b = bj / a.nkv, j = bj - b * a.nkv;
    if (a.q_kept) {  // uniform: the kept rows gathered by the query pass, one trip
      const uint16_t* kr = a.q_kept + (static_cast<size_t>(b) * a.nkv + j) * a.group * a.nq_keep * D +
                           8 * (threadIdx.x % CH);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int n = min((static_cast<int>(threadIdx.x) + 64 * kScoreWaves * u) / CH, a.nq_keep - 1);
#pragma unroll
        for (int gg = 0; gg < GB; ++gg) {
          const int g = min(g0 + gg, a.group - 1);
          x[u][gg] = ld16(kr + (static_cast<size_t>(g) * a.nq_keep + n) * D);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    const int32_t* qi = a.q_idx + (static_cast<size_t>(b) * a.nkv + j) * a.group * a.nq_keep;
    const uint16_t* qb = a.q + (static_cast<size_t>(b) * a.nkv + j) * a.group * a.bcp * D;
    const int c = threadIdx.x % CH;
    int pos[U][GB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = min((static_cast<int>(threadIdx.x) + 64 * kScoreWaves * u) / CH, a.nq_keep - 1);
#pragma unroll
      for (int gg = 0; gg < GB; ++gg) {
        const int g = min(g0 + gg, a.group - 1);
        pos[u][gg] = min(max(qi[g * a.nq_keep + n], 0), a.bcp - 1);
      }
    }
    // every index load goes out before the first one is used (the scheduler
    // would otherwise sink each load down to its use and wait on it there)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int gg = 0; gg < GB; ++gg) {
        const int g = min(g0 + gg, a.group - 1);
        x[u][gg] = ld16(qb + (static_cast<size_t>(g) * a.bcp + pos[u][gg]) * D + 8 * c);
      }
    __builtin_amdgcn_sched_barrier(0);
  }

  // DOT: the kept rows enter unnormalised (dot-product scoring variant)
  template <bool DOT>
  __device__ __forceinline__ void accumulate(const ScoreArgs& a, int g0, float (&acc)[U][8]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int gg = 0; gg < GB; ++gg) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[2 * e] = bf16lo(x[u][gg][e]); v[2 * e + 1] = bf16hi(x[u][gg][e]); }
        float inv = g0 + gg < a.group ? 1.0f : 0.f;
        if constexpr (!DOT) {
          float n2 = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) n2 += v[e] * v[e];
#pragma unroll
          for (int o = CH / 2; o > 0; o >>= 1) n2 += __shfl_xor(n2, o);
          inv *= 1.0f / fmaxf(sqrtf(n2), kEps);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u][e] += v[e] * inv;
      }
  }

  // Completes the group queries from the rows of the first batch (already
  // issued) and writes them to LDS; the caller then passes an LDS barrier.
  template <bool DOT>
  __device__ __forceinline__ void build(const ScoreArgs& a, int bj, uint16_t* s_hi,
                                        uint16_t* s_lo) {
    const int c = threadIdx.x % CH;
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[u][e] = 0.f;
    accumulate<DOT>(a, 0, acc);
    for (int g0 = GB; g0 < a.group; g0 += GB) {
      issue(a, bj, g0);
      accumulate<DOT>(a, g0, acc);
    }
    const float inv_g = 1.0f / static_cast<float>(a.group);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int n = (static_cast<int>(threadIdx.x) + 64 * kScoreWaves * u) / CH;
      u32x4 hi, lo;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float x0 = acc[u][2 * p] * inv_g, x1 = acc[u][2 * p + 1] * inv_g;
        const uint16_t h0 = f32_to_bf16(x0), h1 = f32_to_bf16(x1);
        hi[p] = static_cast<uint32_t>(h0) | (static_cast<uint32_t>(h1) << 16);
        lo[p] = pack_bf16x2(x0 - bf16_to_f32(h0), x1 - bf16_to_f32(h1));
      }
      if (n < a.nq_keep) {
        *reinterpret_cast<u32x4*>(s_hi + n * LD + 8 * c) = hi;
        *reinterpret_cast<u32x4*>(s_lo + n * LD + 8 * c) = lo;
      }
    }
  }
};

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for the global loads in flight (the key blocks of the ring).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two E4M3 codes (bytes 2 SEL, 2 SEL + 1 of w) as a bf16 pair.  The hardware
// decode to fp32 is exact, and so is keeping the upper half of the fp32
// values: an E4M3 value has 3 mantissa bits.
template <bool SEL>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), SEL);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// FP8: keys are E4M3 bytes; lane (c, h) loads key c's bytes [32j + 16h, +16)
// per load j and decodes them into the operands of steps 2j and 2j + 1, so
// step s of lane half h covers d-slots qofs(s, h) .. + 8 (the group queries
// are read in the same order; a dot product does not depend on the order of
// d).  DOT: no key norm (dot-product scoring variant).
template <bool FP8>
__device__ __forceinline__ int qofs(int s, int half) {
  return FP8 ? 32 * (s >> 1) + 16 * half + 8 * (s & 1) : 16 * s + 8 * half;
}

// Waves per SIMD the launch grid counts on (kResident below): two, except for
// d = 256 and two query blocks, whose registers allow one.
template <int D, int NQB>
constexpr int score_waves_per_simd() { return (D == 256 || NQB > 1) ? 1 : 2; }

template <int D, int NQB, int STAGES, bool GROUPED, bool FP8, bool DOT, int GB>
__global__ __launch_bounds__(64 * kScoreWaves, (score_waves_per_simd<D, NQB>())) void kvscore_bf16_kernel(ScoreArgs a) {
  constexpr int NS = D / 16;  // k-steps per key
  constexpr int NL = FP8 ? D / 32 : NS;  // 16-byte loads per key
  static_assert(GROUPED || (!FP8 && !DOT), "variants form their group queries");
  using GBuild = GroupBuild<D, NQB, GB>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  // a workgroup's waves all score one (b, KV head)
  const int bj = blockIdx.x / a.wgs_per_bj;
  const int waves_per_bj = a.wgs_per_bj * kScoreWaves;
  // Wave wi of this (b, KV head) takes blocks wi, wi + W, wi + 2W, ... (W the
  // waves per head): at any moment the head's waves read neighbouring blocks,
  // so the concurrent streams spread over the HBM channels instead of every
  // wave sitting at the same offset of an equally aligned private run.
  const int wi = (blockIdx.x - bj * a.wgs_per_bj) * kScoreWaves + wave;
  const int nblk = wi < a.blocks_per_bj ? (a.blocks_per_bj - wi + waves_per_bj - 1) / waves_per_bj : 0;
  auto block_of = [&](int m) { return wi + m * waves_per_bj; };

  // this lane's first byte of key row 0 of the (b, KV head)
  const char* kb = static_cast<const char*>(a.k) +
                   (static_cast<size_t>(bj) * a.kv_cap * D + (FP8 ? 16 : 8) * half) * (FP8 ? 1 : 2);
  float* out = a.s_agg + static_cast<size_t>(bj) * a.t_past;

  // Histogram of the scores written, over the level-1 bins of the selection
  // that follows: counted in LDS, added to the row's histogram at the end
  // (one atomic per bin the workgroup touched).
  __shared__ int lh[kL1Bins];
  const bool with_hist = a.hist != nullptr;  // uniform
  if (with_hist)
    for (int i = threadIdx.x; i < kL1Bins; i += 64 * kScoreWaves) lh[i] = 0;

  GBuild gb;
  if constexpr (GROUPED) gb.issue(a, bj, 0);  // kept positions, then their rows

  // The chunk's own key rows stored as E4M3 codes (qk_select with 8-bit keys:
  // the rows this chunk appends, scored by later passes).  The grid's
  // workgroups split the (b, KV head, row, 16 elements) units; up to d <= 128
  // a thread's first unit is requested with the kept rows, before any key,
  // and stored once the query build has waited for them; the rest (and every
  // unit at d = 256, whose registers are full) at the end.
  const int conv_total = a.conv_dst ? a.conv_total : 0;  // uniform
  const int conv_per = conv_total ? (conv_total + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x) : 0;
  const int conv_lo = static_cast<int>(blockIdx.x) * conv_per;
  const int conv_hi = min(conv_lo + conv_per, conv_total);
  auto conv_off = [&](int u) {  // element offset of unit u in the cache
    constexpr int UPR = D / 16;
    const int c16 = u % UPR, rr = u / UPR;
    const int r = rr % a.bcp, bjc = rr / a.bcp;
    return (static_cast<size_t>(bjc) * a.kv_cap + a.t_past + r) * D + 16 * c16;
  };
  auto conv_store = [&](size_t off, const u32x4* w) {
    float x[16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * h + 2 * e] = bf16lo(w[h][e]);
        x[8 * h + 2 * e + 1] = bf16hi(w[h][e]);
      }
    st16(a.conv_dst + off, e4m3x16(x));
  };
  constexpr bool kConvEarly = D <= 128;
  u32x4 cw[2] = {u32x4{}, u32x4{}};
  size_t coff = 0;
  if constexpr (kConvEarly) {
    if (conv_total) {  // uniform; clamped, so every thread loads
      coff = conv_off(min(conv_lo + static_cast<int>(threadIdx.x), conv_total - 1));
      cw[0] = ld16(a.conv_src + coff);
      cw[1] = ld16(a.conv_src + coff + 8);
    }
  }

  u32x4 buf[STAGES][NL];
  auto load_block = [&](int blk, u32x4* dst) {
    const int row = min(blk * kBlock + col, a.kv_cap - 1);
    const char* src = kb + static_cast<size_t>(row) * D * (FP8 ? 1 : 2);
#pragma unroll
    for (int s = 0; s < NL; ++s) dst[s] = ld16(src + 32 * s);
  };
  // First blocks in flight while the query fragments are built.  The loads
  // are unconditional (a wave with fewer blocks re-reads its first one, or a
  // clamped row): behind a branch, the wait before the kept rows' first use
  // would have to assume that no key load is in flight and wait for all.
  // Grouped, shallow ring (few blocks per wave, short rows): one block before
  // the kept rows are used, the rest of the ring after.  Every key request in
  // flight on the chip delays the kept rows (they queue behind the key lines
  // in the memory pipeline), and the rows gate every wave's first product;
  // one block per wave measured best there.  With the deep ring (long rows)
  // the whole ring goes out first: the wait for the rows is then covered
  // (measured 5 % faster at 128K keys, 7 % slower at 32K).
  constexpr int kEarly = (GROUPED && STAGES <= 3) ? 1 : STAGES - 1;
#pragma unroll
  for (int i = 0; i < kEarly; ++i) load_block(block_of(i < nblk ? i : 0), buf[i]);
  __builtin_amdgcn_sched_barrier(0);

  bf16x8 qhi[NQB][NS], qlo[NQB][NS];
  if constexpr (GROUPED) {
    __shared__ __align__(16) uint16_t s_hi[GBuild::ROWS * GBuild::LD];
    __shared__ __align__(16) uint16_t s_lo[GBuild::ROWS * GBuild::LD];
    gb.template build<DOT>(a, bj, s_hi, s_lo);
    if constexpr (kConvEarly)
      if (conv_total && conv_lo + static_cast<int>(threadIdx.x) < conv_hi) conv_store(coff, cw);
#pragma unroll
    for (int i = kEarly; i < STAGES - 1; ++i) load_block(block_of(i < nblk ? i : 0), buf[i]);
    lds_barrier();
    // (with the histogram or a conversion, every wave goes on to the end)
    if (nblk == 0 && !with_hist && !conv_total) return;
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      int row = mb * 32 + col;
      if (row >= a.nq_keep) row = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int off = row * GBuild::LD + qofs<FP8>(s, half);
        qhi[mb][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(s_hi + off));
        qlo[mb][s] = as_bf16x8(*reinterpret_cast<const u32x4*>(s_lo + off));
      }
    }
  } else {
    if (with_hist) lds_barrier();  // the cleared histogram before any count
    if (nblk == 0 && !with_hist && !conv_total) return;
    const float* qg = a.q_group + static_cast<size_t>(bj) * a.nq_keep * D;
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) {
      int row = mb * 32 + col;
      if (row >= a.nq_keep) row = 0;
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

  // Scores are staged per wave in LDS and written in bursts of kBurst blocks
  // (two blocks per store instruction): a store of 128 bytes after every
  // block, between the key reads, cost 7 % of the pass at 128K keys per head
  // and in the decode batch (measured; without any stores the pass reads at
  // the rate of a bare streaming read).
  constexpr int kBurst = 64;
  __shared__ float sstage[kScoreWaves][kBurst][kBlock];
  int nst = 0;  // blocks staged, uniform
  auto burst = [&](int m_end) {  // this wave's blocks m_end - nst .. m_end - 1
    for (int t = half; t < nst; t += 2) {
      const int key = block_of(m_end - nst + t) * kBlock + col;
      if (key < a.t_past) out[key] = sstage[wave][t][col];
    }
    nst = 0;
  };
  auto score_block = [&](int blk, const u32x4* w) {
    f32x16 acc[NQB];
#pragma unroll
    for (int mb = 0; mb < NQB; ++mb) acc[mb] = f32x16{};
    float n2 = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8 kf;
      if constexpr (FP8) {
        const u32x4& x = w[s >> 1];
        const uint32_t w0 = (s & 1) ? x[2] : x[0], w1 = (s & 1) ? x[3] : x[1];
        u32x4 y;
        y[0] = e4m3x2_to_bf16x2<false>(w0);
        y[1] = e4m3x2_to_bf16x2<true>(w0);
        y[2] = e4m3x2_to_bf16x2<false>(w1);
        y[3] = e4m3x2_to_bf16x2<true>(w1);
        kf = as_bf16x8(y);
      } else {
        kf = as_bf16x8(w[s]);
      }
      // |k|^2: one packed bf16 dot product per pair (the products are exact in
      // fp32, accumulation in fp32).  The pairs are taken from the bf16x8
      // operand by shuffles: a bit cast of a single 32-bit vector element was
      // observed to read the wrong register at -O3.
      if constexpr (!DOT) {
        n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 0, 1),
                                             __builtin_shufflevector(kf, kf, 0, 1), n2, false);
        n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 2, 3),
                                             __builtin_shufflevector(kf, kf, 2, 3), n2, false);
        n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 4, 5),
                                             __builtin_shufflevector(kf, kf, 4, 5), n2, false);
        n2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(kf, kf, 6, 7),
                                             __builtin_shufflevector(kf, kf, 6, 7), n2, false);
      }
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
    const int key = blk * kBlock + col;
    float v = m;
    if constexpr (!DOT) {
      n2 += __shfl_xor(n2, 32);
      // m / max(|k|, eps) as m * rsqrt(max(|k|^2, eps^2))
      v = m * __builtin_amdgcn_rsqf(fmaxf(n2, kEps * kEps));
    }
    if (with_hist && half == 0 && key < a.t_past) atomicAdd(&lh[l1_bin(order_key(v))], 1);
    if (half == 0) sstage[wave][nst][col] = v;
    ++nst;
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
      if (nst == kBurst) burst(m + 1);
    }
  }
  burst(nblk);
  for (int u = conv_lo + (kConvEarly ? 64 * kScoreWaves : 0) + static_cast<int>(threadIdx.x); u < conv_hi;
       u += 64 * kScoreWaves) {
    const size_t off = conv_off(u);
    const u32x4 w[2] = {ld16(a.conv_src + off), ld16(a.conv_src + off + 8)};
    conv_store(off, w);
  }
  if (with_hist) {
    lds_barrier();
    int* gh = a.hist + static_cast<size_t>(bj) * kL1Bins;
    for (int i = threadIdx.x; i < kL1Bins; i += 64 * kScoreWaves) {
      const int c = lh[i];
      if (c) atomicAdd(gh + i, c);
    }
  }
}

// Measurement only: the scoring pass's key loads -- the same grid, block
// order, lane layout and ring of blocks in flight -- with nothing computed.
// The loaded words are folded by XOR; the fold reaches the sink only if it
// equals a fixed sentinel, which keeps every load live while writing nothing
// in practice.  Its duration is the floor of a scoring pass over these bytes.
template <int D, int STAGES, bool FP8>
__global__ __launch_bounds__(64 * kScoreWaves) void read_keys_kernel(ScoreArgs a, u32x4* sink) {
  constexpr int NL = FP8 ? D / 32 : D / 16;  // 16-byte loads per key
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int bj = blockIdx.x / a.wgs_per_bj;
  const int waves_per_bj = a.wgs_per_bj * kScoreWaves;
  const int wi = (blockIdx.x - bj * a.wgs_per_bj) * kScoreWaves + wave;
  const int nblk = wi < a.blocks_per_bj ? (a.blocks_per_bj - wi + waves_per_bj - 1) / waves_per_bj : 0;
  auto block_of = [&](int m) { return wi + m * waves_per_bj; };
  const char* kb = static_cast<const char*>(a.k) +
                   (static_cast<size_t>(bj) * a.kv_cap * D + (FP8 ? 16 : 8) * half) * (FP8 ? 1 : 2);
  u32x4 buf[STAGES][NL];
  auto load_block = [&](int blk, u32x4* dst) {
    const int row = min(blk * kBlock + col, a.kv_cap - 1);
    const char* src = kb + static_cast<size_t>(row) * D * (FP8 ? 1 : 2);
#pragma unroll
    for (int s = 0; s < NL; ++s) dst[s] = ld16(src + 32 * s);
  };
#pragma unroll
  for (int i = 0; i < STAGES - 1; ++i) load_block(block_of(i < nblk ? i : 0), buf[i]);
  u32x4 fold = u32x4{0u, 0u, 0u, 0u};
  for (int base = 0; base < nblk; base += STAGES) {
#pragma unroll
    for (int i = 0; i < STAGES; ++i) {
      const int m = base + i;
      if (m >= nblk) break;
      const int nxt = m + STAGES - 1;
      if (nxt < nblk) load_block(block_of(nxt), buf[(i + STAGES - 1) % STAGES]);
#pragma unroll
      for (int s = 0; s < NL; ++s) fold ^= buf[i][s];
    }
  }
  if ((fold[0] ^ fold[1] ^ fold[2] ^ fold[3]) == 0x5eed1e55u) *sink = fold;
}

// fp32 path: one thread per key, group queries staged in LDS (copied, or
// formed from the kept queries as in the bf16 path: per (n, g) the inverse norm
// of the kept row, then the mean of the normalised rows).
__global__ __launch_bounds__(256) void kvscore_f32_kernel(ScoreCall c) {
  extern __shared__ float sq[];  // [nq_keep * d] group queries, then [nq_keep * G] inverse norms
  const int bj = blockIdx.y, d = c.d, nq_keep = c.nq_keep;
  if (c.q_group) {
    const float* qg = c.q_group + static_cast<size_t>(bj) * nq_keep * d;
    for (int e = threadIdx.x; e < nq_keep * d; e += blockDim.x) sq[e] = qg[e];
  } else {
    const int G = c.nq / c.nkv, b = bj / c.nkv, j = bj - b * c.nkv;
    const float* qb = static_cast<const float*>(c.q) + (static_cast<size_t>(b) * c.nq + j * G) * c.bcp * d;
    const int32_t* qi = c.q_idx + (static_cast<size_t>(b) * c.nq + j * G) * nq_keep;
    float* inv = sq + nq_keep * d;
    auto row = [&](int n, int g) {
      const int pos = min(max(qi[g * nq_keep + n], 0), c.bcp - 1);
      return qb + (static_cast<size_t>(g) * c.bcp + pos) * d;
    };
    for (int e = threadIdx.x; e < nq_keep * G; e += blockDim.x) {
      const float* r = row(e / G, e % G);
      float n2 = 0.f;
      for (int x = 0; x < d; ++x) n2 += r[x] * r[x];
      inv[e] = c.dot ? 1.0f : 1.0f / fmaxf(sqrtf(n2), kEps);
    }
    __syncthreads();
    const float inv_g = 1.0f / static_cast<float>(G);
    for (int e = threadIdx.x; e < nq_keep * d; e += blockDim.x) {
      const int n = e / d, x = e - n * d;
      float acc = 0.f;
      for (int g = 0; g < G; ++g) acc += row(n, g)[x] * inv[n * G + g];
      sq[e] = acc * inv_g;
    }
  }
  __syncthreads();
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= c.t_past) return;
  const float* kr = static_cast<const float*>(c.k) + (static_cast<size_t>(bj) * c.kv_cap + t) * d;
  float n2 = 0.f;
  for (int e = 0; e < d; ++e) n2 += kr[e] * kr[e];
  float m = -INFINITY;
  for (int n = 0; n < nq_keep; ++n) {
    float dot = 0.f;
    for (int e = 0; e < d; ++e) dot += sq[n * d + e] * kr[e];
    m = fmaxf(m, dot);
  }
  c.s_agg[static_cast<size_t>(bj) * c.t_past + t] = c.dot ? m : m / fmaxf(sqrtf(n2), kEps);
}

template <int D, int NQB, int STAGES, int GB>
void launch_variant(const ScoreArgs& a, bool fp8, bool dot, dim3 grid, hipStream_t st) {
  const dim3 block(64 * kScoreWaves);
  if (!fp8 && !dot)
    hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES, true, false, false, GB>), grid, block, 0, st, a);
  else if (!fp8)
    hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES, true, false, true, GB>), grid, block, 0, st, a);
  else if (!dot)
    hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES, true, true, false, GB>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES, true, true, true, GB>), grid, block, 0, st, a);
}

// Heads per batch of kept-row loads: every head of groups up to 8 in the
// first batch (the one issued ahead of the key blocks).
template <int D, int NQB, int STAGES>
void launch_grid(const ScoreArgs& a, bool fp8, bool dot, dim3 grid, hipStream_t st) {
  if (a.q_group)
    hipLaunchKernelGGL((kvscore_bf16_kernel<D, NQB, STAGES, false, false, false, 1>), grid,
                       dim3(64 * kScoreWaves), 0, st, a);
  else if (a.group <= 4)
    launch_variant<D, NQB, STAGES, 4>(a, fp8, dot, grid, st);
  else
    launch_variant<D, NQB, STAGES, 8>(a, fp8, dot, grid, st);
}

template <int D, int NQB>
void launch_bf16(const ScoreCall& c, hipStream_t st) {
  const int bnkv = c.b * c.nkv;
  ScoreArgs a;
  a.q_group = c.q_group;
  a.q = static_cast<const uint16_t*>(c.q);
  a.q_idx = c.q_idx;
  a.q_kept = static_cast<const uint16_t*>(c.q_kept);
  a.k = c.k;
  a.s_agg = c.s_agg;
  a.hist = c.hist;
  a.conv_src = static_cast<const uint16_t*>(c.conv_src);
  a.conv_dst = c.conv_dst;
  a.conv_total = c.conv_src ? c.b * c.nkv * c.bcp * (c.d / 16) : 0;
  a.nkv = c.nkv;
  a.group = c.nq / c.nkv;
  a.bcp = c.bcp;
  a.t_past = c.t_past;
  a.kv_cap = c.kv_cap;
  a.nq_keep = c.nq_keep;
  a.blocks_per_bj = (c.t_past + kBlock - 1) / kBlock;
  // about as many waves as are resident (two per SIMD where the registers
  // allow, else one), each streaming its share of blocks
  constexpr long long kResident = 1024LL * score_waves_per_simd<D, NQB>();
  const long long total = static_cast<long long>(a.blocks_per_bj) * bnkv;
  long long bpw = (total + kResident - 1) / kResident;
  if (bpw < 2) bpw = 2;
  if (bpw > a.blocks_per_bj) bpw = a.blocks_per_bj;
  const long long waves_per_bj = (a.blocks_per_bj + bpw - 1) / bpw;
  a.wgs_per_bj = static_cast<int>((waves_per_bj + kScoreWaves - 1) / kScoreWaves);
  const dim3 grid(a.wgs_per_bj * bnkv);
  // Blocks kept in flight per wave.  A wave with few blocks to score (short
  // rows) does better with a shallower ring (measured at d = 128: 3 for up to
  // 4 blocks per wave, 4 beyond).
  const bool shallow = D == 128 && NQB == 1 && bpw <= 4;
  if (c.read_sink) {
    u32x4* sink = static_cast<u32x4*>(c.read_sink);
    if (shallow && c.k_e4m3) hipLaunchKernelGGL((read_keys_kernel<D, 3, true>), grid, dim3(64 * kScoreWaves), 0, st, a, sink);
    else if (shallow) hipLaunchKernelGGL((read_keys_kernel<D, 3, false>), grid, dim3(64 * kScoreWaves), 0, st, a, sink);
    else if (c.k_e4m3) hipLaunchKernelGGL((read_keys_kernel<D, 4, true>), grid, dim3(64 * kScoreWaves), 0, st, a, sink);
    else hipLaunchKernelGGL((read_keys_kernel<D, 4, false>), grid, dim3(64 * kScoreWaves), 0, st, a, sink);
    return;
  }
  if (shallow) launch_grid<D, NQB, 3>(a, c.k_e4m3, c.dot, grid, st);
  else launch_grid<D, NQB, 4>(a, c.k_e4m3, c.dot, grid, st);
}

}  // namespace

size_t kvscore_f32_lds_bytes(int d, int nq_keep, int group) {
  return sizeof(float) * (static_cast<size_t>(nq_keep) * d + static_cast<size_t>(nq_keep) * group);
}

hipError_t launch_kvscore(const ScoreCall& c, hipStream_t st) {
  const int bnkv = c.b * c.nkv;
  if (c.t_past == 0) return hipSuccess;
  if (!c.bf16) {
    dim3 grid((c.t_past + 255) / 256, bnkv);
    const size_t lds = c.q_group ? sizeof(float) * c.nq_keep * c.d
                                 : kvscore_f32_lds_bytes(c.d, c.nq_keep, c.nq / c.nkv);
    hipLaunchKernelGGL(kvscore_f32_kernel, grid, dim3(256), lds, st, c);
    return hipGetLastError();
  }
  const int nqb = (c.nq_keep + 31) / 32;
  if (c.d == 128 && nqb == 1) launch_bf16<128, 1>(c, st);
  else if (c.d == 128 && nqb == 2) launch_bf16<128, 2>(c, st);
  else if (c.d == 64 && nqb == 1) launch_bf16<64, 1>(c, st);
  else if (c.d == 64 && nqb == 2) launch_bf16<64, 2>(c, st);
  else if (c.d == 256 && nqb == 1) launch_bf16<256, 1>(c, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace qk
