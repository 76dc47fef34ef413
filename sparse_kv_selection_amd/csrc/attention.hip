// Attention of a chunk over a set of past keys plus the chunk itself.
//
// QUOKA write-up, section 4.2 question 3: the selected KV is the KV input of a
// flash-style attention with the causal mask disabled over it.  Every chunk
// query sees all selected past keys; chunk query i also sees chunk keys u <= i
// (bottom-right aligned causal).  The dense reference path is the same kernel
// with every past key.
//
// bf16 kernel (gfx950 matrix cores, 32x32x16 bf16 tiles):
//   * GQA packing: the G query heads of one KV head are one matrix of G*bcp
//     rows, row r = query position r / G of head r % G (position-major, so a
//     row block spans few positions and causal chunk tiles can be skipped);
//   * a workgroup of WAVES waves owns WAVES * NB * 32 rows and walks one split
//     of the key range in tiles of 64 keys; tiles are fetched one ahead into
//     registers with 16-byte loads (rows through the index list when the
//     selection is not gathered), then stored to LDS: K row-major with a
//     16-byte row pad, V transposed (d-major) with the keys of each 16-key
//     group permuted so that one 16-byte LDS read yields a matrix-core operand;
//   * S^T = K Q^T: keys are the matrix rows, queries the columns, so every
//     softmax statistic of a query lives in one lane pair (lane l and l ^ 32);
//   * online softmax in base 2 with the scale folded into one multiply;
//     probabilities are rounded to bf16 and O^T = V^T P^T accumulates in fp32,
//     again one query per lane column, so the rescale is a per-lane multiply;
//   * key splits write normalised fp32 partials and a log-sum-exp; a combine
//     kernel merges them.
// fp32 kernel: one thread per query row, fp32 throughout (small workloads).
#include <math.h>

#include <type_traits>

#include "qk_device.h"
#include "qk_internal.h"

namespace qk {
namespace {

struct AttnParams {
  const uint16_t* q;
  const uint16_t* pk;
  const uint16_t* pv;
  long long past_bj_rows;
  const int32_t* idx;
  int ld_idx;
  const int32_t* sel_len;
  int n_past;
  const uint16_t* k;
  const uint16_t* v;
  int kv_cap, t_past;
  uint16_t* out;
  float* lse;
  float* part_o;
  float* part_lse;
  int b, nq, nkv, G, bcp;
  int n_qtiles, n_split;
  float scale_log2;
};

constexpr int kKeyTile = 64;

template <int D, int NB, int WAVES, int OCC>
__global__ __launch_bounds__(64 * WAVES, OCC) void attn_bf16_kernel(AttnParams p) {
  constexpr int NT = 64 * WAVES;
  constexpr int ROWS = WAVES * NB * 32;
  constexpr int KSTR = D + 8;          // sK row stride, elements
  constexpr int VSTR = kKeyTile + 8;   // sVT row stride, elements
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int KUNITS = kKeyTile * CH;
  constexpr int VUNITS = 16 * CH;      // units of 4 rows x 16 bytes
  constexpr int KPER = (KUNITS + NT - 1) / NT;
  constexpr int VPER = (VUNITS + NT - 1) / NT;
  constexpr bool kPrefetch = true;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kKeyTile * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t sVT[D * VSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int L = xcd_swizzle(blockIdx.x, gridDim.x);
  const int qtile = L % p.n_qtiles;
  const int rest = L / p.n_qtiles;
  const int split = rest % p.n_split;
  const int bj = rest / p.n_split;
  const int b = bj / p.nkv, j = bj % p.nkv;
  const int G = p.G, bcp = p.bcp;
  const int M = G * bcp;

  // past rows available: the index list length, or the rows of the past buffer
  const int past_cap = p.idx ? p.ld_idx : static_cast<int>(p.past_bj_rows);
  // wave-uniform (readfirstlane): tile classification below branches on it
  const int n_past =
      __builtin_amdgcn_readfirstlane(min(p.sel_len ? p.sel_len[bj] : p.n_past, past_cap));
  const int past_tiles = (n_past + kKeyTile - 1) / kKeyTile;
  // splits are balanced over this (b, KV head)'s own selection length
  const int split_tiles = (past_tiles + p.n_split - 1) / p.n_split;
  const int pt0 = split * split_tiles;
  const int pt1 = min(pt0 + split_tiles, past_tiles);
  const int npt = pt1 > pt0 ? pt1 - pt0 : 0;
  const int row0 = qtile * ROWS;
  const int i_max = (min(row0 + ROWS, M) - 1) / G;
  const bool last = split == p.n_split - 1;
  const int nct = last ? i_max / kKeyTile + 1 : 0;
  const int n_tiles = npt + nct;

  const uint16_t* pk = p.pk + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* pv = p.pv + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* ck = p.k + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const uint16_t* cv = p.v + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const int32_t* idx = p.idx ? p.idx + static_cast<size_t>(bj) * p.ld_idx : nullptr;
  const int row_hi = static_cast<int>(p.past_bj_rows) - 1;

  // Element offset of tile key r.  Keys past the end of the range are clamped
  // onto a valid row: they are masked to -inf, so their weight is exactly 0.
  auto key_off = [&](int t, int r) -> int {
    if (t < npt) {
      const int kk = min((pt0 + t) * kKeyTile + r, n_past - 1);
      const int row = idx ? min(max(idx[kk], 0), row_hi) : kk;
      return row * D;
    }
    return min((t - npt) * kKeyTile + r, bcp - 1) * D;
  };

  // query fragments: lane (col, half) holds row col of block nb, d slots 16s + 8half + [0,8)
  bf16x8 qf[NB][D / 16];
  int iq[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int r = row0 + (wave * NB + nb) * 32 + col;
    const bool valid = r < M;
    const int i = r / G, g = r - (r / G) * G;
    iq[nb] = i;
    const uint16_t* qp = p.q + ((static_cast<size_t>(b) * p.nq + j * G + g) * bcp + i) * D;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[nb][s] = valid ? as_bf16x8(ld16(qp + 16 * s + 8 * half)) : bf16x8{};
  }

  // a wave whose rows are all padding only helps with the tile loads
  const bool wave_active = row0 + wave * NB * 32 < M;

  f32x16 acc[NB][D / 32];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[nb][db] = f32x16{};
  }

  // Tile loads.  Offsets for tile t+1 are computed (index loads) while tile t
  // is in flight, so index and data loads never wait on each other.
  int koff[KPER], voff[VPER][4];
  u32x4 kreg[KPER];
  u32x4 vreg[VPER][4];
  auto offsets = [&](int t) {
#pragma unroll
    for (int pp = 0; pp < KPER; ++pp) {
      const int u = tid + pp * NT;
      if (KUNITS % NT == 0 || u < KUNITS) koff[pp] = key_off(t, u / CH) + 8 * (u % CH);
    }
#pragma unroll
    for (int pp = 0; pp < VPER; ++pp) {
      const int u = tid + pp * NT;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int sg = u & 15, c = u >> 4;
        const int q4 = sg & 3;
        const int kb4 = (sg >> 2) * 16 + (q4 & 1) * 8 + (q4 >> 1) * 4;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) voff[pp][e4] = key_off(t, kb4 + e4) + 8 * c;
      }
    }
  };
  auto fetch = [&](int t) {
    const uint16_t* kbase = t < npt ? pk : ck;
    const uint16_t* vbase = t < npt ? pv : cv;
#pragma unroll
    for (int pp = 0; pp < KPER; ++pp) {
      const int u = tid + pp * NT;
      if (KUNITS % NT == 0 || u < KUNITS) kreg[pp] = ld16(kbase + koff[pp]);
    }
#pragma unroll
    for (int pp = 0; pp < VPER; ++pp) {
      const int u = tid + pp * NT;
      if (VUNITS % NT == 0 || u < VUNITS) {
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) vreg[pp][e4] = ld16(vbase + voff[pp][e4]);
      }
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int pp = 0; pp < KPER; ++pp) {
      const int u = tid + pp * NT;
      if (KUNITS % NT == 0 || u < KUNITS) {
        const int r = u / CH, c = u - (u / CH) * CH;
        st16(sK + r * KSTR + 8 * c, kreg[pp]);
      }
    }
#pragma unroll
    for (int pp = 0; pp < VPER; ++pp) {
      const int u = tid + pp * NT;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int sg = u & 15, c = u >> 4;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t d0, d1;
          if ((e & 1) == 0) {
            d0 = (vreg[pp][0][w] & 0xffffu) | (vreg[pp][1][w] << 16);
            d1 = (vreg[pp][2][w] & 0xffffu) | (vreg[pp][3][w] << 16);
          } else {
            d0 = (vreg[pp][0][w] >> 16) | (vreg[pp][1][w] & 0xffff0000u);
            d1 = (vreg[pp][2][w] >> 16) | (vreg[pp][3][w] & 0xffff0000u);
          }
          uint2 pr;
          pr.x = d0;
          pr.y = d1;
          *reinterpret_cast<uint2*>(sVT + (8 * c + e) * VSTR + 4 * sg) = pr;
        }
      }
    }
  };

  const float c2 = p.scale_log2;
  if (n_tiles > 0) {
    offsets(0);
    fetch(0);
    if (n_tiles > 1) offsets(1);
  }
  auto tile = [&](int t, auto masked_tag) {
    constexpr bool kMasked = decltype(masked_tag)::value;
    __syncthreads();
    store();
    __syncthreads();
    if (kPrefetch && t + 1 < n_tiles) {
      fetch(t + 1);
      if (t + 2 < n_tiles) offsets(t + 2);
    }
    if (!wave_active) return;

    // S^T = K Q^T for 64 keys x (NB * 32) queries
    f32x16 S[2][NB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[kb][nb] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = as_bf16x8(
            *reinterpret_cast<const u32x4*>(sK + (kb * 32 + col) * KSTR + 16 * s + 8 * half));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) S[kb][nb] = mfma32(a, qf[nb][s], S[kb][nb]);
      }
    }

    // mask (boundary and chunk tiles only), online softmax in base 2
    const bool is_chunk = t >= npt;
    const int kbase = is_chunk ? (t - npt) * kKeyTile : (pt0 + t) * kKeyTile;
    bf16x8 P[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if constexpr (kMasked) {
          const int klimit = is_chunk ? min(bcp, iq[nb] + 1) : n_past;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (kbase + kb * 32 + acc_row(r, half) >= klimit) S[kb][nb][r] = -INFINITY;
        }
        float mx = S[0][nb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][nb][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * c2;
        const float m_new = fmaxf(m_run[nb], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run[nb] - m_use);
        m_run[nb] = m_new;
        float ps = 0.f;
#pragma unroll
        for (int g16 = 0; g16 < 4; ++g16) {
          const int kb = g16 >> 1, r0 = 8 * (g16 & 1);
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][nb][r0 + 2 * e], c2, -m_use));
            const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][nb][r0 + 2 * e + 1], c2, -m_use));
            ps += x0 + x1;
            w[e] = pack_bf16x2(x0, x1);
          }
          P[nb][g16] = as_bf16x8(w);
        }
        l_run[nb] = l_run[nb] * alpha + ps;
        if (__any(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) acc[nb][db] *= alpha;
        }
      }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int g16 = 0; g16 < 4; ++g16) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            sVT + (db * 32 + col) * VSTR + 16 * g16 + 8 * half));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb][db] = mfma32(a, P[nb][g16], acc[nb][db]);
      }
    }
  };
  // leading tiles wholly inside the past range need no mask
  const int n_full = min(max(n_past / kKeyTile - pt0, 0), npt);
  for (int t = 0; t < n_full; ++t) tile(t, std::false_type{});
  for (int t = n_full; t < n_tiles; ++t) tile(t, std::true_type{});

  // epilogue: lane (col, half) holds query col, d rows db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = l_run[nb] + __shfl_xor(l_run[nb], 32);
    const int r = row0 + (wave * NB + nb) * 32 + col;
    if (r >= M) continue;
    const int i = iq[nb], g = r - (r / G) * G;
    const size_t orow = (static_cast<size_t>(b) * p.nq + j * G + g) * bcp + i;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? m_run[nb] + log2f(lt) : -INFINITY;
    if (p.n_split == 1) {
      uint16_t* op = p.out + orow * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * half;
          uint2 w;
          w.x = pack_bf16x2(acc[nb][db][4 * r4] * inv, acc[nb][db][4 * r4 + 1] * inv);
          w.y = pack_bf16x2(acc[nb][db][4 * r4 + 2] * inv, acc[nb][db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(op + d0) = w;
        }
      if (p.lse && half == 0) p.lse[orow] = lse2 * kLn2;
    } else {
      const size_t rows_total = static_cast<size_t>(p.b) * p.nq * bcp;
      float* op = p.part_o + (static_cast<size_t>(split) * rows_total + orow) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = db * 32 + 8 * r4 + 4 * half;
          f32x4 w = {acc[nb][db][4 * r4] * inv, acc[nb][db][4 * r4 + 1] * inv,
                     acc[nb][db][4 * r4 + 2] * inv, acc[nb][db][4 * r4 + 3] * inv};
          *reinterpret_cast<f32x4*>(op + d0) = w;
        }
      if (half == 0) p.part_lse[static_cast<size_t>(split) * rows_total + orow] = lse2;
    }
  }
}

// Merge key-split partials, one wave per output row:
//   O = sum_s w_s O_s / sum_s w_s,  w_s = 2^(lse_s - max_s lse_s)
// Lane s < n_split (<= 64) holds split s's log-sum-exp; every lane then loads
// its d-slots of all splits at once.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse, int n_split,
                                                           long long rows) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  const long long row = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float ls = lane < n_split ? part_lse[lane * rows + row] : -INFINITY;
  const float mx = wave_max(ls);
  const float w = (ls == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ls - mx);
  const float wsum = wave_sum(w);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  constexpr int kBatch = 16;
  for (int s0 = 0; s0 < n_split; s0 += kBatch) {
    float x[kBatch][PER];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sidx = min(s0 + u, n_split - 1);
      const float* src = part_o + (sidx * rows + row) * D + lane;
#pragma unroll
      for (int e = 0; e < PER; ++e) x[u][e] = src[64 * e];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wu = s0 + u < n_split ? __shfl(w, s0 + u) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += wu * x[u][e];
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  uint16_t* op = out + row * D + lane;
#pragma unroll
  for (int e = 0; e < PER; ++e) op[64 * e] = f32_to_bf16(acc[e] * inv);
  if (lse && lane == 0) lse[row] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
}

// fp32 path: one thread per packed query row, natural-base online softmax.
template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ pk, const float* __restrict__ pv,
    long long past_bj_rows, const int32_t* __restrict__ idx, int ld_idx,
    const int32_t* __restrict__ sel_len, int n_past_fixed, const float* __restrict__ k,
    const float* __restrict__ v, int kv_cap, int t_past, float* __restrict__ out,
    float* __restrict__ lse, int nq, int nkv, int bcp, float scale) {
  const int bj = blockIdx.y;
  const int b = bj / nkv, j = bj % nkv, G = nq / nkv;
  const int r = blockIdx.x * 64 + threadIdx.x;
  if (r >= G * bcp) return;
  const int i = r / G, g = r % G;
  const size_t orow = (static_cast<size_t>(b) * nq + j * G + g) * bcp + i;
  float qv[D], acc[D];
  for (int e = 0; e < D; ++e) { qv[e] = q[orow * D + e]; acc[e] = 0.f; }
  float m = -INFINITY, l = 0.f;
  auto visit = [&](const float* kr, const float* vr) {
    float dot = 0.f;
    for (int e = 0; e < D; ++e) dot += qv[e] * kr[e];
    const float x = dot * scale;
    const float m_new = fmaxf(m, x);
    const float alpha = expf(m - m_new);
    const float pw = expf(x - m_new);
    l = l * alpha + pw;
    for (int e = 0; e < D; ++e) acc[e] = acc[e] * alpha + pw * vr[e];
    m = m_new;
  };
  const int past_cap = idx ? ld_idx : static_cast<int>(past_bj_rows);
  const int n_past = min(sel_len ? sel_len[bj] : n_past_fixed, past_cap);
  const float* pkb = pk + static_cast<size_t>(bj) * past_bj_rows * D;
  const float* pvb = pv + static_cast<size_t>(bj) * past_bj_rows * D;
  for (int s = 0; s < n_past; ++s) {
    const int row = idx ? min(max(idx[static_cast<size_t>(bj) * ld_idx + s], 0),
                              static_cast<int>(past_bj_rows) - 1)
                        : s;
    visit(pkb + static_cast<size_t>(row) * D, pvb + static_cast<size_t>(row) * D);
  }
  const size_t cb = (static_cast<size_t>(bj) * kv_cap + t_past) * D;
  for (int u = 0; u <= i; ++u) visit(k + cb + static_cast<size_t>(u) * D, v + cb + static_cast<size_t>(u) * D);
  const float inv = 1.f / l;
  for (int e = 0; e < D; ++e) out[orow * D + e] = acc[e] * inv;
  if (lse) lse[orow] = m + logf(l);
}

struct Plan {
  int waves, nb, rows, n_qtiles, n_split;
};

Plan make_plan(int b, int nq, int nkv, int d, int bcp, int n_past_max) {
  Plan pl{};
  const int G = nq / nkv;
  const int M = G * bcp;
  pl.waves = 4;
  pl.nb = 1;
  pl.rows = pl.waves * pl.nb * 32;
  pl.n_qtiles = (M + pl.rows - 1) / pl.rows;
  const int past_tiles = (n_past_max + kKeyTile - 1) / kKeyTile;
  const long long base = static_cast<long long>(pl.n_qtiles) * b * nkv;
  // key splits fill the resident slots (256 CUs x workgroups per CU) without
  // spilling into a second, mostly idle round; at least 4 key tiles per split
  const long long slots = 256LL * (d == 256 ? 1 : 2);
  long long ns = slots / base;
  const long long max_split = past_tiles / 4 > 1 ? past_tiles / 4 : 1;
  if (ns > max_split) ns = max_split;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  pl.n_split = static_cast<int>(ns);
  return pl;
}

template <int D, int NB, int WAVES, int OCC>
hipError_t run_bf16(const AttnParams& p, int grid, hipStream_t st) {
  hipLaunchKernelGGL((attn_bf16_kernel<D, NB, WAVES, OCC>), dim3(grid), dim3(64 * WAVES), 0, st, p);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(bool bf16, int b, int nq, int nkv, int d, int bcp, int n_past_max) {
  if (!bf16) return 0;
  const Plan pl = make_plan(b, nq, nkv, d, bcp, n_past_max);
  if (pl.n_split <= 1) return 0;
  const size_t rows = static_cast<size_t>(b) * nq * bcp;
  return static_cast<size_t>(pl.n_split) * rows * (d + 1) * sizeof(float);
}

hipError_t launch_attention(const AttnCall& c, hipStream_t st) {
  const int G = c.nq / c.nkv;
  const float scale = c.scale > 0.f ? c.scale : 1.0f / sqrtf(static_cast<float>(c.d));
  if (!c.bf16) {
    dim3 grid((G * c.bcp + 63) / 64, c.b * c.nkv);
#define QK_F32_ATTN(DD)                                                                           \
  hipLaunchKernelGGL(attn_f32_kernel<DD>, grid, dim3(64), 0, st, static_cast<const float*>(c.q), \
                     static_cast<const float*>(c.pk), static_cast<const float*>(c.pv),           \
                     c.past_bj_rows, c.idx, c.ld_idx, c.sel_len, c.n_past,                       \
                     static_cast<const float*>(c.k), static_cast<const float*>(c.v), c.kv_cap,    \
                     c.t_past, static_cast<float*>(c.out), c.lse, c.nq, c.nkv, c.bcp, scale)
    if (c.d == 64) QK_F32_ATTN(64);
    else if (c.d == 128) QK_F32_ATTN(128);
    else return hipErrorInvalidValue;
#undef QK_F32_ATTN
    return hipGetLastError();
  }
  const Plan pl = make_plan(c.b, c.nq, c.nkv, c.d, c.bcp, c.n_past);
  AttnParams p{};
  p.q = static_cast<const uint16_t*>(c.q);
  p.pk = static_cast<const uint16_t*>(c.pk);
  p.pv = static_cast<const uint16_t*>(c.pv);
  p.past_bj_rows = c.past_bj_rows;
  p.idx = c.idx;
  p.ld_idx = c.ld_idx;
  p.sel_len = c.sel_len;
  p.n_past = c.n_past;
  p.k = static_cast<const uint16_t*>(c.k);
  p.v = static_cast<const uint16_t*>(c.v);
  p.kv_cap = c.kv_cap;
  p.t_past = c.t_past;
  p.out = static_cast<uint16_t*>(c.out);
  p.lse = c.lse;
  p.b = c.b;
  p.nq = c.nq;
  p.nkv = c.nkv;
  p.G = G;
  p.bcp = c.bcp;
  p.n_qtiles = pl.n_qtiles;
  p.n_split = pl.n_split;
  p.scale_log2 = scale * kLog2e;
  const size_t rows = static_cast<size_t>(c.b) * c.nq * c.bcp;
  if (pl.n_split > 1) {
    p.part_o = static_cast<float*>(c.ws);
    p.part_lse = p.part_o + static_cast<size_t>(pl.n_split) * rows * c.d;
  }
  const int grid = pl.n_qtiles * c.b * c.nkv * pl.n_split;
  hipError_t e;
  if (c.d == 128) e = run_bf16<128, 1, 4, 2>(p, grid, st);
  else if (c.d == 64) e = run_bf16<64, 1, 4, 2>(p, grid, st);
  else if (c.d == 256) e = run_bf16<256, 1, 4, 1>(p, grid, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || pl.n_split == 1) return e;
  const dim3 cgrid(static_cast<unsigned>((rows + 3) / 4)), cblock(256);
  if (c.d == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, cblock, 0, st, p.part_o, p.part_lse,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  else if (c.d == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, cblock, 0, st, p.part_o, p.part_lse,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  else
    hipLaunchKernelGGL(attn_combine_kernel<256>, cgrid, cblock, 0, st, p.part_o, p.part_lse,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  return hipGetLastError();
}

}  // namespace qk
