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
//   * a workgroup of WAVES waves owns WAVES * NB * 32 rows and walks one split of
//     the key range in tiles of 64 keys; each tile is copied global -> LDS by
//     16-byte direct loads (rows through the index list when the selection is
//     not gathered; index entries fetched one tile ahead), with the 16-byte
//     chunks of each row XOR-swizzled so that the matrix-core reads spread
//     over all banks; two LDS stages, so tile t + 1 streams in while tile t is
//     computed; V stays row-major and its transposed operand comes from the
//     LDS transpose read;
//   * S^T = K Q^T: keys are the matrix rows, queries the columns, so every
//     softmax statistic of a query lives in one lane pair (lane l and l ^ 32);
//   * online softmax in base 2 with the scale folded into one multiply;
//     probabilities are rounded to bf16 and O^T = V^T P^T accumulates in fp32,
//     again one query per lane column, so the rescale is a per-lane multiply;
//   * key splits write normalised partials (fp16, scaled per row) and a
//     log-sum-exp; a combine kernel merges them.
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
  uint32_t* part_o;   // split partials, fp16 pairs scaled to [-1, 1]
  float2* part_ls;    // per (split, row): (base-2 log-sum-exp, scale)
  int b, nq, nkv, G, bcp;
  int n_qtiles, n_split;
  float scale_log2;
};

constexpr int kKeyTile = 64;
constexpr float kSlack = 8.f;  // lazy-rescale slack, base-2 exponent units

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS; the wave's 64 lanes
// fill 1 KiB at lds (wave-uniform) in lane order.
__device__ __forceinline__ void lds_load16(const uint16_t* g, uint16_t* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds, 16, 0, 0);
}
// Two transposed 8-byte LDS reads (rows p and p + 8 * stride) as one 8-slot
// matrix-core operand.
__device__ __forceinline__ bf16x8 lds_read_tr_pair(const uint16_t* p, int stride) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * stride));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// 16-byte chunk swizzles of the K and V tiles in LDS.  Chunk c of tile row r
// is stored at chunk position c ^ swz(r); the functions spread the matrix-core
// reads over all LDS banks (row reads of K, transposed reads of V).
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3);
}

// Sum of the eight bf16 probabilities of one matrix-core operand, added to
// acc in fp32: the softmax denominator is formed from the same rounded
// weights that enter the value products.
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 one = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// Epilogue of one 32-row block.  Lane (col, half) holds query row r (of the
// packed G * bcp rows, query position i) and the d rows db * 32 + 8 * (rr / 4)
// + 4 * half + rr % 4 of O^T in acc[db][rr]; l_run is its half of the
// denominator.  With one key split the row is normalised and written (bf16)
// with its log-sum-exp; otherwise the normalised partial (fp16, scaled by the
// row's largest magnitude) and (base-2 log-sum-exp, scale) go to the
// workspace.  Called by whole waves (the two lanes of a row exchange values).
template <int D>
__device__ __forceinline__ void finish_rows(const AttnParams& p, const f32x16 (&acc)[D / 32],
                                            float m_run, float l_run, int r, int M, int i, int b,
                                            int j, int split) {
  const int half = (threadIdx.x & 63) >> 5;
  const int G = p.G, bcp = p.bcp;
  const float lt = l_run + __shfl_xor(l_run, 32);
  if (r >= M) return;
  const int g = r - (r / G) * G;
  const size_t orow = (static_cast<size_t>(b) * p.nq + j * G + g) * bcp + i;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = lt > 0.f ? m_run + log2f(lt) : -INFINITY;
  if (p.n_split == 1) {
    uint16_t* op = p.out + orow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * half;
        uint2 w;
        w.x = pack_bf16x2(acc[db][4 * r4] * inv, acc[db][4 * r4 + 1] * inv);
        w.y = pack_bf16x2(acc[db][4 * r4 + 2] * inv, acc[db][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (p.lse && half == 0) p.lse[orow] = lse2 * kLn2;
  } else {
    // normalised partial, scaled by its row's largest magnitude M so that
    // fp16 keeps a relative precision of 2^-11 of M whatever the range of V;
    // M and the log-sum-exp stay fp32
    const size_t rows_total = static_cast<size_t>(p.b) * p.nq * bcp;
    float mag = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mag = fmaxf(mag, fabsf(acc[db][rr]));
    mag = fmaxf(mag, __shfl_xor(mag, 32)) * inv;
    const float sc = mag > 0.f ? inv / mag : 0.f;
    uint32_t* op = p.part_o + (static_cast<size_t>(split) * rows_total + orow) * (D / 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = db * 32 + 8 * r4 + 4 * half;
        uint2 w;
        w.x = pack_f16x2(acc[db][4 * r4] * sc, acc[db][4 * r4 + 1] * sc);
        w.y = pack_f16x2(acc[db][4 * r4 + 2] * sc, acc[db][4 * r4 + 3] * sc);
        *reinterpret_cast<uint2*>(op + d0 / 2) = w;
      }
    if (half == 0) p.part_ls[static_cast<size_t>(split) * rows_total + orow] = float2{lse2, mag};
  }
}

template <int D, int NB, int WAVES, int OCC, bool IDX>
__global__ __launch_bounds__(64 * WAVES, OCC) void attn_bf16_kernel(AttnParams p) {
  constexpr int ROWS = WAVES * NB * 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int RPI = 64 / CH;                // tile rows per wave-wide 16-byte load
  constexpr int IPW = kKeyTile / (RPI * WAVES);  // such loads per wave per matrix
  constexpr int TILE = kKeyTile * D;          // elements per K (or V) tile
  static_assert(IPW >= 1 && IPW * RPI * WAVES == kKeyTile, "tile split");
  // two stages (double buffer), separate objects so that the compiler sees
  // that reads of one stage do not alias the loads in flight into the other
  __shared__ __attribute__((aligned(16))) uint16_t sK0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV0[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sK1[TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV1[TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int past_cap = IDX ? p.ld_idx : static_cast<int>(p.past_bj_rows);
  // wave-uniform (readfirstlane): tile classification below branches on it
  const int n_past =
      __builtin_amdgcn_readfirstlane(min(p.sel_len ? p.sel_len[bj] : p.n_past, past_cap));
  const int past_tiles = (n_past + kKeyTile - 1) / kKeyTile;
  const int row0 = qtile * ROWS;
  const int i_max = (min(row0 + ROWS, M) - 1) / G;
  // The key range of this row tile is the selected past tiles followed by the
  // chunk tiles its queries reach (causal); the splits divide that combined
  // range evenly (sizes differ by at most one tile), so the chunk tiles do not
  // pile onto one split.
  const int chunk_tiles = i_max / kKeyTile + 1;
  const int total_tiles = past_tiles + chunk_tiles;
  const int g0 = static_cast<int>(static_cast<long long>(split) * total_tiles / p.n_split);
  const int g1 = static_cast<int>(static_cast<long long>(split + 1) * total_tiles / p.n_split);
  const int pt0 = g0;                                   // first past tile
  const int npt = max(0, min(g1, past_tiles) - g0);     // past tiles of this split
  const int c0 = max(g0, past_tiles) - past_tiles;      // first chunk tile
  const int nct = max(0, g1 - max(g0, past_tiles));     // chunk tiles of this split
  const int n_tiles = npt + nct;

  const uint16_t* pk = p.pk + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* pv = p.pv + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* ck = p.k + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const uint16_t* cv = p.v + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const int32_t* idx = IDX ? p.idx + static_cast<size_t>(bj) * p.ld_idx : nullptr;
  const int row_hi = static_cast<int>(p.past_bj_rows) - 1;

  // ---- tile loads: global -> LDS directly, 16 bytes per lane ----
  // Load i of this wave fills tile rows (wave * IPW + i) * RPI + [0, RPI); lane
  // l writes chunk position l % CH of row r = ... + l / CH and so fetches the
  // global chunk (l % CH) ^ swz(r) of that key's row.
  int trow[IPW];     // tile row of each load of this lane
  int kchunk[IPW];   // byte offset of the fetched chunk in its row, K
  int vchunk[IPW];   // byte offset of the fetched chunk in its row, V
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * RPI + lane / CH;
    trow[i] = r;
    kchunk[i] = 16 * ((lane % CH) ^ swz_k<D>(r));
    vchunk[i] = 16 * ((lane % CH) ^ swz_v<D>(r));
  }
  // Key rows of a tile.  Keys past the end of the range are clamped onto a
  // valid row; they are masked to -inf, so their weight is exactly 0.  Index
  // entries are loaded one tile ahead of the data loads that use them.
  int krow[IPW];
  auto rows_of = [&](int t, int* rr) {
    const int k0 = (pt0 + t) * kKeyTile;  // uniform
    if (t < npt && k0 + kKeyTile <= n_past) {  // uniform: a whole past tile, no clamp
      // entries at a wave-uniform base plus the lane's fixed row offset
      const int32_t* it = IDX ? idx + k0 : nullptr;
#pragma unroll
      for (int i = 0; i < IPW; ++i) rr[i] = IDX ? it[static_cast<uint32_t>(trow[i])] : k0 + trow[i];
    } else if (t < npt) {
#pragma unroll
      for (int i = 0; i < IPW; ++i) {
        const int kk = min(k0 + trow[i], n_past - 1);
        rr[i] = IDX ? idx[kk] : kk;
      }
    } else {
#pragma unroll
      for (int i = 0; i < IPW; ++i) rr[i] = min((c0 + t - npt) * kKeyTile + trow[i], bcp - 1);
    }
  };
  auto issue = [&](int t, uint16_t* dK, uint16_t* dV, const int* rr) {
    const bool past = t < npt;
    const uint16_t* kbase = past ? pk : ck;
    const uint16_t* vbase = past ? pv : cv;
    const int hi = past ? row_hi : bcp - 1;
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      // one 32-bit byte offset from a wave-uniform base (scalar-base loads)
      const uint32_t ro = static_cast<uint32_t>(min(max(rr[i], 0), hi)) * (2 * D);
      uint16_t* lk = dK + (wave * IPW + i) * 512;
      uint16_t* lv = dV + (wave * IPW + i) * 512;
      lds_load16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(kbase) +
                                                   (ro + static_cast<uint32_t>(kchunk[i]))),
                 lk);
      lds_load16(reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(vbase) +
                                                   (ro + static_cast<uint32_t>(vchunk[i]))),
                 lv);
    }
  };

  // The index entries of the first two tiles go out before the query loads:
  // loads retire in order, so the first tile's copy then waits for its own
  // indices only, while the query fragments are still in flight.
  int krow0[IPW];
  if (n_tiles > 0) {
    rows_of(0, krow0);
    if (n_tiles > 1) rows_of(1, krow);
  }

  // query fragments: lane (col, half) holds row col of block nb, d slots
  // 16s + 8half + [0,8); a wave owns NB independent blocks of 32 rows, whose
  // softmax and products the compiler can interleave
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

  // LDS read offsets (elements).  K: lane (col, half), step s reads row
  // kb*32 + col, chunk 2s + half -> position (2s) ^ fk with fk = half ^ swz.
  constexpr int NKA = D / 16 < 8 ? D / 16 : 8;
  int kofs[NKA];
  {
    const int fk = half ^ swz_k<D>(col);
#pragma unroll
    for (int s = 0; s < NKA; ++s) kofs[s] = col * D + 8 * ((2 * s) ^ fk);
  }
  // V (transposed reads, 16-lane groups): lane (g = lane/16, jl = lane%16)
  // addresses row 4*(g/2) + jl/4 (+16 g16 + 8 q), columns 32 db + 16 (g%2) +
  // 4 (jl%4) + [0,4); the hardware hands lane i of the group element i%4 of
  // group lane 4k + i/4 as its k-th value, i.e. keys 4*(g/2) + [0,4) (+8 q) of
  // column 32 db + 16 (g%2) + i: the B-operand key order of P below.
  int vofs[D / 32];
  {
    const int g = lane >> 4, jl = lane & 15, jj = jl >> 2;
    const int vr = 4 * (g >> 1) + jj;
    const int x = 2 * (g & 1) + ((jl & 3) >> 1);
    const int fv = swz_v<D>(vr);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      vofs[db] = vr * D + 8 * ((4 * db + x) ^ fv) + 4 * (jl & 1);
  }

  f32x16 acc[NB][D / 32];
  float m_run[NB], l_run[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) acc[nb][db] = f32x16{};
  }

  const float c2 = p.scale_log2;

  const int n_full = min(max(n_past / kKeyTile - pt0, 0), npt);
  auto compute = [&](int t, const uint16_t* cK, const uint16_t* cV) {
    // S^T = K Q^T for 64 keys x (NB * 32) queries
    f32x16 S[2][NB];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) S[kb][nb] = f32x16{};
    // K fragments are read one d-step ahead of the products that use them
    auto kfrag = [&](int s, int kb) {
      return as_bf16x8(*reinterpret_cast<const u32x4*>(cK + kb * 32 * D + kofs[s % NKA] +
                                                       128 * (s / NKA)));
    };
    bf16x8 ka0 = kfrag(0, 0), ka1 = kfrag(0, 1);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const bf16x8 c0 = ka0, c1 = ka1;
      if (s + 1 < D / 16) {
        ka0 = kfrag(s + 1, 0);
        ka1 = kfrag(s + 1, 1);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        S[0][nb] = mfma32(c0, qf[nb][s], S[0][nb]);
        S[1][nb] = mfma32(c1, qf[nb][s], S[1][nb]);
      }
    }
    const bool is_chunk = t >= npt;
    const int kbase = is_chunk ? (c0 + t - npt) * kKeyTile : (pt0 + t) * kKeyTile;
    if (t >= n_full) {  // uniform: boundary and chunk tiles only
      // key kbase + 32 kb + acc_row(r, half) is masked when it reaches the limit;
      // the lane's offset is folded into one bound, the rest are immediates
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int lim = (is_chunk ? min(bcp, iq[nb] + 1) : n_past) - kbase - 4 * half;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) S[kb][nb][r] = -INFINITY;
      }
    }
    // Lazy rescale: the reference maximum of a query only moves when a score
    // exceeds it by more than kSlack (base 2), so probabilities stay below
    // 2^kSlack and the accumulator is rescaled on few tiles; the softmax is
    // unchanged (numerator and denominator share the reference).  Both lanes
    // of a query (l and l ^ 32) take the same decision from the exchanged
    // maxima, so their halves of the key sum share one reference, and the
    // common case needs no exchange at all.
    bf16x8 P[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float mx = S[0][nb][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][nb][r]);
      mx *= c2;
      if (__any(mx > m_run[nb] + kSlack)) {
        const float mq = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = mq > m_run[nb] + kSlack ? mq : m_run[nb];
        const float alpha = m_run[nb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[nb] - m_new);
        m_run[nb] = m_new;
        l_run[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) acc[nb][db] *= alpha;
      }
      const float m_use = m_run[nb] == -INFINITY ? 0.f : m_run[nb];
      // P^T operand: lane half h, 16-key group g16, slot e <-> key
      // 16 g16 + 8 (e / 4) + 4 h + e % 4 (the accumulator row order of S^T)
      // the denominator sums the bf16 weights that the value products use
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int g16 = 0; g16 < 4; ++g16) {
        const int kb = g16 >> 1, r0 = 8 * (g16 & 1);
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][nb][r0 + 2 * e], c2, -m_use));
          const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][nb][r0 + 2 * e + 1], c2, -m_use));
          w[e] = pack_bf16x2(x0, x1);
        }
        P[nb][g16] = as_bf16x8(w);
        if (g16 & 1) ps1 = sum_bf16x8(P[nb][g16], ps1);
        else ps0 = sum_bf16x8(P[nb][g16], ps0);
      }
      l_run[nb] += ps0 + ps1;
    }
    // O^T += V^T P^T, the key groups in order so that the products of the
    // first half can start while the second half's exponentials run; V^T
    // operands come from transposed LDS reads, one product ahead, each used
    // for the NB row blocks
    auto vfrag = [&](int n) {  // key group n / (D / 32), d block n % (D / 32)
      return lds_read_tr_pair(cV + vofs[n % (D / 32)] + (n / (D / 32)) * 16 * D, D);
    };
    // The value products run at raised wave priority: while this wave feeds
    // the matrix cores its tile's vector work is done, and the other resident
    // wave's exponentials fill the gaps (measured: about 3 % faster than
    // raising it for the key products).
    __builtin_amdgcn_s_setprio(1);
    bf16x8 va = vfrag(0);
#pragma unroll
    for (int n = 0; n < D / 8; ++n) {
      const bf16x8 cur = va;
      if (n + 1 < D / 8) va = vfrag(n + 1);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb][n % (D / 32)] = mfma32(cur, P[nb][n / (D / 32)], acc[nb][n % (D / 32)]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Tile t lives in stage t & 1.  Iteration t: wait for its loads (own, then
  // everyone's via the barrier, which also retires all reads of tile t - 1),
  // start the loads of tile t + 1 into the other stage and the index loads of
  // tile t + 2, then compute tile t.
  if (n_tiles > 0) issue(0, sK0, sV0, krow0);
  auto step = [&](int t, uint16_t* cK, uint16_t* cV, uint16_t* nK, uint16_t* nV) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this lane's loads of tile t landed
    __syncthreads();
    if (t + 1 < n_tiles) {
      issue(t + 1, nK, nV, krow);
      if (t + 2 < n_tiles) rows_of(t + 2, krow);
    }
    if (wave_active) compute(t, cK, cV);
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, sK0, sV0, sK1, sV1);
    if (t + 1 < n_tiles) step(t + 1, sK1, sV1, sK0, sV0);
  }

  // epilogue: lane (col, half) holds query col, d rows db*32 + 8*(r/4) + 4*half + r%4
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    finish_rows<D>(p, acc[nb], m_run[nb], l_run[nb], row0 + (wave * NB + nb) * 32 + col, M, iq[nb],
                   b, j, split);
}

// Workgroup barrier without a memory fence.  __syncthreads() also waits for
// every load in flight; the ping-pong kernel keeps the tile copies of the
// next iteration in flight across its barriers and waits explicitly (vmcnt)
// for the ones the next tile needs.  The clobber keeps the compiler from
// moving memory accesses across the barrier.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// 16 bytes per lane from base + voff straight into LDS at lds_addr (uniform
// byte address; lane l fills lds_addr + 16 l), like lds_load16, issued so that
// the compiler does not treat the copy as a pending write to every LDS array:
// otherwise it waits for all copies in flight before each LDS read, and the
// kernel keeps copies for later tiles in flight while reading the current
// one.  The instruction writes no register; the kernel's explicit vmcnt waits
// before its barriers order the copies with their readers.
__device__ __forceinline__ void lds_load16_async(const void* base, uint32_t voff, uint32_t lds_addr) {
  // M0 holds the LDS address (bound by the operand constraint); the nop is
  // the wait state between writing M0 and an LDS DMA reading it
  asm volatile(
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(base), "{m0}"(lds_addr)
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  const lds_void* lp = (const lds_void*)p;
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lp));
}

// Ping-pong form for eight-wave workgroups at d = 128.
//
// Waves 0-3 and 4-7 are two groups with one wave of each on every SIMD (the
// waves of a workgroup are placed on the SIMDs in turn, so waves w and w + 4
// share one).  A key tile's work splits into a matrix block (the value
// products of the previous tile, then the key products of this tile) and a
// vector block (the online softmax of one tile).  Group 0 runs each tile as
// matrix block then softmax; group 1 runs the softmax of the previous tile
// then its matrix block, so on every SIMD one wave feeds the matrix core
// while the other computes exponentials.
//
// One barrier serves a pair of tiles: every workgroup barrier brings the two
// waves of a SIMD back into step, and between barriers they settle into
// overlapping each other.  Tiles go through rings of four LDS slots per
// matrix (slot = tile % 4).  Iteration p covers tiles a = 2p and a + 1 and
// reads K(a), K(a + 1), V(a - 1), V(a); after its barrier every wave issues
// its share of the copies of K(a + 2), K(a + 3), V(a + 1), V(a + 2) between
// its first matrix products, into slots whose readers finished before the
// barrier, and the index entries of tiles a + 4, a + 5, all landed by the
// next barrier.
template <bool IDX>
__global__ __launch_bounds__(512, 1) void attn_pp_kernel(AttnParams p) {
  constexpr int D = 128;
  constexpr int WAVES = 8;
  constexpr int ROWS = WAVES * 32;
  constexpr int CH = D / 8;                   // 16-byte chunks per row
  constexpr int RPI = 64 / CH;                // tile rows per wave-wide 16-byte load
  constexpr int IPW = kKeyTile / (RPI * WAVES);  // such loads per wave per matrix
  constexpr int TILE = kKeyTile * D;
  constexpr int NS = D / 16;                  // d-steps of the key products
  constexpr int NDB = D / 32;                 // d blocks of the value products
  constexpr int NPV = 4 * NDB;                // value products per tile
  constexpr int NQK = 2 * NS;                 // key products per tile
  constexpr int RING = 6;                     // operands read ahead of their product
  static_assert(IPW == 2 && NPV == 16 && NQK == 16, "copy placement below assumes d = 128");
  // one array per matrix: slot offsets (16 KiB apart) and the read offsets fit
  // the 16-bit immediate of the LDS reads
  __shared__ __attribute__((aligned(16))) uint16_t sK[4 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[4 * TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int col = lane & 31, half = lane >> 5;

  const int L = xcd_swizzle(blockIdx.x, gridDim.x);
  const int qtile = L % p.n_qtiles;
  const int rest = L / p.n_qtiles;
  const int split = rest % p.n_split;
  const int bj = rest / p.n_split;
  const int b = bj / p.nkv, j = bj % p.nkv;
  const int G = p.G, bcp = p.bcp;
  const int M = G * bcp;

  const int past_cap = IDX ? p.ld_idx : static_cast<int>(p.past_bj_rows);
  const int n_past =
      __builtin_amdgcn_readfirstlane(min(p.sel_len ? p.sel_len[bj] : p.n_past, past_cap));
  const int past_tiles = (n_past + kKeyTile - 1) / kKeyTile;
  const int row0 = qtile * ROWS;
  const int i_max = (min(row0 + ROWS, M) - 1) / G;
  // selected past tiles, then the chunk tiles this row tile reaches, divided
  // evenly over the splits
  const int chunk_tiles = i_max / kKeyTile + 1;
  const int total_tiles = past_tiles + chunk_tiles;
  const int g0 = static_cast<int>(static_cast<long long>(split) * total_tiles / p.n_split);
  const int g1 = static_cast<int>(static_cast<long long>(split + 1) * total_tiles / p.n_split);
  const int pt0 = g0;
  const int npt = max(0, min(g1, past_tiles) - g0);
  const int c0 = max(g0, past_tiles) - past_tiles;
  const int nct = max(0, g1 - max(g0, past_tiles));
  const int n_tiles = npt + nct;

  const uint16_t* pk = p.pk + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* pv = p.pv + static_cast<size_t>(bj) * p.past_bj_rows * D;
  const uint16_t* ck = p.k + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const uint16_t* cv = p.v + (static_cast<size_t>(bj) * p.kv_cap + p.t_past) * D;
  const int32_t* idx = IDX ? p.idx + static_cast<size_t>(bj) * p.ld_idx : nullptr;
  const int row_hi = static_cast<int>(p.past_bj_rows) - 1;

  // tile copies (global -> LDS, 16 bytes per lane, layouts of attn_bf16_kernel)
  int trow[IPW], kchunk[IPW], vchunk[IPW];
#pragma unroll
  for (int i = 0; i < IPW; ++i) {
    const int r = (wave * IPW + i) * RPI + lane / CH;
    trow[i] = r;
    kchunk[i] = 16 * ((lane % CH) ^ swz_k<D>(r));
    vchunk[i] = 16 * ((lane % CH) ^ swz_v<D>(r));
  }
  // Index entries of tile x's rows (IDX), loaded without branches: every call
  // issues the same loads (clamped into the list), and a row is resolved when
  // its copy is issued.  Without an index list the entries are the positions.
  auto rows_of = [&](int x, int* rr) __attribute__((always_inline)) {
    const int k0 = (pt0 + x) * kKeyTile;
#pragma unroll
    for (int i = 0; i < IPW; ++i)
      rr[i] = IDX ? idx[max(min(k0 + trow[i], n_past - 1), 0)] : k0 + trow[i];
  };
  // load i of tile x's K (or V) copy into slot x % 4 of dst
  auto copy_one = [&](int x, int i, const int* rr, const uint16_t* pbase, const uint16_t* cbase,
                      const int* chunk, uint16_t* dst) __attribute__((always_inline)) {
    const bool past = x < npt;  // uniform
    const uint16_t* base = past ? pbase : cbase;
    const int row = past ? min(max(rr[i], 0), row_hi)
                         : min((c0 + x - npt) * kKeyTile + trow[i], bcp - 1);
    lds_load16_async(base, static_cast<uint32_t>(row) * (2 * D) + static_cast<uint32_t>(chunk[i]),
                     __builtin_amdgcn_readfirstlane(
                         lds_addr_of(dst + (x & 3) * TILE + (wave * IPW + i) * 512)));
  };

  bf16x8 qf[NS];
  const int r_me = row0 + wave * 32 + col;
  const int iq = r_me / G;
  {
    // branch-free: padding rows read a valid row and zero it
    const bool valid = r_me < M;
    const int rc = valid ? r_me : M - 1;
    const int ic = rc / G, g = rc - ic * G;
    const uint16_t* qp = p.q + ((static_cast<size_t>(b) * p.nq + j * G + g) * bcp + ic) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const u32x4 w = ld16(qp + 16 * s + 8 * half);
      qf[s] = as_bf16x8(valid ? w : u32x4{0, 0, 0, 0});
    }
  }
  const bool wave_active = row0 + wave * 32 < M;

  // LDS read offsets in bytes from the matrix's array (the layouts of
  // attn_bf16_kernel); every read adds only an immediate (slot, block)
  constexpr int NKA = NS < 8 ? NS : 8;
  int kofs[NKA];
  {
    const int fk = half ^ swz_k<D>(col);
#pragma unroll
    for (int s = 0; s < NKA; ++s) kofs[s] = 2 * (col * D + 8 * ((2 * s) ^ fk));
  }
  int vofs[NDB];
  {
    const int g = lane >> 4, jl = lane & 15, jj = jl >> 2;
    const int vr = 4 * (g >> 1) + jj;
    const int x = 2 * (g & 1) + ((jl & 3) >> 1);
    const int fv = swz_v<D>(vr);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vofs[db] = 2 * (vr * D + 8 * ((4 * db + x) ^ fv) + 4 * (jl & 1));
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = p.scale_log2;
  const int n_full = min(max(n_past / kKeyTile - pt0, 0), npt);

  f32x16 S[2];      // S^T of the tile whose key products ran last
  bf16x8 P[4];      // its probabilities (operands of the next value products)
  bf16x8 ring[RING];

  // The value products of one tile (operand i: key group i / NDB, d block
  // i % NDB) and the key products of one tile (operand i: d-step i / 2, key
  // block i % 2), each with RING operands read ahead of their product.
  auto pv_read = [&](int i, const uint16_t* cV) __attribute__((always_inline)) {
    return lds_read_tr_pair(
        reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(cV) + vofs[i % NDB]) +
            (i / NDB) * 16 * D,
        D);
  };
  auto qk_read = [&](int i, const uint16_t* cK) __attribute__((always_inline)) {
    const int s = i >> 1, kb = i & 1;
    return as_bf16x8(*reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(cK) + kofs[s % NKA] +
                                                     2 * (kb * 32 * D + 128 * (s / NKA))));
  };
  auto pv_head = [&](const uint16_t* cV) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RING; ++i) ring[i] = pv_read(i, cV);
  };
  // side(i) runs after product i (the interleaved copies)
  auto pv_body = [&](const uint16_t* cV, auto side) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      acc[i % NDB] = mfma32(ring[i % RING], P[i / NDB], acc[i % NDB]);
      if (i + RING < NPV) ring[i % RING] = pv_read(i + RING, cV);
      side(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto qk_head = [&](const uint16_t* cK) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < RING; ++i) ring[i] = qk_read(i, cK);
  };
  auto qk_body = [&](const uint16_t* cK, auto side) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
      const int s = i >> 1, kb = i & 1;
      S[kb] = mfma32(ring[i % RING], qf[s], s == 0 ? f32x16{} : S[kb]);
      if (i + RING < NQK) ring[i % RING] = qk_read(i + RING, cK);
      side(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto no_side = [](int) {};

  // softmax of tile x (S -> P), with the lazy rescale of attn_bf16_kernel
  auto softmax = [&](int x) __attribute__((always_inline)) {
    if (x >= n_full) {  // uniform: boundary and chunk tiles only
      const bool is_chunk = x >= npt;
      const int kbase = is_chunk ? (c0 + x - npt) * kKeyTile : (pt0 + x) * kKeyTile;
      const int lim = (is_chunk ? min(bcp, iq + 1) : n_past) - kbase - 4 * half;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + 8 * (r >> 2) + (r & 3) >= lim) S[kb][r] = -INFINITY;
    }
    float mx = fmaxf(S[0][0], S[1][0]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx *= c2;
    if (__any(mx > m_run + kSlack)) {
      const float mq = swap_op<32>(mx, [](float a, float c) { return fmaxf(a, c); });
      const float m_new = mq > m_run + kSlack ? mq : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int g16 = 0; g16 < 4; ++g16) {
      const int kb = g16 >> 1, r0 = 8 * (g16 & 1);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r0 + 2 * e], c2, -m_use));
        const float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[kb][r0 + 2 * e + 1], c2, -m_use));
        w[e] = pack_bf16x2(x0, x1);
      }
      P[g16] = as_bf16x8(w);
      if (g16 & 1) ps1 = sum_bf16x8(P[g16], ps1);
      else ps0 = sum_bf16x8(P[g16], ps0);
    }
    l_run += ps0 + ps1;
  };

  // Tile step t (slot constants ST = t % 4): the matrix block reads K(t) and
  // V(t - 1).  side(i) runs after matrix product i of the step (value
  // products first, then key products).  EDGE: the step may lack its value
  // products (t = 0) or its key products (t = n_tiles), checked at run time.
  auto tile_step = [&](int t, auto grp_c, auto st, auto edge, auto side) __attribute__((always_inline)) {
    constexpr int GRP = decltype(grp_c)::value;
    constexpr int ST = decltype(st)::value;
    constexpr bool EDGE = decltype(edge)::value;
    const uint16_t* kcur = sK + ST * TILE;
    const uint16_t* vprev = sV + ((ST + 3) & 3) * TILE;
    const bool has_pv = !EDGE || (t >= 1 && t <= n_tiles);
    const bool has_qk = !EDGE || t < n_tiles;
    auto side_qk = [&](int i) __attribute__((always_inline)) { side(i + NPV); };
    if (GRP == 0) {
      if (has_pv) {
        pv_head(vprev);
        pv_body(vprev, side);
      } else {
#pragma unroll
        for (int i = 0; i < NPV; ++i) side(i);
      }
      if (has_qk) {
        qk_head(kcur);
        qk_body(kcur, side_qk);
        softmax(t);
      } else {
#pragma unroll
        for (int i = 0; i < NQK; ++i) side_qk(i);
      }
    } else {
      if (has_pv) {
        pv_head(vprev);
        softmax(t - 1);
        pv_body(vprev, side);
      } else {
#pragma unroll
        for (int i = 0; i < NPV; ++i) side(i);
      }
      if (has_qk) {
        qk_head(kcur);
        qk_body(kcur, side_qk);
      } else {
#pragma unroll
        for (int i = 0; i < NQK; ++i) side_qk(i);
      }
    }
  };

  // Row entries: rk0 / rk1 those of tiles a + 2 / a + 3 (K copies; a + 2 also
  // for its V copy), rv those of tile a + 1 (V copy), loaded an iteration
  // ahead and landed by the barrier.
  int rk0[IPW], rk1[IPW], rv[IPW];

  // the copies and index loads of iteration a, as side work: copies after
  // products 1, 5, 9, ... of tile a's 32, index loads after 30 and 31
  auto copy_side = [&](int a, int i) __attribute__((always_inline)) {
    if (i < 30 && (i & 3) == 1) {
      const int n = i >> 2;   // 0..7: K(a+2) x2, K(a+3) x2, V(a+1) x2, V(a+2) x2
      const int i2 = n & 1;
      if (n < 2) {
        if (a + 2 < n_tiles) copy_one(a + 2, i2, rk0, pk, ck, kchunk, sK);
      } else if (n < 4) {
        if (a + 3 < n_tiles) copy_one(a + 3, i2, rk1, pk, ck, kchunk, sK);
      } else if (n < 6) {
        if (a + 1 < n_tiles) copy_one(a + 1, i2, rv, pv, cv, vchunk, sV);
      } else {
        if (a + 2 < n_tiles) copy_one(a + 2, i2, rk0, pv, cv, vchunk, sV);
      }
    } else if (i == 30) {
#pragma unroll
      for (int u = 0; u < IPW; ++u) rv[u] = rk1[u];
      rows_of(a + 4, rk0);
    } else if (i == 31) {
      rows_of(a + 5, rk1);
    }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's copies and index loads landed
    barrier_no_fence();
    // The read offsets are marked as redefined here (no instruction), so that
    // the compiler forms each read address next to its read, where the slot
    // and block fold into the instruction's offset, instead of keeping one
    // register per address and slot across the loop.
#pragma unroll
    for (int s2 = 0; s2 < NKA; ++s2) asm volatile("" : "+v"(kofs[s2]));
#pragma unroll
    for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(vofs[db]));
  };
  // Iteration over tiles a and a + 1 (SA = a % 4): the barrier, then the two
  // tile steps with the copies and index loads among tile a's products.
  auto iteration = [&](int a, auto grp_c, auto sa, auto edge) __attribute__((always_inline)) {
    constexpr int SA = decltype(sa)::value;
    sync();
    tile_step(a, grp_c, sa, edge, [&](int i) __attribute__((always_inline)) { copy_side(a, i); });
    tile_step(a + 1, grp_c, std::integral_constant<int, (SA + 1) & 3>{}, edge, no_side);
  };
  using A0 = std::integral_constant<int, 0>;
  using A2 = std::integral_constant<int, 2>;
  using T_ = std::true_type;
  using F_ = std::false_type;
  // Tile steps 0 .. n_tiles in pairs: the first pair (no value products at
  // step 0), a steady loop while both steps of a pair have all their work,
  // then the last pairs; per group (uniform per wave), so that each copy keeps
  // only its own values live across iterations.
  auto run = [&](auto g) __attribute__((always_inline)) {
    iteration(0, g, A0{}, T_{});
    int a = 2;
    for (; a + 3 < n_tiles; a += 4) {
      iteration(a, g, A2{}, F_{});
      iteration(a + 2, g, A0{}, F_{});
    }
    // a % 4 == 2 here; at most two pairs remain (steps up to n_tiles)
    if (a <= n_tiles) {
      iteration(a, g, A2{}, T_{});
      if (a + 2 <= n_tiles) iteration(a + 2, g, A0{}, T_{});
    }
  };
  // waves whose rows are all padding: the same barriers, copies and index loads
  auto run_idle = [&]() __attribute__((always_inline)) {
    for (int a = 0; a <= n_tiles; a += 2) {
      sync();
#pragma unroll
      for (int i = 0; i < NPV + NQK; ++i) copy_side(a, i);
    }
  };

  if (n_tiles > 0) {
    // K(0), K(1), V(0), then the entries of tiles 2 and 3 for iteration 0
    rows_of(0, rk0);
    rows_of(1, rk1);
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
      copy_one(0, i, rk0, pk, ck, kchunk, sK);
      copy_one(0, i, rk0, pv, cv, vchunk, sV);
      if (n_tiles > 1) copy_one(1, i, rk1, pk, ck, kchunk, sK);
    }
#pragma unroll
    for (int i = 0; i < IPW; ++i) rv[i] = rk1[i];
    rows_of(2, rk0);
    rows_of(3, rk1);
    if (!wave_active) run_idle();
    else if (grp == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  }
  __builtin_amdgcn_s_waitcnt(0x0f70);

  finish_rows<D>(p, acc, m_run, l_run, r_me, M, iq, b, j, split);
}

// Merge key-split partials:
//   O = sum_s w_s M_s P_s / sum_s w_s,  w_s = 2^(lse_s - max_s lse_s),
// P_s the fp16 partial scaled by 1 / M_s.  A row's D fp16 values are covered
// by D / 8 lanes with 16 bytes each, so one wave handles 512 / D consecutive
// rows and each of its loads of one split reads 1 KiB contiguous.  Every lane
// of a row reads that row's (lse, M) of all splits (same addresses within a
// row: one request) and forms the weights itself.
template <int D>
__global__ __launch_bounds__(256) void attn_combine_kernel(const uint32_t* __restrict__ part_o,
                                                           const float2* __restrict__ part_ls,
                                                           uint16_t* __restrict__ out,
                                                           float* __restrict__ lse, int n_split,
                                                           long long rows) {
  constexpr int LPR = D / 8;           // lanes per row
  constexpr int RPW = 64 / LPR;        // rows per wave
  constexpr int kBatch = 16;           // splits loaded together
  const int lane = threadIdx.x & 63;
  const long long row0 = (static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW;
  const long long row = row0 + lane / LPR;
  const int c = lane % LPR;            // this lane's 8 values: d = 8c .. 8c + 7
  const bool live = row < rows;
  const long long r = live ? row : rows - 1;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float mx = -INFINITY, wsum = 0.f;
  // one batch of splits: (lse, M) and the partial words loaded together
  auto batch = [&](int s0, bool find_max) {
    float2 lm[kBatch];
    u32x4 x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // a uniform branch: only the row's splits are read (no clamped repeats)
      if (s0 + u < n_split) {
        const long long sidx = s0 + u;
        lm[u] = part_ls[sidx * rows + r];
        x[u] = *reinterpret_cast<const u32x4*>(part_o + (sidx * rows + r) * (D / 2) + 4 * c);
      }
    }
    if (find_max) {
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u < n_split) mx = fmaxf(mx, lm[u].x);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (s0 + u >= n_split) break;
      const float w = lm[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lm[u].x - mx);
      wsum += w;
      const float f = w * lm[u].y;  // weight of the scaled partial
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 v = unpack_f16x2(x[u][e]);
        acc[2 * e] += f * v[0];
        acc[2 * e + 1] += f * v[1];
      }
    }
  };
  if (n_split <= kBatch) {
    batch(0, true);  // the usual case: one memory round trip
  } else {
    for (int s = 0; s < n_split; ++s)
      mx = fmaxf(mx, part_ls[static_cast<long long>(s) * rows + r].x);
    for (int s0 = 0; s0 < n_split; s0 += kBatch) batch(s0, false);
  }
  if (!live) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
  *reinterpret_cast<u32x4*>(out + row * D + 8 * c) = o;
  if (lse && c == 0) lse[row] = wsum > 0.f ? (mx + log2f(wsum)) * kLn2 : -INFINITY;
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

// Row blocks per wave at d = 128.  One block and two waves per SIMD measured
// faster than two blocks and one wave per SIMD (the accumulators of two
// blocks overflow the architectural registers and shuttle through AGPRs).
constexpr int kNB128 = 1;
// Waves per workgroup at d = 128 when a KV head has more than 128 query rows:
// eight (256 rows, one workgroup per CU, two waves per SIMD), so that a K/V
// tile in LDS serves twice the rows of a four-wave workgroup and each CU
// copies half as many tiles (measured: 2-3 % faster at llama3b_32k, equal at
// 128K past).  Fewer rows (decode) keep four waves: there the waves past the
// rows only help copy tiles, and eight were 8 % slower.
constexpr int kWaves128 = 8;

struct Plan {
  int waves, nb, rows, n_qtiles, n_split;
  bool pp;  // the ping-pong kernel (eight waves at d = 128)
};

Plan make_plan(int b, int nq, int nkv, int d, int bcp, int n_past_max) {
  Plan pl{};
  const int G = nq / nkv;
  const int M = G * bcp;
  pl.waves = d == 128 && M > 128 ? kWaves128 : 4;
  pl.nb = d == 128 ? kNB128 : 1;
  pl.rows = pl.waves * pl.nb * 32;
  pl.n_qtiles = (M + pl.rows - 1) / pl.rows;
  const int past_tiles = (n_past_max + kKeyTile - 1) / kKeyTile;
  const long long base = static_cast<long long>(pl.n_qtiles) * b * nkv;
  // key splits fill the resident slots (256 CUs x workgroups per CU: one for
  // d = 256, two row blocks per wave or eight waves, else two) without
  // spilling into a second, mostly idle round; at least 4 key tiles per split
  const long long wg_per_cu = (d == 256 || pl.nb == 2 || pl.waves == 8) ? 1 : 2;
  const long long slots = 256LL * wg_per_cu;
  long long ns = slots / base;
  const long long max_split = past_tiles / 4 > 1 ? past_tiles / 4 : 1;
  if (ns > max_split) ns = max_split;
  if (ns > 64) ns = 64;
  if (ns < 1) ns = 1;
  pl.pp = d == 128 && pl.waves == 8;
  pl.n_split = static_cast<int>(ns);
  return pl;
}

template <int D, int NB, int WAVES, int OCC>
hipError_t run_bf16(const AttnParams& p, int grid, hipStream_t st) {
  if (p.idx)
    hipLaunchKernelGGL((attn_bf16_kernel<D, NB, WAVES, OCC, true>), dim3(grid), dim3(64 * WAVES), 0, st, p);
  else
    hipLaunchKernelGGL((attn_bf16_kernel<D, NB, WAVES, OCC, false>), dim3(grid), dim3(64 * WAVES), 0, st, p);
  return hipGetLastError();
}

}  // namespace

size_t attn_workspace_bytes(bool bf16, int b, int nq, int nkv, int d, int bcp, int n_past_max) {
  if (!bf16) return 0;
  const Plan pl = make_plan(b, nq, nkv, d, bcp, n_past_max);
  if (pl.n_split <= 1) return 0;
  const size_t rows = static_cast<size_t>(b) * nq * bcp;
  // fp16 partial outputs + (log-sum-exp, scale) per split and row
  return static_cast<size_t>(pl.n_split) * rows * (d * 2 + sizeof(float2));
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
    p.part_o = static_cast<uint32_t*>(c.ws);
    p.part_ls = reinterpret_cast<float2*>(p.part_o + static_cast<size_t>(pl.n_split) * rows * c.d / 2);
  }
  const int grid = pl.n_qtiles * c.b * c.nkv * pl.n_split;
  hipError_t e;
  if (pl.pp) {
    if (p.idx)
      hipLaunchKernelGGL((attn_pp_kernel<true>), dim3(grid), dim3(512), 0, st, p);
    else
      hipLaunchKernelGGL((attn_pp_kernel<false>), dim3(grid), dim3(512), 0, st, p);
    e = hipGetLastError();
  }
  else if (c.d == 128 && pl.waves == kWaves128) e = run_bf16<128, kNB128, kWaves128, 1>(p, grid, st);
  else if (c.d == 128) e = run_bf16<128, kNB128, 4, 2>(p, grid, st);
  else if (c.d == 64) e = run_bf16<64, 1, 4, 2>(p, grid, st);
  else if (c.d == 256) e = run_bf16<256, 1, 4, 1>(p, grid, st);
  else return hipErrorInvalidValue;
  if (e != hipSuccess || pl.n_split == 1) return e;
  const size_t rows_per_wg = 4 * (512 / c.d);  // 4 waves, 512 / d rows each
  const dim3 cgrid(static_cast<unsigned>((rows + rows_per_wg - 1) / rows_per_wg)), cblock(256);
  if (c.d == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, cgrid, cblock, 0, st, p.part_o, p.part_ls,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  else if (c.d == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, cgrid, cblock, 0, st, p.part_o, p.part_ls,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  else
    hipLaunchKernelGGL(attn_combine_kernel<256>, cgrid, cblock, 0, st, p.part_o, p.part_ls,
                       static_cast<uint16_t*>(c.out), c.lse, pl.n_split, static_cast<long long>(rows));
  return hipGetLastError();
}

}  // namespace qk
