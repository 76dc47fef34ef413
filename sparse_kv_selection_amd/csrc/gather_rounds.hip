// Row gather of the selected keys/values, and the round-granular selection.
//
// Gather: the selected KV is the attention's KV input (QUOKA write-up,
// section 4.2 question 3).  Each row is d elements; a thread moves 16 bytes,
// so a wave moves 1 KiB of consecutive row data per instruction.
//
// Rounds: Round Attention press release (Moore Threads), sections 01-02: the
// KV cache is cut at dialogue-round boundaries and the most relevant rounds are
// kept as whole blocks.  A round's score is the max of the aggregated key score
// over its positions; the latest round is always kept.  One workgroup per
// (sequence, KV head): wave-level max per round, a rank count for the top
// rounds (ties: lower round id), then the chosen rounds' positions are written
// out in ascending order.
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

constexpr int kRoundThreads = 256;

__global__ __launch_bounds__(kRoundThreads) void round_select_kernel(
    const float* __restrict__ s_agg, int t_past, int n_rounds, const int32_t* __restrict__ off,
    int top_r, int keep_latest, int32_t* __restrict__ idx, int ld_idx,
    int32_t* __restrict__ sel_len, float* __restrict__ s_round_out) {
  extern __shared__ float rs[];                              // [n_rounds] round scores
  int* base = reinterpret_cast<int*>(rs + n_rounds);         // [n_rounds] output offsets, -1 = not chosen
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bj = blockIdx.x;
  const float* row = s_agg + static_cast<size_t>(bj) * t_past;

  // round bounds are clamped into [0, t_past] (valid offsets are unaffected)
  auto lo = [&](int r) { return min(max(off[r], 0), t_past); };
  for (int r = wave; r < n_rounds; r += kRoundThreads / 64) {
    float m = -INFINITY;
    for (int t = lo(r) + lane; t < lo(r + 1); t += 64) m = fmaxf(m, row[t]);
    m = wave_max(m);
    if (lane == 0) {
      rs[r] = m;
      if (s_round_out) s_round_out[static_cast<size_t>(bj) * n_rounds + r] = m;
    }
  }
  __syncthreads();

  const int n_cand = keep_latest ? n_rounds - 1 : n_rounds;
  for (int r = tid; r < n_rounds; r += kRoundThreads) {
    bool chosen;
    if (r >= n_cand) {
      chosen = true;  // the latest round
    } else {
      const float s = rs[r];
      int rank = 0;
      for (int r2 = 0; r2 < n_cand; ++r2) {
        const float s2 = rs[r2];
        rank += (s2 > s) | ((s2 == s) & (r2 < r));
      }
      chosen = rank < top_r;
    }
    base[r] = chosen ? 1 : -1;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int r = 0; r < n_rounds; ++r) {
      if (base[r] > 0) {
        base[r] = acc;
        acc += max(lo(r + 1) - lo(r), 0);
      }
    }
    sel_len[bj] = min(acc, ld_idx);
  }
  __syncthreads();
  int32_t* out = idx + static_cast<size_t>(bj) * ld_idx;
  for (int r = wave; r < n_rounds; r += kRoundThreads / 64) {
    const int b0 = base[r];
    if (b0 < 0) continue;
    for (int t = lo(r) + lane; t < lo(r + 1); t += 64) {
      const int o = b0 + (t - lo(r));
      if (o < ld_idx) out[o] = t;
    }
  }
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
                               int ld_idx, int32_t* sel_len, float* s_round, hipStream_t st) {
  const size_t shm = static_cast<size_t>(n_rounds) * (sizeof(float) + sizeof(int));
  hipLaunchKernelGGL(round_select_kernel, dim3(bnkv), dim3(kRoundThreads), shm, st, s_agg, t_past,
                     n_rounds, off, top_r, keep_latest, idx, ld_idx, sel_len, s_round);
  return hipGetLastError();
}

}  // namespace qk
