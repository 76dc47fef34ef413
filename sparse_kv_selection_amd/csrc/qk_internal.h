// Host-side launchers of the kernels, called by the C ABI after validation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

// Query sub-selection + group aggregation.  zero: nullptr, or zero_bytes (a
// multiple of 16) of 16-byte aligned memory that the kernel also clears (the
// histograms of the scoring pass that follows).  q_kept: nullptr, or
// (b, nq, nq_keep, d) in q's dtype, 16-byte aligned, to which the kept rows
// are copied in rank order.
hipError_t launch_qsel(bool bf16, const void* q, int32_t* q_idx, float* sq, float* q_group,
                       int b, int nq, int nkv, int d, int bcp, int nq_keep, int* zero,
                       size_t zero_bytes, void* q_kept, hipStream_t st);

// Key scoring pass.  q_group == nullptr: the group queries are formed from
// (q, q_idx) inside the scoring kernel.
struct ScoreCall {
  bool bf16;
  const float* q_group;
  const void* q;
  const int32_t* q_idx;
  const void* k;
  float* s_agg;
  int b, nq, nkv, d, bcp, t_past, kv_cap, nq_keep;
  bool k_e4m3 = false;  // k holds E4M3 bytes (bf16 queries, grouped only)
  bool dot = false;     // dot-product scoring (grouped only)
  // bf16 only: nullptr, or (b * nkv, kL1Bins) int32, zeroed, to which the pass
  // adds every row's histogram of its scores over the level-1 bins
  int* hist = nullptr;
  // bf16 grouped only: nullptr, or (b, nq, nq_keep, d) the kept rows by rank,
  // as the query pass gathers them (q_idx is then not read)
  const void* q_kept = nullptr;
  // bf16 grouped only: nullptr, or the bf16 cache whose chunk rows [t_past,
  // t_past + bcp) the pass also stores as E4M3 codes into conv_dst
  const void* conv_src = nullptr;
  uint8_t* conv_dst = nullptr;
  // measurement only (bf16): when set, the launch reads the keys with the
  // scoring grid and ring but computes nothing (16-byte sink, see the kernel)
  void* read_sink = nullptr;
};
hipError_t launch_kvscore(const ScoreCall& c, hipStream_t st);

// Rows [row0, row0 + nrows) of every (b, KV head) block of k (bf16 or f32) as
// E4M3 bytes at the same element positions of k8.
hipError_t launch_keys_e4m3(bool bf16, const void* k, uint8_t* k8, int bnkv, int kv_cap, int d,
                            int row0, int nrows, hipStream_t st);
// LDS bytes of the fp32 scoring kernel when it forms the group queries itself.
size_t kvscore_f32_lds_bytes(int d, int nq_keep, int group);

// Per-row top-k, ascending indices.  ws: topk_workspace_bytes of scratch.
// row_hist (only where topk_uses_row_hist): the workspace starts with every
// row's histogram over the level-1 bins (rows x kL1Bins int32), filled by the
// scoring pass, and the top-k skips its own counting pass.
size_t topk_workspace_bytes(int rows, int n, bool row_hist = false);
int topk_max_row();  // longest row qk_topk supports
bool topk_uses_row_hist(int rows, int n, int k);
constexpr int kL1BinsHost = 2048;  // the level-1 bins (kL1Bins of the device code)
hipError_t launch_topk(int rows, int n, int k, const float* scores, int ld_scores, int32_t* idx,
                       int ld_idx, void* ws, bool row_hist, hipStream_t st);

// Round scores, selection and ragged expansion.
hipError_t launch_round_select(const float* s_agg, int bnkv, int t_past, int n_rounds,
                               const int32_t* off, int top_r, int keep_latest, int32_t* idx,
                               int ld_idx, int32_t* sel_len, float* s_round, uint8_t* chosen,
                               int shared_nkv, hipStream_t st);

// Row gather of selected K/V rows.
hipError_t launch_gather(int esz, const void* k, const void* v, const int32_t* idx, int ld_idx,
                         const int32_t* sel_len, int n_sel, void* k_sel, void* v_sel, int bnkv,
                         int d, int kv_cap, hipStream_t st);

// Attention over past rows (gathered, indexed or contiguous) plus the causal chunk.
struct AttnCall {
  bool bf16;
  const void* q;
  const void* pk;           // past key rows
  const void* pv;           // past value rows
  long long past_bj_rows;   // rows between consecutive (b, kv head) blocks of pk / pv
  const int32_t* idx;       // past row list per (b, kv head) or nullptr (identity)
  int ld_idx;
  const int32_t* sel_len;   // per (b, kv head) past count, or nullptr
  int n_past;               // past count when sel_len is nullptr; upper bound otherwise
  const void* k;            // cache (chunk rows read at t_past + u)
  const void* v;
  int kv_cap, t_past;
  void* out;
  float* lse;
  void* ws;
  int b, nq, nkv, d, bcp;
  float scale;
};
size_t attn_workspace_bytes(bool bf16, int b, int nq, int nkv, int d, int bcp, int n_past_max);
hipError_t launch_attention(const AttnCall& c, hipStream_t st);

}  // namespace qk
