// C ABI of the library: argument validation on the host, then kernel launches.
// Every check runs before anything is enqueued, so a rejected call launches
// nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include "../../include/qk.h"
#include "qk_internal.h"

namespace {

inline hipStream_t hs(qk_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

qk_status hip_status(hipError_t e) { return e == hipSuccess ? QK_OK : QK_ERR_HIP; }

// Checks shared by every call that takes a qk_shape.
qk_status check_shape(const qk_shape* s) {
  if (!s) return QK_ERR_NULL;
  if (s->dtype != QK_F32 && s->dtype != QK_BF16) return QK_ERR_DTYPE;
  if (s->b < 1 || s->nkv < 1 || s->nq < s->nkv || s->nq % s->nkv != 0) return QK_ERR_SHAPE;
  if (s->d != 64 && s->d != 128 && s->d != 256) return QK_ERR_UNSUPPORTED;
  if (s->nq / s->nkv > 64) return QK_ERR_UNSUPPORTED;
  if (s->bcp < 1 || s->bcp > 4096) return QK_ERR_SHAPE;
  if (s->t_past < 0) return QK_ERR_SHAPE;
  if (static_cast<int64_t>(s->kv_cap) < static_cast<int64_t>(s->t_past) + s->bcp) return QK_ERR_SHAPE;
  if (!(s->scale >= 0.f) || isinf(s->scale)) return QK_ERR_SHAPE;
  // one (sequence, KV head) block of the cache is addressed with 32-bit offsets
  if (static_cast<int64_t>(s->kv_cap) * s->d * 4 > INT32_MAX) return QK_ERR_UNSUPPORTED;
  return QK_OK;
}

inline bool is_bf16(const qk_shape* s) { return s->dtype == QK_BF16; }
inline int n_sel_of(const qk_shape* s) { return s->bsa < s->t_past ? s->bsa : s->t_past; }

// Largest selection the attention plan is sized for.
inline int attn_past_max(const qk_shape* s, bool dense) { return dense ? s->t_past : n_sel_of(s); }

qk_status check_attn_common(const qk_shape* s, const void* q, const void* k, const void* v,
                            const void* out) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!q || !k || !v || !out) return QK_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return QK_ERR_ALIGN;
  if (!is_bf16(s) && s->d == 256) return QK_ERR_UNSUPPORTED;
  return QK_OK;
}

qk_status check_ws(const qk_shape* s, int32_t op, const void* ws, size_t ws_bytes) {
  const size_t need = qk_workspace_bytes(s, op);
  if (need == 0) return QK_OK;
  if (!ws) return QK_ERR_NULL;
  if (!aligned16(ws)) return QK_ERR_ALIGN;
  if (ws_bytes < need) return QK_ERR_WORKSPACE;
  return QK_OK;
}

qk_status kvscore_common(const qk_shape* s, const float* q_group, const void* q,
                         const int32_t* q_idx, const void* k, float* s_agg, qk_stream_t stream,
                         bool k_e4m3 = false, bool dot = false, bool check_only = false,
                         int* hist = nullptr, const void* q_kept = nullptr,
                         const void* conv_src = nullptr) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!k || !s_agg) return QK_ERR_NULL;
  if (k_e4m3 && !is_bf16(s)) return QK_ERR_DTYPE;
  if (s->nq_keep < 1 || s->nq_keep > s->bcp) return QK_ERR_SHAPE;
  if (is_bf16(s) ? (s->nq_keep > (s->d == 256 ? 32 : 64)) : (s->nq_keep * s->d > 16384))
    return QK_ERR_UNSUPPORTED;
  if (!is_bf16(s) && !q_group &&
      qk::kvscore_f32_lds_bytes(s->d, s->nq_keep, s->nq / s->nkv) > 65536)
    return QK_ERR_UNSUPPORTED;
  if ((q_group && !aligned16(q_group)) || (q && !aligned16(q)) || (q_idx && !aligned4(q_idx)) ||
      !aligned16(k) || !aligned4(s_agg))
    return QK_ERR_ALIGN;
  qk::ScoreCall c;
  c.bf16 = is_bf16(s);
  c.q_group = q_group;
  c.q = q;
  c.q_idx = q_idx;
  c.k = k;
  c.s_agg = s_agg;
  c.b = s->b;
  c.nq = s->nq;
  c.nkv = s->nkv;
  c.d = s->d;
  c.bcp = s->bcp;
  c.t_past = s->t_past;
  c.kv_cap = s->kv_cap;
  c.nq_keep = s->nq_keep;
  c.k_e4m3 = k_e4m3;
  c.dot = dot;
  c.hist = hist;
  c.q_kept = q_kept;
  c.conv_src = conv_src;
  c.conv_dst = conv_src ? static_cast<uint8_t*>(const_cast<void*>(k)) : nullptr;
  if (check_only) return QK_OK;
  return hip_status(qk::launch_kvscore(c, hs(stream)));
}

qk_status qsel_check(const qk_shape* s, const void* q, const int32_t* q_idx, const float* sq,
                     const float* q_group) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!q || !q_idx) return QK_ERR_NULL;
  if (s->nq_keep < 1 || s->nq_keep > s->bcp || s->nq_keep > 256) return QK_ERR_SHAPE;
  if (!aligned16(q) || (q_group && !aligned16(q_group)) || !aligned4(q_idx) || (sq && !aligned4(sq)))
    return QK_ERR_ALIGN;
  return QK_OK;
}

// qk_select: the scoring pass fills the rows' level-1 histograms (bf16, and
// only where the top-k spreads a row over several workgroups).
inline bool select_row_hist(const qk_shape* s) {
  return is_bf16(s) && qk::topk_uses_row_hist(s->b * s->nkv, s->t_past, s->bsa);
}
// qk_select's workspace: the top-k's (starting with the rows' histograms when
// the scoring pass fills them), then -- bf16 -- the kept query rows in rank
// order, (b, nq, NQ, d), which the query pass writes and the scoring pass
// reads instead of looking the positions up.
size_t select_topk_bytes(const qk_shape* s) {
  if (s->bsa >= s->t_past) return 0;  // every key kept: nothing to count
  return qk::topk_workspace_bytes(s->b * s->nkv, s->t_past, select_row_hist(s));
}
size_t select_kept_offset(const qk_shape* s) { return (select_topk_bytes(s) + 255) & ~static_cast<size_t>(255); }
size_t select_ws_bytes(const qk_shape* s) {
  if (!is_bf16(s)) return select_topk_bytes(s);
  return select_kept_offset(s) +
         static_cast<size_t>(s->b) * s->nq * s->nq_keep * s->d * sizeof(uint16_t);
}
// Bytes at the start of the qk_select workspace that the scoring pass
// accumulates into (cleared by the query pass before it).
size_t select_hist_bytes(const qk_shape* s) {
  return static_cast<size_t>(s->b) * s->nkv * qk::kL1BinsHost * sizeof(int);
}

}  // namespace

extern "C" {

int32_t qk_abi_version(void) { return 1; }

const char* qk_status_string(qk_status s) {
  switch (s) {
    case QK_OK: return "ok";
    case QK_ERR_NULL: return "a required pointer is NULL";
    case QK_ERR_SHAPE: return "a size is out of range or inconsistent";
    case QK_ERR_DTYPE: return "dtype not supported by this call";
    case QK_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case QK_ERR_WORKSPACE: return "workspace smaller than qk_workspace_bytes";
    case QK_ERR_UNSUPPORTED: return "head dim or size not handled by the kernels";
    case QK_ERR_HIP: return "the HIP runtime refused a launch";
    case QK_ERR_SCRATCH_LIMIT:
      return "the call needs more scratch than the library's fixed array holds";
  }
  return "unknown status";
}

size_t qk_workspace_bytes(const qk_shape* s, int32_t op) {
  if (op == QK_OP_TOPK) return s ? qk::topk_workspace_bytes(s->b, s->t_past) : 0;
  if (op == QK_OP_QSEL || op == QK_OP_KVSCORE || op == QK_OP_ROUND_SELECT || op == QK_OP_GATHER)
    return 0;
  if (check_shape(s) != QK_OK) return 0;
  if (op == QK_OP_SELECT) return s->t_past >= 1 && s->bsa >= 1 ? select_ws_bytes(s) : 0;
  if (op == QK_OP_SPARSE_ATTN || op == QK_OP_DENSE_ATTN)
    return qk::attn_workspace_bytes(is_bf16(s), s->b, s->nq, s->nkv, s->d, s->bcp,
                                    attn_past_max(s, op == QK_OP_DENSE_ATTN));
  return 0;
}

qk_status qk_qsel(const qk_shape* s, const void* q, int32_t* q_idx, float* sq, float* q_group,
                  qk_stream_t stream) {
  const qk_status st = qsel_check(s, q, q_idx, sq, q_group);
  if (st != QK_OK) return st;
  return hip_status(qk::launch_qsel(is_bf16(s), q, q_idx, sq, q_group, s->b, s->nq, s->nkv, s->d,
                                    s->bcp, s->nq_keep, nullptr, 0, nullptr, hs(stream)));
}

qk_status qk_kvscore(const qk_shape* s, const float* q_group, const void* k, float* s_agg,
                     qk_stream_t stream) {
  if (!q_group) return QK_ERR_NULL;
  return kvscore_common(s, q_group, nullptr, nullptr, k, s_agg, stream);
}

qk_status qk_kvscore_grouped(const qk_shape* s, const void* q, const int32_t* q_idx,
                             const void* k, float* s_agg, qk_stream_t stream) {
  if (!q || !q_idx) return QK_ERR_NULL;
  return kvscore_common(s, nullptr, q, q_idx, k, s_agg, stream);
}

qk_status qk_kvscore_variant(const qk_shape* s, const void* q, const int32_t* q_idx,
                             const void* k, int32_t key_format, int32_t mode, float* s_agg,
                             qk_stream_t stream) {
  if (!q || !q_idx) return QK_ERR_NULL;
  if ((key_format != QK_KEYS_DTYPE && key_format != QK_KEYS_E4M3) ||
      (mode != QK_SCORE_COSINE && mode != QK_SCORE_DOT))
    return QK_ERR_UNSUPPORTED;
  return kvscore_common(s, nullptr, q, q_idx, k, s_agg, stream, key_format == QK_KEYS_E4M3,
                        mode == QK_SCORE_DOT);
}

qk_status qk_calib_read_rate(const qk_shape* s, const void* k, int32_t key_format, void* sink,
                             qk_stream_t stream) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!k || !sink) return QK_ERR_NULL;
  if (key_format != QK_KEYS_DTYPE && key_format != QK_KEYS_E4M3) return QK_ERR_UNSUPPORTED;
  if (!is_bf16(s)) return QK_ERR_DTYPE;
  // the grid follows the scoring pass's, which depends on NQ
  if (s->nq_keep < 1 || s->nq_keep > s->bcp) return QK_ERR_SHAPE;
  if (s->nq_keep > (s->d == 256 ? 32 : 64)) return QK_ERR_UNSUPPORTED;
  if (!aligned16(k) || !aligned16(sink)) return QK_ERR_ALIGN;
  qk::ScoreCall c;
  c.bf16 = true;
  c.q_group = nullptr;
  c.q = nullptr;
  c.q_idx = nullptr;
  c.k = k;
  c.s_agg = nullptr;
  c.b = s->b;
  c.nq = s->nq;
  c.nkv = s->nkv;
  c.d = s->d;
  c.bcp = s->bcp;
  c.t_past = s->t_past;
  c.kv_cap = s->kv_cap;
  c.nq_keep = s->nq_keep;
  c.k_e4m3 = key_format == QK_KEYS_E4M3;
  c.read_sink = sink;
  return hip_status(qk::launch_kvscore(c, hs(stream)));
}

qk_status qk_keys_to_e4m3(const qk_shape* s, const void* k, int32_t row0, int32_t nrows,
                          uint8_t* k8, qk_stream_t stream) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!k || !k8) return QK_ERR_NULL;
  if (row0 < 0 || nrows < 0 || static_cast<int64_t>(row0) + nrows > s->kv_cap) return QK_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(k8)) return QK_ERR_ALIGN;
  if (nrows == 0) return QK_OK;
  return hip_status(qk::launch_keys_e4m3(is_bf16(s), k, k8, s->b * s->nkv, s->kv_cap, s->d, row0,
                                         nrows, hs(stream)));
}

qk_status qk_topk(int32_t rows, int32_t n, int32_t k, const float* scores, int32_t ld_scores,
                  int32_t* idx, int32_t ld_idx, void* ws, size_t ws_bytes, qk_stream_t stream) {
  if (rows < 0 || n < 0 || k < 1 || ld_scores < n) return QK_ERR_SHAPE;
  const int kk = k < n ? k : n;
  if (ld_idx < kk) return QK_ERR_SHAPE;
  if (rows == 0 || n == 0) return QK_OK;
  if (n > qk::topk_max_row()) return QK_ERR_UNSUPPORTED;
  if (!scores || !idx) return QK_ERR_NULL;
  if (!aligned4(scores) || !aligned4(idx)) return QK_ERR_ALIGN;
  const size_t need = qk::topk_workspace_bytes(rows, n);
  if (need > 0) {
    if (!ws) return QK_ERR_NULL;
    if (!aligned16(ws)) return QK_ERR_ALIGN;
    if (ws_bytes < need) return QK_ERR_WORKSPACE;
  }
  return hip_status(qk::launch_topk(rows, n, k, scores, ld_scores, idx, ld_idx, ws, false, hs(stream)));
}

qk_status qk_select(const qk_shape* s, const void* q, const void* k, int32_t key_format,
                    int32_t mode, const void* k_new, int32_t* q_idx, float* sq, float* s_agg,
                    int32_t* idx, int32_t ld_idx, void* ws, size_t ws_bytes,
                    qk_stream_t stream) {
  qk_status st = qsel_check(s, q, q_idx, sq, nullptr);
  if (st != QK_OK) return st;
  if ((key_format != QK_KEYS_DTYPE && key_format != QK_KEYS_E4M3) ||
      (mode != QK_SCORE_COSINE && mode != QK_SCORE_DOT))
    return QK_ERR_UNSUPPORTED;
  const bool e4m3 = key_format == QK_KEYS_E4M3, dot = mode == QK_SCORE_DOT;
  if (k_new && !e4m3) return QK_ERR_UNSUPPORTED;
  if (k_new && !aligned16(k_new)) return QK_ERR_ALIGN;
  st = kvscore_common(s, nullptr, q, q_idx, k, s_agg, stream, e4m3, dot, true);
  if (st != QK_OK) return st;
  if (s->t_past < 1 || s->bsa < 1) return QK_ERR_SHAPE;
  const int rows = s->b * s->nkv, n = s->t_past, kk = n_sel_of(s);
  if (ld_idx < kk) return QK_ERR_SHAPE;
  if (n > qk::topk_max_row()) return QK_ERR_UNSUPPORTED;
  if (!idx) return QK_ERR_NULL;
  if (!aligned4(idx)) return QK_ERR_ALIGN;
  st = check_ws(s, QK_OP_SELECT, ws, ws_bytes);
  if (st != QK_OK) return st;
  const bool row_hist = select_row_hist(s);
  int* hist = row_hist ? static_cast<int*>(ws) : nullptr;
  void* q_kept = is_bf16(s) ? static_cast<char*>(ws) + select_kept_offset(s) : nullptr;
  hipError_t e = qk::launch_qsel(is_bf16(s), q, q_idx, sq, nullptr, s->b, s->nq, s->nkv, s->d,
                                 s->bcp, s->nq_keep, hist, row_hist ? select_hist_bytes(s) : 0,
                                 q_kept, hs(stream));
  if (e != hipSuccess) return QK_ERR_HIP;
  st = kvscore_common(s, nullptr, q, q_idx, k, s_agg, stream, e4m3, dot, false, hist, q_kept,
                      k_new);
  if (st != QK_OK) return st;
  return hip_status(qk::launch_topk(rows, n, s->bsa, s_agg, n, idx, ld_idx, ws, row_hist,
                                    hs(stream)));
}

qk_status qk_round_select(const qk_shape* s, const float* s_agg, int32_t n_rounds,
                          const int32_t* round_off, int32_t top_r, int32_t keep_latest,
                          int32_t* idx, int32_t ld_idx, int32_t* sel_len, float* s_round,
                          uint8_t* chosen, qk_stream_t stream) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!s_agg || !round_off || !idx || !sel_len) return QK_ERR_NULL;
  if (n_rounds < 1 || n_rounds > 4096 || top_r < 1) return QK_ERR_SHAPE;
  const bool latest = (keep_latest & QK_ROUNDS_KEEP_LATEST) != 0;
  const bool shared = (keep_latest & QK_ROUNDS_SHARED) != 0;
  if (keep_latest & ~(QK_ROUNDS_KEEP_LATEST | QK_ROUNDS_SHARED)) return QK_ERR_UNSUPPORTED;
  if (shared && !s_round) return QK_ERR_NULL;  // the heads' round scores meet there
  if (top_r + (latest ? 1 : 0) > n_rounds) return QK_ERR_SHAPE;
  if (s->t_past < n_rounds || ld_idx < s->t_past) return QK_ERR_SHAPE;
  if (!aligned4(s_agg) || !aligned4(round_off) || !aligned4(idx) || !aligned4(sel_len) ||
      (s_round && !aligned4(s_round)))
    return QK_ERR_ALIGN;
  return hip_status(qk::launch_round_select(s_agg, s->b * s->nkv, s->t_past, n_rounds, round_off,
                                            top_r, latest ? 1 : 0, idx, ld_idx, sel_len,
                                            s_round, chosen, shared ? s->nkv : 0, hs(stream)));
}

qk_status qk_gather(const qk_shape* s, const void* k, const void* v, const int32_t* idx,
                    int32_t ld_idx, const int32_t* sel_len, void* k_sel, void* v_sel,
                    qk_stream_t stream) {
  qk_status st = check_shape(s);
  if (st != QK_OK) return st;
  if (!k || !v || !idx || !k_sel || !v_sel) return QK_ERR_NULL;
  if (!sel_len && s->bsa < 1) return QK_ERR_SHAPE;
  if (ld_idx < (sel_len ? 1 : n_sel_of(s))) return QK_ERR_SHAPE;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_sel) || !aligned16(v_sel) ||
      !aligned4(idx) || (sel_len && !aligned4(sel_len)))
    return QK_ERR_ALIGN;
  return hip_status(qk::launch_gather(is_bf16(s) ? 2 : 4, k, v, idx, ld_idx, sel_len,
                                      n_sel_of(s), k_sel, v_sel, s->b * s->nkv, s->d, s->kv_cap,
                                      hs(stream)));
}

static qk_status attn_common(const qk_shape* s, const void* q, const void* pk, const void* pv,
                             long long past_bj_rows, const int32_t* idx, int32_t ld_idx,
                             const int32_t* sel_len, int n_past, const void* k, const void* v,
                             void* out, float* lse, void* ws, size_t ws_bytes, int32_t op,
                             qk_stream_t stream) {
  qk_status st = check_ws(s, op, ws, ws_bytes);
  if (st != QK_OK) return st;
  if (lse && !aligned4(lse)) return QK_ERR_ALIGN;
  qk::AttnCall c{};
  c.bf16 = is_bf16(s);
  c.q = q;
  c.pk = pk;
  c.pv = pv;
  c.past_bj_rows = past_bj_rows;
  c.idx = idx;
  c.ld_idx = ld_idx;
  c.sel_len = sel_len;
  c.n_past = n_past;
  c.k = k;
  c.v = v;
  c.kv_cap = s->kv_cap;
  c.t_past = s->t_past;
  c.out = out;
  c.lse = lse;
  c.ws = ws;
  c.b = s->b;
  c.nq = s->nq;
  c.nkv = s->nkv;
  c.d = s->d;
  c.bcp = s->bcp;
  c.scale = s->scale;
  return hip_status(qk::launch_attention(c, hs(stream)));
}

qk_status qk_sparse_attn(const qk_shape* s, const void* q, const void* k_sel, const void* v_sel,
                         int32_t ld_sel, const int32_t* sel_len, const void* k, const void* v,
                         void* out, float* lse, void* ws, size_t ws_bytes, qk_stream_t stream) {
  qk_status st = check_attn_common(s, q, k, v, out);
  if (st != QK_OK) return st;
  if (!sel_len && s->bsa < 1) return QK_ERR_SHAPE;
  const int n_sel = n_sel_of(s);
  if (n_sel > 0 || sel_len) {
    if (!k_sel || !v_sel) return QK_ERR_NULL;
    if (!aligned16(k_sel) || !aligned16(v_sel) || (sel_len && !aligned4(sel_len)))
      return QK_ERR_ALIGN;
  }
  if (ld_sel < (sel_len ? 1 : n_sel)) return QK_ERR_SHAPE;
  if (static_cast<int64_t>(ld_sel) * s->d * 4 > INT32_MAX) return QK_ERR_UNSUPPORTED;
  return attn_common(s, q, k_sel, v_sel, ld_sel, nullptr, 0, sel_len, n_sel, k, v, out, lse, ws,
                     ws_bytes, QK_OP_SPARSE_ATTN, stream);
}

qk_status qk_sparse_attn_indexed(const qk_shape* s, const void* q, const void* k, const void* v,
                                 const int32_t* idx, int32_t ld_idx, const int32_t* sel_len,
                                 void* out, float* lse, void* ws, size_t ws_bytes,
                                 qk_stream_t stream) {
  qk_status st = check_attn_common(s, q, k, v, out);
  if (st != QK_OK) return st;
  if (!sel_len && s->bsa < 1) return QK_ERR_SHAPE;
  const int n_sel = n_sel_of(s);
  if (!idx) return QK_ERR_NULL;
  if (!aligned4(idx) || (sel_len && !aligned4(sel_len))) return QK_ERR_ALIGN;
  if (ld_idx < (sel_len ? 1 : n_sel)) return QK_ERR_SHAPE;
  return attn_common(s, q, k, v, s->kv_cap, idx, ld_idx, sel_len, n_sel, k, v, out, lse, ws,
                     ws_bytes, QK_OP_SPARSE_ATTN, stream);
}

qk_status qk_dense_attn(const qk_shape* s, const void* q, const void* k, const void* v, void* out,
                        float* lse, void* ws, size_t ws_bytes, qk_stream_t stream) {
  qk_status st = check_attn_common(s, q, k, v, out);
  if (st != QK_OK) return st;
  return attn_common(s, q, k, v, s->kv_cap, nullptr, 0, nullptr, s->t_past, k, v, out, lse, ws,
                     ws_bytes, QK_OP_DENSE_ATTN, stream);
}

}  // extern "C"
