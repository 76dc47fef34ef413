/*
 * qk.h -- C ABI of the query-oriented sparse KV selection library (gfx950).
 *
 * One prefill chunk (or one decode token) of attention with QUOKA-style key
 * selection:
 *
 *   qk_qsel         mean query, negated cosine scores, top-NQ queries per head,
 *                   normalise and average over each GQA group
 *   qk_kvscore      cosine score of every past key against the group queries,
 *                   max over the kept queries
 *   qk_kvscore_grouped  same, forming the group queries from the kept
 *                   positions inside the scoring pass
 *   qk_kvscore_variant  the grouped scoring pass with a choice of score
 *                   (cosine, or the dot-product baseline) and of key storage
 *                   (the dtype, or 8-bit E4M3 keys)
 *   qk_keys_to_e4m3 store key rows as E4M3 bytes for the 8-bit scoring pass
 *   qk_topk         per-row top-k indices of fp32 scores (ascending order)
 *   qk_select       qk_qsel + qk_kvscore_variant + qk_topk in one call, the
 *                   scoring pass also counting what the top-k needs first
 *   qk_round_select round-granular variant: round score = max over the round,
 *                   keep the latest round plus the top rounds
 *   qk_gather       copy the selected K/V rows into dense buffers
 *   qk_sparse_attn  softmax attention of the chunk over gathered selected keys
 *                   (no mask) plus the chunk's own keys (causal)
 *   qk_sparse_attn_indexed  same, reading the selected rows straight from the
 *                   cache through the index list (gather fused into the loads)
 *   qk_dense_attn   the same chunk over every past key (reference path)
 *
 * Sources: the "QUOKA" technical write-up (bqwf.cn) -- section 2.1 Algorithm 1
 * (query sub-selection), section 2.2 (cosine score S_ij), section 2.3
 * (aggregation listing), section 4.2 question 3 (the selected KV is the
 * attention's KV input, causal mask disabled); the Round Attention press
 * release (Moore Threads), sections 01-02 (round-granular block top-K).
 *
 * Conventions shared by every call
 * --------------------------------
 * Pointers are DEVICE pointers unless marked [host].  Tensors are row-major and
 * contiguous:
 *     q        (b, nq,  bcp,    d)     the chunk's queries (bcp = 1: decode)
 *     k, v     (b, nkv, kv_cap, d)     rows [0, t_past) are the past,
 *                                      rows [t_past, t_past + bcp) the chunk's own
 *     out      (b, nq,  bcp,    d)     same dtype as q
 *     q_group  (b, nkv, nq_keep, d)    fp32
 *     s_agg    (b, nkv, t_past)        fp32
 *     idx      (b, nkv, ld_idx)        int32 past positions
 * Query head h uses KV head h / (nq / nkv).
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer past
 * return and allocates nothing.  Outputs must not alias inputs.  Scratch memory
 * comes from the caller as (ws, ws_bytes), sized by qk_workspace_bytes; its
 * contents need no initialisation and are dead after the call.  Calls that use
 * one workspace concurrently (different streams) race.
 *
 * Execution: every call validates its arguments on the host, enqueues its
 * kernels on `stream` and returns without synchronising.  Apart from the
 * fixed scratch array of qk_sparse_attn_indexed_noalloc, the library holds no
 * mutable global state; calls on different streams are independent.
 *
 * Errors: validation happens before any launch; on error nothing is launched
 * and nothing is written.  A failed launch returns QK_ERR_HIP.  Faults inside a
 * kernel surface at the caller's next synchronisation.  Inputs must be finite.
 */
#ifndef QK_H_
#define QK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* qk_stream_t; /* a hipStream_t; NULL = default stream */

typedef enum {
  QK_OK = 0,
  QK_ERR_NULL = 1,        /* a required pointer is NULL                       */
  QK_ERR_SHAPE = 2,       /* a size is out of range or inconsistent           */
  QK_ERR_DTYPE = 3,       /* dtype not supported by this call                 */
  QK_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned          */
  QK_ERR_WORKSPACE = 5,   /* ws_bytes smaller than qk_workspace_bytes         */
  QK_ERR_UNSUPPORTED = 6, /* head dim or size beyond what the kernels handle  */
  QK_ERR_HIP = 7,         /* the HIP runtime refused a launch                 */
  QK_ERR_SCRATCH_LIMIT = 8 /* more scratch needed than the library's fixed
                              array holds (QK_NOALLOC_SCRATCH_BYTES)          */
} qk_status;

typedef enum { QK_F32 = 0, QK_BF16 = 1 } qk_dtype;

/* [host] Problem description shared by the calls. */
typedef struct {
  int32_t b;        /* sequences in the batch, >= 1                              */
  int32_t nq;       /* query heads, a multiple of nkv, at most 64 * nkv          */
  int32_t nkv;      /* KV heads, >= 1                                            */
  int32_t d;        /* head dim: 64, 128 or 256                                  */
  int32_t bcp;      /* chunk queries, 1 .. 4096 (1 = decode)                     */
  int32_t t_past;   /* T, past positions scored, >= 0 (>= 1 for selection)        */
  int32_t kv_cap;   /* rows per (sequence, KV head) in k and v, >= t_past + bcp;
                       kv_cap * d * 4 must not exceed INT32_MAX (else
                       QK_ERR_UNSUPPORTED)                                    */
  int32_t nq_keep;  /* NQ, kept queries per head, 1 .. min(bcp, 256)             */
  int32_t bsa;      /* BSA, kept keys per KV head, >= 1; values above T act as T */
  float scale;      /* softmax scale; 0 means 1/sqrt(d)                          */
  int32_t dtype;    /* qk_dtype of q, k, v and out                               */
} qk_shape;

/* Operation codes for qk_workspace_bytes. */
typedef enum {
  QK_OP_QSEL = 0,
  QK_OP_KVSCORE = 1,
  QK_OP_TOPK = 2,
  QK_OP_ROUND_SELECT = 3,
  QK_OP_GATHER = 4,
  QK_OP_SPARSE_ATTN = 5,
  QK_OP_DENSE_ATTN = 6,
  QK_OP_SELECT = 7
} qk_op;

/* [host] Version of this ABI (bumped on any incompatible change). */
int32_t qk_abi_version(void);

/* [host] Text for a status code; never NULL. */
const char* qk_status_string(qk_status s);

/* [host] Scratch bytes `op` needs for shape `s` (0 if none).  For QK_OP_TOPK,
 * s->b is read as the row count and s->t_past as the row length.  For the
 * attention ops with a ragged selection (sel_len != NULL), s->bsa must be the
 * largest selection length.  Returns 0 for an invalid shape. */
size_t qk_workspace_bytes(const qk_shape* s, int32_t op);

/* Query sub-selection and group aggregation (QUOKA write-up, section 2.1
 * Algorithm 1 and section 2.3 listing).
 *   MQ[b,h]  = mean over the chunk of q[b,h,i]
 *   SQ[b,h,i] = -(q.MQ) / (max(|q|,1e-12) max(|MQ|,1e-12))
 *   q_idx[b,h,0..NQ) = positions of the NQ largest SQ, largest first (ties:
 *                      lower position)
 *   q_group[b,j,n] = mean over g < G of q[b,jG+g,q_idx[b,jG+g,n]] / |.|
 * q: (b,nq,bcp,d) f32 or bf16.  q_idx: (b,nq,NQ) int32.  sq: (b,nq,bcp) f32 or
 * NULL.  q_group: (b,nkv,NQ,d) f32, or NULL to skip the group means (for
 * qk_kvscore_grouped, which forms them itself).  Arithmetic is fp32. */
qk_status qk_qsel(const qk_shape* s, const void* q, int32_t* q_idx, float* sq,
                  float* q_group, qk_stream_t stream);

/* Key scoring (QUOKA write-up, section 2.2 S_ij and section 2.3 listing).
 *   s_agg[b,j,t] = max over n < NQ of q_group[b,j,n].k[b,j,t] / max(|k[b,j,t]|,1e-12)
 * for t < T.  k: (b,nkv,kv_cap,d) f32 or bf16.  Reads every past key once.
 * bf16: products on the matrix cores with q_group split into a bf16 high and
 * low part (about 2^-16 relative), fp32 accumulation.  f32: fp32 FMA. */
qk_status qk_kvscore(const qk_shape* s, const float* q_group, const void* k,
                     float* s_agg, qk_stream_t stream);

/* Key scoring with the group queries formed inside the scoring pass (QUOKA
 * write-up, section 2.3 listing: normalise the kept queries, average them over
 * the GQA group, score every past key).  Equals qk_qsel's q_group followed by
 * qk_kvscore, without the q_group round trip through memory and its launch.
 * q: (b,nq,bcp,d), same dtype as k.  q_idx: (b,nq,NQ) int32 as written by
 * qk_qsel; entries outside [0, bcp) are clamped into it.  Limits as qk_kvscore;
 * f32 additionally needs NQ*(d+G)*4 <= 65536 bytes (else QK_ERR_UNSUPPORTED). */
qk_status qk_kvscore_grouped(const qk_shape* s, const void* q, const int32_t* q_idx,
                             const void* k, float* s_agg, qk_stream_t stream);

/* Scoring variants of qk_kvscore_variant. */
typedef enum {
  QK_SCORE_COSINE = 0, /* the method's score: as qk_kvscore_grouped                  */
  QK_SCORE_DOT = 1     /* dot-product baseline (QUOKA write-up, section 2.2, its
                          Table 9 comparison): the listing without its two L2
                          normalisations,
                          s_agg[b,j,t] = max over n of
                            (mean over g < G of q[b,jG+g,q_idx[b,jG+g,n]]) . k[b,j,t] */
} qk_score_mode;
typedef enum {
  QK_KEYS_DTYPE = 0, /* k has s->dtype, (b,nkv,kv_cap,d)                              */
  QK_KEYS_E4M3 = 1   /* k is (b,nkv,kv_cap,d) uint8 E4M3 codes (qk_keys_to_e4m3); the
                        scores use the decoded values; needs s->dtype == QK_BF16
                        (bf16 queries), else QK_ERR_DTYPE                             */
} qk_key_format;

/* The grouped scoring pass with a choice of score (`mode`, a qk_score_mode) and
 * key storage (`key_format`, a qk_key_format).  Cosine scoring of dtype keys
 * equals qk_kvscore_grouped.  8-bit keys halve the bytes the pass streams (the
 * attention co-design knowledge card, "Co-Designing AI Model Attention for
 * Fast, Interactive Long-Context Inference", lists FP8 KV caches among its
 * measured kernels); each code is decoded exactly to bf16 and multiplied on the
 * matrix cores as in the bf16 path.  Arguments and limits as
 * qk_kvscore_grouped; an unknown mode or format returns QK_ERR_UNSUPPORTED. */
qk_status qk_kvscore_variant(const qk_shape* s, const void* q, const int32_t* q_idx,
                             const void* k, int32_t key_format, int32_t mode, float* s_agg,
                             qk_stream_t stream);

/* Store rows [row0, row0 + nrows) of every (b, KV head) block of k
 * ((b,nkv,kv_cap,d), s->dtype) as OCP E4M3 codes at the same element positions
 * of k8 ((b,nkv,kv_cap,d) uint8, caller-owned): the code nearest to each value,
 * ties to the even code, magnitudes above 448 (the largest finite code)
 * saturating to 448, the sign bit kept (OCP 8-bit floating point
 * specification, E4M3).  Meant to be called on the rows a chunk appends.
 * Errors: QK_ERR_SHAPE if row0 < 0, nrows < 0 or row0 + nrows > kv_cap;
 * QK_ERR_ALIGN unless k and k8 are 16-byte aligned.  nrows == 0 launches
 * nothing.  Inputs must be finite. */
qk_status qk_keys_to_e4m3(const qk_shape* s, const void* k, int32_t row0, int32_t nrows,
                          uint8_t* k8, qk_stream_t stream);

/* Per-row top-k of fp32 scores (QUOKA write-up, section 2.3: top-BSA keys per
 * KV head).  scores: (rows, n), row stride ld_scores >= n.  idx: (rows, k)
 * int32, row stride ld_idx >= k: the k positions with the largest score (ties:
 * lower position; -0.0 equals +0.0), in ascending position order.  k > n acts
 * as n; positions k..ld_idx of each row are left untouched.  Needs
 * qk_workspace_bytes(QK_OP_TOPK) bytes of scratch (ws, 16-byte aligned; NULL
 * allowed when that is 0): non-zero for rows longer than 16384 scores, and for
 * fewer than 128 rows longer than 4096, where one row is spread over several
 * workgroups.  n <= 8388608 (else QK_ERR_UNSUPPORTED). */
qk_status qk_topk(int32_t rows, int32_t n, int32_t k, const float* scores,
                  int32_t ld_scores, int32_t* idx, int32_t ld_idx, void* ws,
                  size_t ws_bytes, qk_stream_t stream);

/* The whole selection of one chunk (QUOKA write-up, section 2.1 Algorithm 1
 * and section 2.3 listing: query sub-selection, scoring of every past key
 * against the group queries, top-BSA keys per KV head) in one call: the
 * results of qk_qsel (q_group not formed), then qk_kvscore_variant(key_format,
 * mode), then qk_topk(rows = b * nkv, n = t_past, k = bsa) over s_agg, bit for
 * bit.  Writes q_idx (b,nq,NQ), sq (b,nq,bcp) unless NULL, s_agg (b,nkv,T) and
 * idx (b,nkv,ld_idx) with ld_idx >= min(bsa, T).  Where the top-k spreads a
 * row over several workgroups (see qk_topk) and s->dtype is QK_BF16, the
 * scoring pass also counts every row's scores into the histogram the top-k
 * starts from, which saves the top-k its own counting pass.  Scratch:
 * qk_workspace_bytes(QK_OP_SELECT) bytes (ws, 16-byte aligned; NULL allowed
 * when that is 0).  Needs T >= 1 and bsa >= 1 (else QK_ERR_SHAPE); other
 * limits and errors as the three calls.
 * k_new: NULL, or -- with QK_KEYS_E4M3 -- the dtype cache (b,nkv,kv_cap,d),
 * 16-byte aligned, whose chunk rows [T, T + bcp) the scoring pass also stores
 * as E4M3 codes into k (the 8-bit copy), byte for byte what
 * qk_keys_to_e4m3(s, k_new, T, bcp, k) writes: the rows this chunk appends,
 * for the chunks after it (this call scores rows [0, T) only).  Non-NULL with
 * QK_KEYS_DTYPE is QK_ERR_UNSUPPORTED. */
qk_status qk_select(const qk_shape* s, const void* q, const void* k, int32_t key_format,
                    int32_t mode, const void* k_new, int32_t* q_idx, float* sq, float* s_agg,
                    int32_t* idx, int32_t ld_idx, void* ws, size_t ws_bytes,
                    qk_stream_t stream);

/* Flags of qk_round_select's keep_latest argument (0 and 1 keep their
 * meaning: nothing, and the latest round kept). */
#define QK_ROUNDS_KEEP_LATEST 1 /* the latest round is always kept                    */
#define QK_ROUNDS_SHARED 2      /* one choice for all KV heads of a sequence (see below) */

/* Round-granular selection (Round Attention press release, sections 01-02).
 * round_off: (n_rounds + 1) int32, off[0] = 0, strictly increasing,
 * off[n_rounds] = t_past.  For each (b, KV head):
 *   s_round[r] = max over off[r] <= t < off[r+1] of s_agg[b,j,t]
 *   chosen     = {n_rounds-1} and the top_r best of the other rounds when
 *                keep_latest has QK_ROUNDS_KEEP_LATEST (else the top_r best of
 *                all); ties: lower id
 *   idx[b,j,0..sel_len) = every position of the chosen rounds, ascending
 * With QK_ROUNDS_SHARED the rounds are ranked by max over the sequence's KV
 * heads j' of s_round[b,j',r], and every head of the sequence gets the same
 * rounds: a caller that keeps rounds off the GPU then brings in top_r (+ 1)
 * rounds rather than the union of every head's choice.  s_round keeps each
 * head's own round scores.
 * idx: (b,nkv,ld_idx) int32 with ld_idx >= the largest possible selection
 * (t_past is always enough); sel_len: (b,nkv) int32; s_round: (b,nkv,n_rounds)
 * f32, or NULL without QK_ROUNDS_SHARED (else QK_ERR_NULL); chosen:
 * (b,nkv,n_rounds) uint8 or NULL, 1 where round r is one of head (b,j)'s
 * chosen rounds, else 0 (what a caller that keeps rounds off the GPU needs to
 * know to bring them in).  1 <= top_r, top_r + (1 with QK_ROUNDS_KEEP_LATEST)
 * <= n_rounds <= 4096; other flag bits: QK_ERR_UNSUPPORTED. */
qk_status qk_round_select(const qk_shape* s, const float* s_agg, int32_t n_rounds,
                          const int32_t* round_off, int32_t top_r,
                          int32_t keep_latest, int32_t* idx, int32_t ld_idx,
                          int32_t* sel_len, float* s_round, uint8_t* chosen,
                          qk_stream_t stream);

/* Gather the selected rows (QUOKA write-up, section 4.2 question 3: the
 * selection is the attention's KV input).
 *   k_sel[b,j,r] = k[b,j,idx[b,j,r]], v_sel likewise, for r < n_sel(b,j)
 * n_sel = sel_len[b,j] if sel_len != NULL, else min(bsa, t_past).
 * idx: (b,nkv,ld_idx); k_sel, v_sel: (b,nkv,ld_idx,d) same dtype as k.
 * Every index must lie in [0, t_past). */
qk_status qk_gather(const qk_shape* s, const void* k, const void* v,
                    const int32_t* idx, int32_t ld_idx, const int32_t* sel_len,
                    void* k_sel, void* v_sel, qk_stream_t stream);

/* Attention over the selected keys (QUOKA write-up, section 4.2 question 3).
 * For query head h (KV head j) and chunk row i, the keys are the n_sel rows of
 * (k_sel, v_sel)[b,j] -- all visible -- and the chunk rows t_past + u of (k, v)
 * for u <= i.
 *   out[b,h,i] = sum_key softmax(scale q.key) value;  lse = log sum exp(scale q.key)
 * k_sel, v_sel: (b,nkv,ld_sel,d); sel_len as in qk_gather; lse: (b,nq,bcp) f32
 * or NULL.  bf16: matrix-core products, fp32 softmax and accumulation; f32:
 * fp32 throughout, d = 64 or 128 (f32 at d = 256: QK_ERR_UNSUPPORTED, as for
 * every attention call).  Scratch: qk_workspace_bytes(QK_OP_SPARSE_ATTN). */
qk_status qk_sparse_attn(const qk_shape* s, const void* q, const void* k_sel,
                         const void* v_sel, int32_t ld_sel, const int32_t* sel_len,
                         const void* k, const void* v, void* out, float* lse,
                         void* ws, size_t ws_bytes, qk_stream_t stream);

/* As qk_sparse_attn, but the selected past keys are read from the cache
 * through idx (b,nkv,ld_idx) -- the gather is fused into the attention's tile
 * loads and no k_sel / v_sel copy is made.  Every index must lie in
 * [0, t_past). */
qk_status qk_sparse_attn_indexed(const qk_shape* s, const void* q, const void* k,
                                 const void* v, const int32_t* idx, int32_t ld_idx,
                                 const int32_t* sel_len, void* out, float* lse,
                                 void* ws, size_t ws_bytes, qk_stream_t stream);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qk_sparse_attn_indexed with
 * its key-split partials in a file-scope device array of
 * QK_NOALLOC_SCRATCH_BYTES that the library owns, instead of a caller
 * workspace.  The call allocates and frees nothing; its first call on a device
 * looks up that device's copy of the array (each GPU the library runs on holds
 * one until the process ends).  A shape whose attention needs more than
 * QK_NOALLOC_SCRATCH_BYTES (qk_workspace_bytes(QK_OP_SPARSE_ATTN)) is rejected
 * with QK_ERR_SCRATCH_LIMIT before anything is launched.  Every call on one GPU
 * shares that array: calls that overlap on one GPU (concurrent streams, or
 * host threads) race and must be serialised by the caller.  Outputs, errors
 * and arithmetic are those of qk_sparse_attn_indexed.  20 MiB covers every
 * shape: the attention plan keeps (key splits x query rows) within the
 * resident workgroup slots times the rows of one workgroup, at most 17.3 MB
 * of partials. */
#define QK_NOALLOC_SCRATCH_BYTES ((size_t)20 << 20)
qk_status qk_sparse_attn_indexed_noalloc(const qk_shape* s, const void* q, const void* k,
                                         const void* v, const int32_t* idx, int32_t ld_idx,
                                         const int32_t* sel_len, void* out, float* lse,
                                         qk_stream_t stream);

/* Dense attention of the chunk over every past key plus itself causally (the
 * dense baseline of the QUOKA write-up's section 3 tables).  Same outputs and
 * scratch rules as qk_sparse_attn (op QK_OP_DENSE_ATTN). */
qk_status qk_dense_attn(const qk_shape* s, const void* q, const void* k,
                        const void* v, void* out, float* lse, void* ws,
                        size_t ws_bytes, qk_stream_t stream);

/* Measurement only (no step of the method): the matrix-core rate that the
 * attention kernel's instruction mix sustains on this GPU.  256 workgroups of
 * eight waves each run `iters` tiles of 32 32x32x16 bf16 products (the value
 * and key products of one 64-key tile at d = 128).  mode bit 0: random bf16
 * operands of magnitude about one (else near-constant); bit 1: operands read
 * from LDS in the attention's layouts (else from registers); bit 2: each tile
 * followed by the softmax vector work that feeds the next value products.
 * Rate = 256 * 8 * iters * 32 * 32768 flops over the call's duration.
 * out: device, 256 * 512 floats (written, meaningless). */
qk_status qk_calib_matrix_rate(int32_t mode, int32_t iters, float* out, qk_stream_t stream);

/* Measurement only (no step of the method): a bare read of the keys a scoring
 * pass reads for shape s (qk_kvscore_grouped, qk_kvscore_variant, qk_select's
 * scoring) with the same grid, block order, lane layout and ring of blocks in
 * flight, and nothing computed or stored.  Its duration is the floor of a
 * scoring pass over these bytes on this GPU; a pass's time over this one's is
 * the fraction of that floor it reaches.  k: device, (b, nkv, kv_cap, d) in
 * the shape's dtype, or its one-byte E4M3 copy with key_format QK_KEYS_E4M3;
 * rows [0, t_past) of each (b, KV head) are read.  sink: device, 16 bytes,
 * 16-byte aligned, written only if the XOR of every word read equals a fixed
 * sentinel (never in practice).  Errors: QK_ERR_NULL; QK_ERR_DTYPE for fp32
 * shapes (the fp32 scoring pass has no ring); QK_ERR_UNSUPPORTED for another
 * key_format or an NQ the bf16 scoring pass does not handle; QK_ERR_SHAPE,
 * QK_ERR_ALIGN as for qk_kvscore_grouped.  t_past = 0 reads nothing. */
qk_status qk_calib_read_rate(const qk_shape* s, const void* k, int32_t key_format, void* sink,
                             qk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_H_ */
