"""Plain fp64 CPU oracle for query-oriented sparse KV selection (QUOKA) and
attention over the selected keys.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the
HIP library and imports nothing from it.

Sources (web pages, cited by title and section):
  * "QUOKA" technical write-up (bqwf.cn), section 2.1 (query sub-selection,
    Algorithm 1 and the NQ rule), section 2.2 (cosine score S_ij), section 2.3
    (group-aware aggregation listing), section 4.2 question 3 (FlashAttention
    takes QUOKA's output as its KV input, with its causal mask disabled).
  * Attention co-design knowledge card ("Co-Designing AI Model Attention for
    Fast, Interactive Long-Context Inference"), methods list: FP8 KV cache,
    the storage the 8-bit scoring variant reads.  The E4M3 code table follows
    the OCP 8-bit floating point specification (OFP8), not the pages.

Every input is widened to fp64 (exact for fp32 and bf16) and all arithmetic is
fp64.  Readings taken where the pages are silent are stated next to the code
they govern.  Tensor shapes follow the write-up's listing:
    q (b, nq, bcp, d), k and v (b, nkv, kv_cap, d) with rows [0, T) past and
    rows [T, T + bcp) the chunk's own keys/values.
Query head h belongs to KV head j = h // G, G = nq // nkv (the listing's
reshape to (b, nkv, nq // nkv, NQ, d)).
"""
from __future__ import annotations

import math
from typing import Sequence

import numpy as np

EPS = 1e-12  # norms are clamped below at EPS (the pages do not treat zero vectors)


def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _norm(x: np.ndarray) -> np.ndarray:
    return np.sqrt(np.sum(x * x, axis=-1))


def topk_order(scores: np.ndarray, k: int) -> np.ndarray:
    """The k indices of the largest entries of a 1-D array, largest first.

    Ties go to the lower index (the pages do not break ties).  Implemented as a
    full sort on the pair (-score, index), then truncation.
    """
    scores = f64(scores)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))
    return order[: min(k, n)]


# --------------------------------------------------------------------------
# Query sub-selection: QUOKA write-up section 2.1, Algorithm 1.
# --------------------------------------------------------------------------
def mean_query(q) -> np.ndarray:
    """MQ: per query head, the mean of the chunk's queries over the token axis
    (axis 2 of the (b, nq, bcp, d) layout)."""
    return f64(q).mean(axis=2)


def query_scores(q, mq=None) -> np.ndarray:
    """SQ = -cos(q_i, MQ) for every chunk query, shape (b, nq, bcp).

    The priority of a query is its negated cosine to the mean query
    (section 2.1, Theorem 1), so the outliers score highest.
    """
    q = f64(q)
    mq = mean_query(q) if mq is None else f64(mq)
    dot = np.einsum("bhid,bhd->bhi", q, mq)
    den = np.maximum(_norm(q), EPS) * np.maximum(_norm(mq), EPS)[..., None]
    return -dot / den


def select_queries(q, nq_keep: int):
    """Top-NQ chunk queries per head by SQ.

    Returns (qidx, sq): qidx (b, nq, NQ) lists positions in decreasing SQ
    (ties: lower position first), sq (b, nq, bcp).
    """
    sq = query_scores(q)
    b, nq, bcp = sq.shape
    if not 1 <= nq_keep <= bcp:
        raise ValueError("need 1 <= NQ <= bcp")
    qidx = np.empty((b, nq, nq_keep), dtype=np.int64)
    for bi in range(b):
        for h in range(nq):
            qidx[bi, h] = topk_order(sq[bi, h], nq_keep)
    return qidx, sq


# --------------------------------------------------------------------------
# Key scoring and group-aware aggregation: section 2.3 listing, section 2.2
# cosine S_ij.
# --------------------------------------------------------------------------
def group_queries(q, qidx, nkv: int) -> np.ndarray:
    """Q_group: the kept queries, each L2-normalised, averaged over the G query
    heads that share a KV head.  Shape (b, nkv, NQ, d).

    Slot n of the average pairs the n-th ranked kept query of every head in the
    group (the listing reshapes the per-head (NQ, d) blocks and means over the
    head axis; the kept queries come out of top-k in rank order).  The average
    is not renormalised: the listing feeds it straight to the matmul.
    """
    q = f64(q)
    b, nq, bcp, d = q.shape
    G = nq // nkv
    sel = np.take_along_axis(q, np.asarray(qidx)[..., None], axis=2)   # (b, nq, NQ, d)
    q_norm = sel / np.maximum(_norm(sel), EPS)[..., None]
    n_keep = sel.shape[2]
    return q_norm.reshape(b, nkv, G, n_keep, d).mean(axis=2)


def key_scores(q_group, k, t_past: int):
    """S[b,j,n,t] = Q_group[b,j,n] . K[b,j,t] / |K[b,j,t]| for the T past keys,
    and S_agg = max over n.  Returns (s (b,nkv,NQ,T), s_agg (b,nkv,T))."""
    qg = f64(q_group)
    kp = f64(k[:, :, :t_past])
    k_norm = kp / np.maximum(_norm(kp), EPS)[..., None]
    s = np.matmul(qg, np.swapaxes(k_norm, -1, -2))
    return s, s.max(axis=2)


# --------------------------------------------------------------------------
# Scoring variants.
#   * Dot-product scoring: the score that section 2.2 of the QUOKA write-up
#     measures the cosine score against (its Table 9), read as the section 2.3
#     listing with both L2 normalisations removed: the group queries are the
#     plain mean of the kept queries over the G heads, and the keys enter
#     unnormalised.  Query sub-selection (section 2.1) is unchanged.
#   * 8-bit keys for the scoring pass: the FP8 KV-cache storage that the
#     attention co-design knowledge card ("Co-Designing AI Model Attention for
#     Fast, Interactive Long-Context Inference", methods list) names among the
#     measured prefill and decode kernels, here in the OCP 8-bit
#     floating-point format E4M3 (sign, 4 exponent bits with bias 7, 3
#     mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the code
#     S.1111.111 is NaN; no infinities; largest finite 448).  A key is stored
#     as the code nearest to its value, ties to the even code (even mantissa),
#     magnitudes above 448 saturating to 448; the sign is kept, so -0.0 and
#     small negative values that round to zero become the code 0x80.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code (uint8), fp64; NaN for 0x7f and 0xff."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where((c >> 7) == 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    val = sign * np.where(e > 0, normal, sub)
    return np.where((e == 15) & (m == 7), np.nan, val)


_E4M3_MAG = e4m3_decode(np.arange(0x7F))  # codes 0x00 .. 0x7e: magnitudes 0 .. 448, increasing


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code (uint8) of each value: ties go to the even code,
    magnitudes above 448 saturate to 448, the sign bit follows the value's."""
    x = f64(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    lo = np.searchsorted(_E4M3_MAG, a, side="right") - 1   # largest magnitude <= a
    hi = np.minimum(lo + 1, 0x7E)
    d_lo = a - _E4M3_MAG[lo]
    d_hi = _E4M3_MAG[hi] - a
    code = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def group_queries_dot(q, qidx, nkv: int) -> np.ndarray:
    """Dot-product variant of the group queries: the kept queries, unnormalised,
    averaged over the G heads of the group.  Shape (b, nkv, NQ, d)."""
    q = f64(q)
    b, nq, bcp, d = q.shape
    G = nq // nkv
    sel = np.take_along_axis(q, np.asarray(qidx)[..., None], axis=2)   # (b, nq, NQ, d)
    return sel.reshape(b, nkv, G, sel.shape[2], d).mean(axis=2)


def key_scores_dot(q_group, k, t_past: int):
    """Dot-product variant: S[b,j,n,t] = Q_group[b,j,n] . K[b,j,t] for the T past
    keys, S_agg = max over n.  Returns (s (b,nkv,NQ,T), s_agg (b,nkv,T))."""
    s = np.matmul(f64(q_group), np.swapaxes(f64(k[:, :, :t_past]), -1, -2))
    return s, s.max(axis=2)


def scoring_keys_e4m3(k) -> np.ndarray:
    """The keys the 8-bit scoring pass sees: each element stored as E4M3 and
    read back (fp64)."""
    return e4m3_decode(e4m3_encode(k))


def select_keys(s_agg, bsa: int) -> np.ndarray:
    """Per (b, KV head): the min(BSA, T) past positions with the largest S_agg
    (ties: lower position), returned in ascending position order.  Attention
    does not depend on key order; ascending order is this library's contract."""
    s_agg = f64(s_agg)
    b, nkv, t = s_agg.shape
    kk = min(bsa, t)
    out = np.empty((b, nkv, kk), dtype=np.int64)
    for bi in range(b):
        for j in range(nkv):
            out[bi, j] = np.sort(topk_order(s_agg[bi, j], kk))
    return out


# --------------------------------------------------------------------------
# Round-granular block selection (Round Attention press release, section 02:
# the KV cache is cut at dialogue-round boundaries, and the top-K rounds are
# chosen as whole blocks).
# --------------------------------------------------------------------------
def round_scores(s_agg, round_off) -> np.ndarray:
    """Score of round r = max of S_agg over the round's positions
    [off[r], off[r+1]).  Shape (b, nkv, R)."""
    s_agg = f64(s_agg)
    off = np.asarray(round_off, dtype=np.int64)
    r = len(off) - 1
    out = np.empty(s_agg.shape[:2] + (r,))
    for ri in range(r):
        out[..., ri] = s_agg[..., off[ri]:off[ri + 1]].max(axis=-1)
    return out


def select_rounds(s_round, top_r: int, keep_latest: bool = True):
    """Chosen round ids per (b, KV head), ascending.  With keep_latest the last
    round is always kept and top_r more are picked from the others by score
    (ties: lower round id)."""
    s_round = f64(s_round)
    b, nkv, r = s_round.shape
    chosen = []
    for bi in range(b):
        row = []
        for j in range(nkv):
            if keep_latest:
                rest = topk_order(s_round[bi, j, : r - 1], top_r)
                ids = np.concatenate([rest, [r - 1]])
            else:
                ids = topk_order(s_round[bi, j], top_r)
            row.append(np.sort(ids))
        chosen.append(row)
    return chosen


def select_rounds_shared(s_round, top_r: int, keep_latest: bool = True):
    """One round choice for all KV heads of a sequence (a variant of the
    per-head choice above, so that a caller that keeps rounds off the GPU
    brings in top_r + 1 rounds rather than the union of every head's).
    Reading: the shared score of round r is the largest of the sequence's KV
    heads' round scores (a round matters if it matters to some head); the
    chosen rounds are picked by that score exactly as select_rounds picks them
    per head, and every head gets the same list."""
    s_round = f64(s_round)
    shared = s_round.max(axis=1, keepdims=True)  # (b, 1, R)
    one = select_rounds(shared, top_r, keep_latest)
    return [[row[0].copy() for _ in range(s_round.shape[1])] for row in one]


def round_key_sets(chosen, round_off):
    """Expand chosen round ids to the ascending past positions they cover."""
    off = np.asarray(round_off, dtype=np.int64)
    return [[np.concatenate([np.arange(off[r], off[r + 1]) for r in ids])
             for ids in row] for row in chosen]


# --------------------------------------------------------------------------
# Attention over a key set: section 4.2 question 3 of the QUOKA write-up (the
# selected KV is the attention's KV input, with no causal mask over it).
# --------------------------------------------------------------------------
def attention(q, k, v, t_past: int, key_sets, scale=None, rows=None, heads=None):
    """Softmax attention of chunk queries over (selected past keys) plus (the
    chunk's own keys, causally).

    key_sets[b][j] holds the past positions (< T) visible to every query of KV
    head j.  Chunk query i additionally sees chunk keys T + u for u <= i.
    O = sum_k softmax(scale * q.K[k]) V[k];  LSE = log sum_k exp(scale * q.K[k]).
    scale defaults to 1/sqrt(d).  rows / heads restrict the output to a subset
    (the result then covers only those entries: shapes (b, len(heads),
    len(rows), d) and (b, len(heads), len(rows))).
    """
    q = f64(q)
    b, nq, bcp, d = q.shape
    nkv = len(key_sets[0])
    G = nq // nkv
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(bcp) if rows is None else np.asarray(rows)
    heads = np.arange(nq) if heads is None else np.asarray(heads)
    o = np.empty((b, len(heads), len(rows), d))
    lse = np.empty((b, len(heads), len(rows)))
    for bi in range(b):
        for hi, h in enumerate(heads):
            j = h // G
            past = np.asarray(key_sets[bi][j], dtype=np.int64)
            kk = np.concatenate([f64(k[bi, j, past]), f64(k[bi, j, t_past:t_past + bcp])])
            vv = np.concatenate([f64(v[bi, j, past]), f64(v[bi, j, t_past:t_past + bcp])])
            qq = q[bi, h, rows]                                   # (r, d)
            logits = sc * (qq @ kk.T)                             # (r, n_past + bcp)
            n_past = len(past)
            u = np.arange(bcp)
            hidden = u[None, :] > rows[:, None]                   # chunk key after the query
            logits[:, n_past:][hidden] = -np.inf
            m = logits.max(axis=1, keepdims=True)
            p = np.exp(logits - m)
            l = p.sum(axis=1, keepdims=True)
            o[bi, hi] = (p @ vv) / l
            lse[bi, hi] = (m + np.log(l))[:, 0]
    return o, lse


def dense_key_sets(b: int, nkv: int, t_past: int):
    all_past = np.arange(t_past)
    return [[all_past for _ in range(nkv)] for _ in range(b)]


def dense_attention(q, k, v, t_past: int, scale=None, rows=None, heads=None):
    """Dense causal attention of the chunk over every past key plus itself."""
    return attention(q, k, v, t_past, dense_key_sets(q.shape[0], k.shape[1], t_past),
                     scale, rows, heads)


# --------------------------------------------------------------------------
# Whole pipeline for one chunk.
# --------------------------------------------------------------------------
def pipeline(q, k, v, t_past: int, nq_keep: int, bsa: int = 0, scale=None,
             round_off=None, top_rounds: int = 0, rows=None, heads=None,
             with_attention: bool = True, score: str = "cosine",
             k_e4m3: bool = False) -> dict:
    """Query sub-selection -> key scoring -> top-BSA (or top rounds) ->
    attention over the selected keys.  Returns every intermediate.

    score: "cosine" (section 2.2, the method) or "dot" (its Table 9 baseline);
    k_e4m3: the scoring pass sees the keys stored as E4M3 (attention still uses
    the keys as given)."""
    q = f64(q)
    nkv = k.shape[1]
    qidx, sq = select_queries(q, nq_keep)
    ks = scoring_keys_e4m3(k[:, :, :t_past]) if k_e4m3 else k
    if score == "cosine":
        qg = group_queries(q, qidx, nkv)
        s, s_agg = key_scores(qg, ks, t_past)
    elif score == "dot":
        qg = group_queries_dot(q, qidx, nkv)
        s, s_agg = key_scores_dot(qg, ks, t_past)
    else:
        raise ValueError("score is 'cosine' or 'dot'")
    out = {"sq": sq, "qidx": qidx, "q_group": qg, "s": s, "s_agg": s_agg}
    if round_off is not None:
        s_round = round_scores(s_agg, round_off)
        chosen = select_rounds(s_round, top_rounds)
        key_sets = round_key_sets(chosen, round_off)
        out.update(s_round=s_round, rounds=chosen, key_sets=key_sets)
    else:
        kidx = select_keys(s_agg, bsa)
        key_sets = [[kidx[bi, j] for j in range(nkv)] for bi in range(kidx.shape[0])]
        out.update(kidx=kidx, key_sets=key_sets)
    if with_attention:
        o, lse = attention(q, k, v, t_past, key_sets, scale, rows, heads)
        out.update(o=o, lse=lse)
    return out


# --------------------------------------------------------------------------
# Whole prompts and layer stacks.
#   * A prompt runs in chunks of BCP queries (QUOKA write-up, section 2.1: the
#     chunk size BCP and its NQ rule); the chunk starting at position t takes
#     positions [0, t) as its past and attends its own keys causally.  Decode
#     steps (section 5.1, generation) are chunks of one query with NQ = 1.
#   * Round Attention press release, section 02: past a watershed layer the
#     layers attend to the history alike, so the top-K made at that layer
#     serves every layer above it.  Reading: layers below the watershed attend
#     densely, the watershed layer selects, the layers above attend over its
#     key sets with their own queries, keys and values.
# --------------------------------------------------------------------------
def prompt_chunks(q, k, v, bcp: int, nq_keep: int, bsa: int, n_decode: int = 0,
                  score: str = "cosine", k_e4m3: bool = False):
    """q (b, nq, P + n_decode, d): the prompt's P queries, then n_decode decode
    queries; k, v (b, nkv, >= P + n_decode, d): keys and values of those
    positions.  The prompt runs in chunks of bcp (the last one may be shorter,
    with NQ = min(nq_keep, its length)); each decode step is a chunk of one
    query with NQ = 1.  Returns (o (b, nq, P + n_decode, d), per-step results
    of `pipeline` in order)."""
    q = f64(q)
    total = q.shape[2]
    prompt = total - n_decode
    outs, steps = [], []
    t = 0
    while t < total:
        n = min(bcp, prompt - t) if t < prompt else 1
        keep = min(nq_keep, n) if t < prompt else 1
        r = pipeline(q[:, :, t:t + n], k, v, t, keep, bsa, score=score, k_e4m3=k_e4m3)
        outs.append(r["o"])
        steps.append(r)
        t += n
    return np.concatenate(outs, axis=2), steps


def layer_stack(qs, ks, vs, t_past: int, nq_keep: int, bsa: int, watershed: int,
                score: str = "cosine", round_off=None, top_rounds: int = 0):
    """One chunk through a stack of layers: qs[l] (b, nq, bcp, d) and ks[l],
    vs[l] (b, nkv, >= t_past + bcp, d) per layer l.  Layers below `watershed`
    attend densely, layer `watershed` runs the whole selection (top-BSA keys,
    or with `round_off` the latest round plus the top rounds), the layers above
    attend over its key sets.  Returns (outputs per layer, the key sets)."""
    if not 0 <= watershed < len(qs):
        raise ValueError("the watershed is one of the layers")
    ref = pipeline(qs[watershed], ks[watershed], vs[watershed], t_past, nq_keep, bsa, score=score,
                   round_off=round_off, top_rounds=top_rounds)
    sets = ref["key_sets"]
    outs = []
    for layer in range(len(qs)):
        if layer < watershed:
            o, _ = dense_attention(qs[layer], ks[layer], vs[layer], t_past)
        elif layer == watershed:
            o = ref["o"]
        else:
            o, _ = attention(qs[layer], ks[layer], vs[layer], t_past, sets)
        outs.append(o)
    return outs, sets
