"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (fixed by the method's statement of the target):
  * fp32 scores (SQ, S_agg, round scores): |delta| <= 1e-3
  * top-NQ / top-BSA / round index sets: identical except items whose oracle
    score lies within 2e-3 of the oracle's k-th value
  * attention output: max |delta| <= 2e-2 (bf16), <= 1e-4 (fp32)
Log-sum-exp of the attention (not part of that statement; bound derived from
the arithmetic): the bf16 kernels round every softmax weight to bf16 before
the value products and form the denominator from those same rounded weights,
so the denominator carries a relative error of at most 2^-8 (half an ulp of
an 8-bit significand) and its log at most ln(1 + 2^-8) = 3.9e-3; the bound
5e-3 adds fp32 accumulation.  The fp32 kernel keeps 1e-4.
"""
import numpy as np
import torch

SCORE_TOL = 1e-3
BOUNDARY_TOL = 2e-3
ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 5e-3, "f32": 1e-4}


def np64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64)


def npi(t) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int64)


def kth_value(scores: np.ndarray, k: int) -> float:
    """the k-th largest value of a 1-D array"""
    return float(np.partition(scores, len(scores) - k)[len(scores) - k])


def assert_set_within_boundary(got, want, scores, k, tol=BOUNDARY_TOL, what="set"):
    """got / want: index collections of size k; scores: the oracle's scores of
    every candidate.  Differences are allowed only for near-boundary items."""
    got, want = np.asarray(got), np.asarray(want)
    assert len(got) == k == len(want), (what, len(got), len(want), k)
    assert len(np.unique(got)) == k, f"{what}: duplicate indices"
    gs, ws = set(got.tolist()), set(want.tolist())
    if gs == ws:
        return 0
    vk = kth_value(scores, k)
    diff = gs ^ ws
    bad = [i for i in diff if abs(scores[i] - vk) > tol]
    assert not bad, f"{what}: {len(bad)} non-boundary differences, e.g. index {bad[0]} " \
                    f"score {scores[bad[0]]:.6f} vs k-th {vk:.6f}"
    return len(diff) // 2


def assert_sorted_unique(idx_row, n):
    a = np.asarray(idx_row)
    assert np.all(np.diff(a) > 0), "indices not strictly ascending"
    assert a.min() >= 0 and a.max() < n


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np64(a) - np64(b)))) if np.asarray(np64(a)).size else 0.0


def group_agreement(gpu_qidx, ref_qidx, G):
    """(b, nkv) bool: True where every head of the KV group kept the same
    queries in the same rank order on both sides.  Slot n of the group mean
    pairs the n-th ranked query of each head, so where two queries of a head
    are within rounding of each other the two sides may legitimately pair
    differently; downstream scores of such a group are then not comparable
    value by value (the query choice itself is checked by the boundary rule)."""
    g = np.asarray(gpu_qidx)
    r = np.asarray(ref_qidx)
    b, nq, _ = g.shape
    same = np.all(g == r, axis=-1).reshape(b, nq // G, G)
    return np.all(same, axis=-1)


# --------------------------------------------------------------------------
# Staged comparison of a whole GPU chunk with the oracle.  Each oracle stage
# consumes the GPU's previous discrete decision, so a legitimate swap at a
# near-tie (two kept queries of a head within rounding of each other, a key
# at the BSA-th score) never cascades into value differences downstream, and
# every KV group is compared.
# --------------------------------------------------------------------------
def staged_selection(qn, kn, t_past, nq_keep, bsa, gpu_sq, gpu_qidx, gpu_s_agg, gpu_idx,
                     score="cosine", k_e4m3=False, round_off=None, top_rounds=0, gpu_sel_len=None,
                     shared_rounds=False, what=""):
    """qn (b, nq, bcp, d), kn (b, nkv, >= t_past + bcp, d): fp64 inputs of the
    chunk; gpu_*: the GPU pipeline's outputs for the same sequences (numpy).

    1. SQ within SCORE_TOL of the oracle's; the kept queries of every head
       equal the oracle's up to near-boundary items (BOUNDARY_TOL), and their
       order is the oracle's SQ order up to the GPU's own SQ error (a rank
       differs from the oracle's run only where two SQ values are closer than
       the fp32 rounding that ranked them).
    2. The oracle's group queries and key scores recomputed on the GPU's kept
       positions: S_agg of every KV group within SCORE_TOL (dot-product scores
       relative to sum |q_group| |k|, the scale of their rounding).
    3. The key sets (or chosen rounds) against the oracle's selection on those
       scores, by the boundary rule.

    Returns (key_sets, stats): key_sets[b][j] the GPU's selected past
    positions (for the attention check); stats: max SQ and S_agg errors, the
    number of KV groups whose kept-query ranks differ from the oracle's own
    run, and the number of boundary swaps."""
    import oracle
    b, nq, bcp, _ = qn.shape
    nkv = kn.shape[1]
    G = nq // nkv
    ref_qidx, ref_sq = oracle.select_queries(qn, nq_keep)
    gpu_sq = np.asarray(gpu_sq, dtype=np.float64)
    err_sq = float(np.abs(gpu_sq - ref_sq).max())
    assert err_sq <= SCORE_TOL, f"{what}: SQ error {err_sq}"
    gi = np.asarray(gpu_qidx, dtype=np.int64)
    rank_tol = 2.0 * err_sq + 1e-7
    for bi in range(b):
        for h in range(nq):
            assert_set_within_boundary(gi[bi, h], ref_qidx[bi, h], ref_sq[bi, h], nq_keep,
                                       what=f"{what} qidx b{bi} h{h}")
            inv = np.diff(ref_sq[bi, h][gi[bi, h]])
            assert np.all(inv <= rank_tol), \
                f"{what} b{bi} h{h}: kept queries out of SQ order by {inv.max():.3e} > {rank_tol:.3e}"
    groups_differ = int((~group_agreement(gi, ref_qidx, G)).sum())

    keys = oracle.scoring_keys_e4m3(kn[:, :, :t_past]) if k_e4m3 else kn
    if score == "cosine":
        qg = oracle.group_queries(qn, gi, nkv)
        _, s_agg = oracle.key_scores(qg, keys, t_past)
    else:
        qg = oracle.group_queries_dot(qn, gi, nkv)
        _, s_agg = oracle.key_scores_dot(qg, keys, t_past)
    g_s = np.asarray(gpu_s_agg, dtype=np.float64)[..., :t_past]
    err = np.abs(g_s - s_agg)
    if score == "cosine":
        err_s = float(err.max()) if err.size else 0.0
        assert err_s <= SCORE_TOL, f"{what}: S_agg error {err_s}"
        tols = np.full((b, nkv), BOUNDARY_TOL)
    else:
        bound = np.matmul(np.abs(qg), np.swapaxes(np.abs(keys[:, :, :t_past]), -1, -2)).max(axis=2)
        err_s = float((err / bound).max()) if err.size else 0.0
        assert err_s <= 3e-5, f"{what}: relative dot-product S_agg error {err_s}"
        tols = np.maximum(BOUNDARY_TOL, 3e-5 * bound.max(axis=-1))

    gidx = np.asarray(gpu_idx, dtype=np.int64)
    swaps = 0
    key_sets = []
    if round_off is not None:
        off = np.asarray(round_off, dtype=np.int64)
        R = len(off) - 1
        s_round = oracle.round_scores(s_agg, off)
        lens = np.asarray(gpu_sel_len, dtype=np.int64)
        for bi in range(b):
            row = []
            for j in range(nkv):
                sel = gidx[bi, j, :lens[bi, j]]
                if len(sel):
                    assert_sorted_unique(sel, t_past)
                got = np.unique(np.searchsorted(off, sel, side="right") - 1)
                assert R - 1 in got, f"{what} b{bi} j{j}: latest round missing"
                assert lens[bi, j] == sum(int(off[r + 1] - off[r]) for r in got), "partial rounds"
                if shared_rounds:  # ranked by the maximum over the sequence's heads
                    want = oracle.select_rounds_shared(s_round[bi:bi + 1], top_rounds)[0][j]
                    rank_by = s_round[bi, :, :R - 1].max(axis=0)
                else:
                    want = oracle.select_rounds(s_round[bi:bi + 1, j:j + 1], top_rounds)[0][0]
                    rank_by = s_round[bi, j, :R - 1]
                swaps += assert_set_within_boundary(got[got != R - 1], want[want != R - 1],
                                                    rank_by, top_rounds,
                                                    what=f"{what} rounds b{bi} j{j}")
                row.append(sel)
            key_sets.append(row)
    else:
        kidx = oracle.select_keys(s_agg, bsa)
        n_sel = min(bsa, t_past)
        for bi in range(b):
            row = []
            for j in range(nkv):
                sel = gidx[bi, j, :n_sel]
                if n_sel:
                    assert_sorted_unique(sel, t_past)
                swaps += assert_set_within_boundary(sel, kidx[bi, j], s_agg[bi, j], n_sel,
                                                    tol=float(tols[bi, j]),
                                                    what=f"{what} kidx b{bi} j{j}")
                row.append(sel)
            key_sets.append(row)
    stats = dict(err_sq=err_sq, err_s_agg=err_s, groups_differ=groups_differ,
                 groups=b * nkv, swaps=swaps)
    return key_sets, stats


def staged_attention(qn, kn, vn, t_past, key_sets, gpu_out, dtype, gpu_lse=None, rows=None,
                     heads=None, what=""):
    """The oracle's attention over the GPU's own key sets, against the GPU's
    output (every row and head unless rows / heads restrict it); returns the
    max error."""
    import oracle
    o_ref, lse_ref = oracle.attention(qn, kn, vn, t_past, key_sets, rows=rows, heads=heads)
    got = np64(gpu_out)
    if heads is not None:
        got = got[:, heads]
    if rows is not None:
        got = got[:, :, rows]
    err = float(np.abs(got - o_ref).max()) if o_ref.size else 0.0
    assert err <= ATTN_TOL[dtype], f"{what}: attention error {err}"
    if gpu_lse is not None:
        gl = np64(gpu_lse)
        if heads is not None:
            gl = gl[:, heads]
        if rows is not None:
            gl = gl[:, :, rows]
        err_l = float(np.abs(gl - lse_ref).max()) if lse_ref.size else 0.0
        assert err_l <= LSE_TOL[dtype], f"{what}: log-sum-exp error {err_l}"
    return err
