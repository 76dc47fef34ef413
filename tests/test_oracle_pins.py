"""Pins for the fp64 CPU oracle: each check ties an oracle function to something
other than itself -- a hand-derived worked example, a closed form, an
invariant the pages state, a special case that reduces to a library routine, or
brute force written independently in plain Python loops.

The mutation check at the end plants typical mistakes in copies of the oracle
and asserts that some pin catches each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import quoka as Q

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# helpers (independent of the oracle's arithmetic)
# ----------------------------------------------------------------------------
def _eval_expr(expr, env):
    ns = {"sqrt": math.sqrt, "exp": math.exp, "log": math.log, "__builtins__": {}}
    ns.update(env)
    return float(eval(expr, ns))  # fixture expressions only: numbers, names, + - * / ( )


def _eval_tree(x, env):
    if isinstance(x, list):
        return [_eval_tree(e, env) for e in x]
    if isinstance(x, str):
        return _eval_expr(x, env)
    return float(x)


def _load_worked():
    with open(os.path.join(HERE, "golden", "quoka_2d_worked.json")) as f:
        g = json.load(f)
    env = {}
    for name, expr, _why in g["defs"]:
        env[name] = _eval_expr(expr, env)
    return g, env


def _py_dot(a, b):
    return sum(x * y for x, y in zip(a, b))


def _py_norm(a):
    return math.sqrt(sum(x * x for x in a))


def _py_cos(a, b):
    return _py_dot(a, b) / (_py_norm(a) * _py_norm(b))


def _brute_rank(scores):
    """positions sorted by (score desc, position asc) using Python's own sort"""
    return sorted(range(len(scores)), key=lambda i: (-scores[i], i))


def _brute_pipeline_scores(q, k, t_past, nq_keep, nkv):
    """S_agg by brute force in pure Python: per-head cosines of the kept
    queries with every key, mean over the heads of the group slot by slot,
    then max over slots."""
    b, nq, bcp, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    G = nq // nkv
    out = []
    for bi in range(b):
        row_b = []
        for j in range(nkv):
            kept = []  # kept[g][n] = query vector
            for g in range(G):
                h = j * G + g
                qs = q[bi][h]
                mq = [sum(qs[i][e] for i in range(bcp)) / bcp for e in range(d)]
                sq = [-_py_cos(qs[i], mq) for i in range(bcp)]
                order = _brute_rank(sq)[:nq_keep]
                kept.append([qs[i] for i in order])
            s_agg = []
            for t in range(t_past):
                best = -float("inf")
                for n in range(nq_keep):
                    cos_mean = sum(_py_cos(kept[g][n], k[bi][j][t]) for g in range(G)) / G
                    best = max(best, cos_mean)
                s_agg.append(best)
            row_b.append(s_agg)
        out.append(row_b)
    return np.array(out)


def _py_attention_row(qv, keys, vals, scale):
    """two-pass softmax attention of one query over explicit key/value lists"""
    logits = [scale * _py_dot(qv, kk) for kk in keys]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    z = sum(w)
    o = [sum(w[i] * vals[i][e] for i in range(len(vals))) / z for e in range(len(vals[0]))]
    return o, m + math.log(z)


def _rand_case(rng, b=1, nq=4, nkv=2, d=6, t=12, bcp=5, extra=0):
    q = rng.standard_normal((b, nq, bcp, d)) + 1.5 * rng.standard_normal((b, nq, 1, d))
    k = rng.standard_normal((b, nkv, t + bcp + extra, d))
    v = rng.standard_normal((b, nkv, t + bcp + extra, d))
    return q, k, v


# ----------------------------------------------------------------------------
# 1. the hand-derived worked example
# ----------------------------------------------------------------------------
def test_worked_example_selection():
    g, env = _load_worked()
    q, k = np.array(g["q"], float), np.array(g["k"], float)
    sh, ex = g["shape"], g["expected"]
    np.testing.assert_allclose(Q.mean_query(q), _eval_tree(ex["mq"], env), atol=1e-15)
    np.testing.assert_allclose(Q.query_scores(q), _eval_tree(ex["sq"], env), atol=1e-15)
    qidx, _ = Q.select_queries(q, sh["nq_keep"])
    assert qidx.tolist() == ex["qidx"]
    qg = Q.group_queries(q, qidx, sh["nkv"])
    np.testing.assert_allclose(qg, _eval_tree(ex["q_group"], env), atol=1e-15)
    s, s_agg = Q.key_scores(qg, k, sh["t_past"])
    np.testing.assert_allclose(s, _eval_tree(ex["s"], env), atol=1e-15)
    np.testing.assert_allclose(s_agg, _eval_tree(ex["s_agg"], env), atol=1e-15)
    assert Q.select_keys(s_agg, sh["bsa"]).tolist() == ex["kidx"]


def test_worked_example_attention():
    g, env = _load_worked()
    q, k, v = (np.array(g[n], float) for n in ("q", "k", "v"))
    sh, ex = g["shape"], g["expected"]
    out = Q.pipeline(q, k, v, sh["t_past"], sh["nq_keep"], sh["bsa"])
    for item in ex["attention"]:
        e = dict(env)
        e["Z"] = _eval_expr(item["Z"], e)
        h, i = item["head"], item["row"]
        np.testing.assert_allclose(out["o"][0, h, i], _eval_tree(item["o"], e), atol=1e-14)
        assert abs(out["lse"][0, h, i] - _eval_expr(item["lse"], e)) < 1e-14
    o_d, lse_d = Q.dense_attention(q, k, v, sh["t_past"])
    for item in ex["dense_attention"]:
        e = dict(env)
        e["Z"] = _eval_expr(item["Z"], e)
        h, i = item["head"], item["row"]
        np.testing.assert_allclose(o_d[0, h, i], _eval_tree(item["o"], e), atol=1e-14)
        assert abs(lse_d[0, h, i] - _eval_expr(item["lse"], e)) < 1e-14


def test_worked_example_rounds():
    g, env = _load_worked()
    q, k, v = (np.array(g[n], float) for n in ("q", "k", "v"))
    sh, ex = g["shape"], g["expected"]
    out = Q.pipeline(q, k, v, sh["t_past"], sh["nq_keep"], round_off=g["round_off"],
                     top_rounds=g["top_rounds"], with_attention=False)
    np.testing.assert_allclose(out["s_round"], _eval_tree(ex["s_round"], env), atol=1e-15)
    assert [[r.tolist() for r in row] for row in out["rounds"]] == ex["rounds"]
    assert [[p.tolist() for p in row] for row in out["key_sets"]] == ex["round_positions"]


# ----------------------------------------------------------------------------
# 2. query scores: range, special cases, 2-D closed form
# ----------------------------------------------------------------------------
def test_sq_range_and_bcp1():
    rng = np.random.default_rng(1)
    q = 3 * rng.standard_normal((2, 4, 33, 16))
    sq = Q.query_scores(q)
    assert sq.shape == (2, 4, 33)
    assert np.all(sq >= -1 - 1e-12) and np.all(sq <= 1 + 1e-12)
    one = Q.query_scores(q[:, :, :1])           # a single query is its own mean
    np.testing.assert_allclose(one, -1.0, atol=1e-15)


def test_sq_equal_queries_and_ties():
    rng = np.random.default_rng(2)
    row = rng.standard_normal(8)
    q = np.tile(row, (1, 3, 10, 1))
    sq = Q.query_scores(q)
    np.testing.assert_allclose(sq, -1.0, atol=1e-15)
    qidx, _ = Q.select_queries(q, 4)
    assert qidx.tolist() == [[[0, 1, 2, 3]] * 3]  # exact ties: lower positions


def test_sq_positive_multiple_of_mean():
    # queries c_i * w (c_i > 0) all have the mean's direction: SQ = -1 each
    rng = np.random.default_rng(3)
    w = rng.standard_normal(5)
    c = rng.uniform(0.5, 3.0, size=7)
    q = (c[:, None] * w[None, :])[None, None]
    np.testing.assert_allclose(Q.query_scores(q), -1.0, atol=1e-14)


def test_sq_2d_closed_form():
    # symmetric pairs at angles phi0 +- delta_i with equal norms per pair put the
    # mean exactly along phi0, so SQ_i = -cos(delta_i) for both members
    phi0 = 0.7
    deltas = [0.1, 0.9, 2.0, 2.8]
    norms = [1.0, 2.5, 0.3, 0.5]   # sum of r*cos(delta) > 0: the mean points along phi0
    qs, want = [], []
    for dl, r in zip(deltas, norms):
        for sgn in (1, -1):
            a = phi0 + sgn * dl
            qs.append([r * math.cos(a), r * math.sin(a)])
            want.append(-math.cos(dl))
    q = np.array(qs)[None, None]
    np.testing.assert_allclose(Q.query_scores(q)[0, 0], want, atol=1e-14)
    # the top-2 are the pair with the widest angle (2.8), lower position first
    qidx, _ = Q.select_queries(q, 2)
    assert qidx[0, 0].tolist() == [6, 7]


def test_mean_query_axis():
    # the mean runs over the token axis, separately per head and per sequence
    q = np.zeros((2, 3, 4, 2))
    for bi in range(2):
        for h in range(3):
            q[bi, h, :, 0] = [1, 2, 3, 4 + 10 * bi + h]
    mq = Q.mean_query(q)
    for bi in range(2):
        for h in range(3):
            assert mq[bi, h, 0] == (1 + 2 + 3 + 4 + 10 * bi + h) / 4
            assert mq[bi, h, 1] == 0


# ----------------------------------------------------------------------------
# 3. top-k: brute force, set properties, degenerate k
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (40, 40), (64, 10), (100, 1)])
def test_topk_bruteforce(n, k):
    rng = np.random.default_rng(n * 100 + k)
    s = rng.integers(-4, 5, size=n).astype(float) / 4   # many exact ties
    got = Q.topk_order(s, k)
    assert got.tolist() == _brute_rank(list(s))[:k]
    chosen = set(got.tolist())
    rest = [s[i] for i in range(n) if i not in chosen]
    if rest:
        assert min(s[list(chosen)]) >= max(rest)


def test_topk_threshold_count_crosscheck():
    # independent check with np.partition: the k-th largest value is the
    # threshold; everything strictly above it is chosen, and the ties at it are
    # filled in position order
    rng = np.random.default_rng(5)
    s = np.round(rng.standard_normal(5000), 2)
    k = 777
    thr = np.partition(s, len(s) - k)[len(s) - k]
    above = np.flatnonzero(s > thr)
    ties = np.flatnonzero(s == thr)[: k - len(above)]
    want = np.sort(np.concatenate([above, ties]))
    got = Q.select_keys(s[None, None], k)[0, 0]
    assert got.tolist() == want.tolist()


def test_select_keys_all_and_clamp():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((2, 3, 50))
    assert Q.select_keys(s, 50).tolist() == [[list(range(50))] * 3] * 2
    assert Q.select_keys(s, 80).shape == (2, 3, 50)   # BSA > T clamps to T
    qidx, _ = Q.select_queries(rng.standard_normal((1, 2, 9, 4)), 9)
    assert sorted(qidx[0, 0].tolist()) == list(range(9))   # NQ = bcp keeps all


# ----------------------------------------------------------------------------
# 4. normalise + group mean + score + max: brute force, closed forms, invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("nq,nkv,nq_keep", [(4, 2, 3), (6, 2, 2), (2, 2, 4), (3, 1, 1), (8, 2, 5)])
def test_scores_bruteforce(nq, nkv, nq_keep):
    rng = np.random.default_rng(nq * 10 + nkv + nq_keep)
    b, d, t, bcp = 2, 5, 11, 6
    q, k, _ = _rand_case(rng, b=b, nq=nq, nkv=nkv, d=d, t=t, bcp=bcp)
    qidx, _ = Q.select_queries(q, nq_keep)
    _, s_agg = Q.key_scores(Q.group_queries(q, qidx, nkv), k, t)
    want = _brute_pipeline_scores(q.tolist(), k.tolist(), t, nq_keep, nkv)
    np.testing.assert_allclose(s_agg, want, atol=1e-12)


def test_group_mean_g1_and_unit_norm():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 3, 8, 5))
    qidx, _ = Q.select_queries(q, 4)
    qg = Q.group_queries(q, qidx, 3)                     # G = 1
    for h in range(3):
        for n in range(4):
            vec = q[0, h, qidx[0, h, n]]
            np.testing.assert_allclose(qg[0, h, n], vec / _py_norm(vec), atol=1e-15)
    assert np.all(np.linalg.norm(Q.group_queries(q, qidx, 1), axis=-1) <= 1 + 1e-12)


def test_key_score_closed_forms():
    rng = np.random.default_rng(8)
    q, k, _ = _rand_case(rng, nq=6, nkv=2, d=7, t=9, bcp=8)
    qidx, _ = Q.select_queries(q, 3)
    qg = Q.group_queries(q, qidx, 2)
    # a key along Q_group[n] scores |Q_group[n]| against that slot
    k2 = k.copy()
    k2[0, 1, 4] = 2.5 * qg[0, 1, 2]
    s, s_agg = Q.key_scores(qg, k2, 9)
    assert abs(s[0, 1, 2, 4] - np.linalg.norm(qg[0, 1, 2])) < 1e-14
    assert np.all(np.abs(s) <= 1 + 1e-12)
    # scaling keys by positive factors leaves every score unchanged
    c = rng.uniform(0.1, 10, size=k.shape[:3] + (1,))
    _, s_agg_c = Q.key_scores(qg, k * c, 9)
    _, s_agg_0 = Q.key_scores(qg, k, 9)
    np.testing.assert_allclose(s_agg_c, s_agg_0, atol=1e-14)
    # one kept query: S_agg is S itself
    s1, a1 = Q.key_scores(qg[:, :, :1], k, 9)
    np.testing.assert_allclose(a1, s1[:, :, 0], atol=0)


def test_zero_norm_clamp():
    q = np.zeros((1, 1, 3, 4))
    q[0, 0, 1] = [1, 0, 0, 0]
    sq = Q.query_scores(q)
    assert np.all(np.isfinite(sq))
    k = np.zeros((1, 1, 5, 4))
    qidx, _ = Q.select_queries(q, 2)
    _, s_agg = Q.key_scores(Q.group_queries(q, qidx, 1), k, 4)
    assert np.all(s_agg == 0)


# ----------------------------------------------------------------------------
# 5. attention: independent loop formulation, library routine, invariants
# ----------------------------------------------------------------------------
def test_attention_vs_python_loops():
    rng = np.random.default_rng(9)
    b, nq, nkv, d, t, bcp = 2, 4, 2, 5, 10, 4
    q, k, v = _rand_case(rng, b=b, nq=nq, nkv=nkv, d=d, t=t, bcp=bcp, extra=2)
    sets = [[np.sort(rng.choice(t, size=rng.integers(1, t + 1), replace=False))
             for _ in range(nkv)] for _ in range(b)]
    scale = 0.37
    o, lse = Q.attention(q, k, v, t, sets, scale=scale)
    G = nq // nkv
    for bi in range(b):
        for h in range(nq):
            j = h // G
            for i in range(bcp):
                ids = list(sets[bi][j]) + [t + u for u in range(i + 1)]
                keys = [k[bi, j, p].tolist() for p in ids]
                vals = [v[bi, j, p].tolist() for p in ids]
                oo, ll = _py_attention_row(q[bi, h, i].tolist(), keys, vals, scale)
                np.testing.assert_allclose(o[bi, h, i], oo, atol=1e-13)
                assert abs(lse[bi, h, i] - ll) < 1e-13


def test_dense_attention_vs_torch_sdpa():
    rng = np.random.default_rng(10)
    b, nq, nkv, d, t, bcp = 1, 6, 2, 8, 20, 7
    q, k, v = _rand_case(rng, b=b, nq=nq, nkv=nkv, d=d, t=t, bcp=bcp)
    o, _ = Q.dense_attention(q, k, v, t)
    G = nq // nkv
    kt = torch.from_numpy(k[:, :, : t + bcp]).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v[:, :, : t + bcp]).repeat_interleave(G, dim=1)
    qt = torch.from_numpy(q)
    # bottom-right aligned causal mask: query i sees keys 0 .. t + i
    mask = torch.arange(t + bcp)[None, :] <= (t + torch.arange(bcp))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    np.testing.assert_allclose(o, ref.numpy(), atol=1e-12)


def test_sparse_equals_dense_when_bsa_is_t():
    rng = np.random.default_rng(11)
    q, k, v = _rand_case(rng, b=1, nq=4, nkv=2, d=6, t=15, bcp=5)
    out = Q.pipeline(q, k, v, 15, nq_keep=2, bsa=15)
    o_d, lse_d = Q.dense_attention(q, k, v, 15)
    np.testing.assert_allclose(out["o"], o_d, atol=1e-12)
    np.testing.assert_allclose(out["lse"], lse_d, atol=1e-12)


def test_attention_special_cases():
    rng = np.random.default_rng(12)
    q, k, v = _rand_case(rng, b=1, nq=2, nkv=1, d=4, t=6, bcp=3)
    empty = [[np.array([], dtype=np.int64)]]
    o, lse = Q.attention(q, k, v, 6, empty)
    np.testing.assert_allclose(o[0, :, 0], np.tile(v[0, 0, 6], (2, 1)), atol=1e-15)  # one key
    # Q = 0: uniform weights, mean of the attended rows, LSE = log(count)
    sets = [[np.array([0, 2, 5])]]
    o0, lse0 = Q.attention(np.zeros_like(q), k, v, 6, sets)
    for i in range(3):
        ids = [0, 2, 5] + [6 + u for u in range(i + 1)]
        np.testing.assert_allclose(o0[0, 0, i], v[0, 0, ids].mean(axis=0), atol=1e-15)
        assert abs(lse0[0, 0, i] - math.log(len(ids))) < 1e-15
    # convex hull of the attended values
    o1, _ = Q.attention(5 * q, k, v, 6, sets)
    for i in range(3):
        ids = [0, 2, 5] + [6 + u for u in range(i + 1)]
        lo, hi = v[0, 0, ids].min(axis=0), v[0, 0, ids].max(axis=0)
        assert np.all(o1[0, :, i] >= lo - 1e-12) and np.all(o1[0, :, i] <= hi + 1e-12)


def test_attention_row_and_head_subsets():
    rng = np.random.default_rng(13)
    q, k, v = _rand_case(rng, b=1, nq=4, nkv=2, d=5, t=9, bcp=6)
    sets = [[np.array([1, 3, 4]), np.array([0, 8])]]
    o, lse = Q.attention(q, k, v, 9, sets)
    o2, lse2 = Q.attention(q, k, v, 9, sets, rows=[5, 1], heads=[3, 0])
    np.testing.assert_allclose(o2[0, 0, 0], o[0, 3, 5], atol=0)
    np.testing.assert_allclose(o2[0, 1, 1], o[0, 0, 1], atol=0)
    assert lse2[0, 0, 1] == lse[0, 3, 1]


# ----------------------------------------------------------------------------
# 6. round selection
# ----------------------------------------------------------------------------
def test_rounds_bruteforce_and_limits():
    rng = np.random.default_rng(14)
    t = 40
    s_agg = rng.standard_normal((1, 2, t))
    off = np.array([0, 3, 10, 11, 25, 33, 40])
    sr = Q.round_scores(s_agg, off)
    for j in range(2):
        for r in range(6):
            assert sr[0, j, r] == max(s_agg[0, j, off[r]:off[r + 1]].tolist())
    chosen = Q.select_rounds(sr, 2)
    for j in range(2):
        rest = _brute_rank(list(sr[0, j, :5]))[:2]
        assert chosen[0][j].tolist() == sorted(rest + [5])
    # keeping every round is the dense key set
    sets = Q.round_key_sets(Q.select_rounds(sr, 5), off)
    assert all(s.tolist() == list(range(t)) for s in sets[0])
    # every token its own round: rounds reduce to token top-k with the last
    # position forced in
    off1 = np.arange(t + 1)
    sets1 = Q.round_key_sets(Q.select_rounds(Q.round_scores(s_agg, off1), 7), off1)
    for j in range(2):
        want = sorted(_brute_rank(list(s_agg[0, j, : t - 1]))[:7] + [t - 1])
        assert sets1[0][j].tolist() == want


def test_rounds_shared_by_the_heads():
    """The head-shared round choice: a hand-worked case (the shared score is
    the per-round maximum over the heads: (0.45, 0.5, 0.45) over the first
    three rounds, so round 1 joins the latest; per head the choices differ),
    one KV head reducing to the per-head choice, and on random scores the
    brute-force ranking of the per-round maxima."""
    sr = np.array([[[0.1, 0.5, 0.45, 0.0], [0.45, 0.1, 0.4, 0.9]]])
    assert [c.tolist() for c in Q.select_rounds(sr, 1)[0]] == [[1, 3], [0, 3]]
    assert [c.tolist() for c in Q.select_rounds_shared(sr, 1)[0]] == [[1, 3], [1, 3]]
    assert [c.tolist() for c in Q.select_rounds_shared(sr, 2)[0]] == [[0, 1, 3], [0, 1, 3]]
    rng = np.random.default_rng(41)
    one = rng.standard_normal((2, 1, 9))
    for keep in (True, False):
        a, b = Q.select_rounds(one, 3, keep), Q.select_rounds_shared(one, 3, keep)
        assert all(np.array_equal(a[i][0], b[i][0]) for i in range(2))
    x = np.round(rng.standard_normal((3, 4, 10)), 1)  # ties between rounds
    got = Q.select_rounds_shared(x, 4)
    for bi in range(3):
        m = [max(x[bi, j, r] for j in range(4)) for r in range(10)]
        want = sorted(_brute_rank(m[:9])[:4] + [9])
        assert all(g.tolist() == want for g in got[bi])


# ----------------------------------------------------------------------------
# 7. the pins catch planted mistakes
# ----------------------------------------------------------------------------
# ----------------------------------------------------------------------------
# scoring variants: E4M3 keys and dot-product scores
# ----------------------------------------------------------------------------
def _brute_dot_scores(q, k, qidx, t_past, nkv):
    """S_agg of the dot-product variant by plain loops: per slot n the mean over
    the group's heads of the raw kept queries, dotted with the raw keys, then
    the max over slots."""
    b, nq, d = len(q), len(q[0]), len(q[0][0][0])
    G = nq // nkv
    n_keep = len(qidx[0][0])
    out = []
    for bi in range(b):
        rows = []
        for j in range(nkv):
            row = []
            for t in range(t_past):
                best = -math.inf
                for n in range(n_keep):
                    tot = 0.0
                    for e in range(d):
                        avg = sum(q[bi][j * G + g][qidx[bi][j * G + g][n]][e] for g in range(G)) / G
                        tot += avg * k[bi][j][t][e]
                    best = max(best, tot)
                row.append(best)
            rows.append(row)
        out.append(rows)
    return np.array(out)


def test_e4m3_code_table():
    # values fixed by the OCP 8-bit floating point specification, E4M3 column
    assert Q.e4m3_decode(0x7E) == 448.0                 # largest finite, S.1111.110
    assert Q.e4m3_decode(0x08) == 2.0 ** -6             # smallest normal, S.0001.000
    assert Q.e4m3_decode(0x07) == 0.875 * 2.0 ** -6     # largest subnormal, S.0000.111
    assert Q.e4m3_decode(0x01) == 2.0 ** -9             # smallest subnormal
    assert Q.e4m3_decode(0x38) == 1.0 and Q.e4m3_decode(0xB8) == -1.0
    assert np.isnan(Q.e4m3_decode(0x7F)) and np.isnan(Q.e4m3_decode(0xFF))
    z = Q.e4m3_decode(0x80)
    assert z == 0.0 and np.signbit(z)
    assert np.all(np.diff(Q.e4m3_decode(np.arange(0x7F))) > 0)
    # every code against torch's float8_e4m3fn, an independent implementation
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = Q.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], got[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(got[fin]))


def test_e4m3_encode_rounding():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert np.array_equal(Q.e4m3_encode(Q.e4m3_decode(codes)), codes.astype(np.uint8))
    # midpoints of neighbouring magnitudes go to the even code; points just off
    # a midpoint go to the nearer code
    mags = Q.e4m3_decode(np.arange(0x7F))
    mid = (mags[:-1] + mags[1:]) / 2
    lo = np.arange(0x7E)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(Q.e4m3_encode(mid), even.astype(np.uint8))
    assert np.array_equal(Q.e4m3_encode(-mid), (even | 0x80).astype(np.uint8))
    off = (mags[1:] - mags[:-1]) * 1e-3
    assert np.array_equal(Q.e4m3_encode(mid - off), lo.astype(np.uint8))
    assert np.array_equal(Q.e4m3_encode(mid + off), (lo + 1).astype(np.uint8))
    # saturation above 448, signed zero
    assert Q.e4m3_encode(1e6) == 0x7E and Q.e4m3_encode(-1e6) == 0xFE
    assert Q.e4m3_encode(464.0) == 0x7E and Q.e4m3_encode(470.0) == 0x7E
    assert Q.e4m3_encode(-1e-30) == 0x80 and Q.e4m3_encode(0.0) == 0x00
    # within range, against torch's round-to-nearest-even conversion from fp32
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 4, rng.standard_normal(5000) * 0.01,
                        rng.uniform(-460, 460, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(Q.e4m3_encode(x), ref)


def test_dot_scores_bruteforce_and_links():
    rng = np.random.default_rng(6)
    q, k, _ = _rand_case(rng, b=2, nq=6, nkv=2, d=5, t=9, bcp=6)
    qi, _ = Q.select_queries(q, 3)
    _, sa = Q.key_scores_dot(Q.group_queries_dot(q, qi, 2), k, 9)
    assert np.allclose(sa, _brute_dot_scores(q.tolist(), k.tolist(), qi.tolist(), 9, 2), atol=1e-12)
    # G = 1: the group queries are the kept rows themselves
    qi1, _ = Q.select_queries(q, 2)
    g1 = Q.group_queries_dot(q, qi1, 6)
    assert np.array_equal(g1, np.take_along_axis(q, qi1[..., None], axis=2))
    # on unit-norm queries and keys the dot variant equals the cosine scores
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    _, sa_cos = Q.key_scores(Q.group_queries(qn, qi, 2), kn, 9)
    _, sa_dot = Q.key_scores_dot(Q.group_queries_dot(qn, qi, 2), kn, 9)
    assert np.allclose(sa_cos, sa_dot, atol=1e-14)
    # scaling the keys by c > 0 scales the dot scores by c, not the cosine ones
    _, sa2 = Q.key_scores_dot(Q.group_queries_dot(q, qi, 2), 3.0 * k, 9)
    assert np.allclose(sa2, 3.0 * sa, atol=1e-12)
    _, c1 = Q.key_scores(Q.group_queries(q, qi, 2), k, 9)
    _, c3 = Q.key_scores(Q.group_queries(q, qi, 2), 3.0 * k, 9)
    assert np.allclose(c1, c3, atol=1e-14)


def test_pipeline_variants_compose():
    rng = np.random.default_rng(7)
    q, k, v = _rand_case(rng, b=1, nq=4, nkv=2, d=6, t=20, bcp=5)
    out = Q.pipeline(q, k, v, 20, 3, 7, score="dot", with_attention=False)
    _, sa = Q.key_scores_dot(Q.group_queries_dot(q, out["qidx"], 2), k, 20)
    assert np.array_equal(out["s_agg"], sa)
    assert np.array_equal(out["kidx"], Q.select_keys(sa, 7))
    out8 = Q.pipeline(q, k, v, 20, 3, 7, k_e4m3=True, with_attention=False)
    k8 = Q.e4m3_decode(Q.e4m3_encode(k[:, :, :20]))
    _, sa8 = Q.key_scores(Q.group_queries(q, out8["qidx"], 2), k8, 20)
    assert np.array_equal(out8["s_agg"], sa8)
    with pytest.raises(ValueError):
        Q.pipeline(q, k, v, 20, 3, 7, score="raw")


# ----------------------------------------------------------------------------
# whole prompts and layer stacks
# ----------------------------------------------------------------------------
def _causal_sdpa(q, k, v):
    """Causal attention of every position over the positions up to it, by
    torch's scaled_dot_product_attention (fp64, GQA heads expanded)."""
    G = q.shape[1] // k.shape[1]
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64)).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(np.asarray(v, np.float64)).repeat_interleave(G, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True).numpy()


@pytest.mark.parametrize("bcp", [3, 7, 16])
def test_prompt_full_budget_is_causal_attention(bcp):
    """With a budget covering every past position, the chunked prompt plus its
    decode steps is plain causal attention over the whole sequence, whatever
    the chunk size (a ragged last chunk included)."""
    rng = np.random.default_rng(8)
    b, nq, nkv, d, total, dec = 2, 4, 2, 8, 23, 3
    q = rng.standard_normal((b, nq, total, d))
    k = rng.standard_normal((b, nkv, total, d))
    v = rng.standard_normal((b, nkv, total, d))
    o, steps = Q.prompt_chunks(q, k, v, bcp, 2, bsa=total, n_decode=dec)
    assert np.allclose(o, _causal_sdpa(q, k, v), atol=1e-12)
    prompt = total - dec
    starts = [st["qidx"].shape[-1] for st in steps]
    assert len(steps) == -(-prompt // bcp) + dec and starts[-dec:] == [1] * dec


def test_prompt_chunk_is_pipeline_and_first_chunk_has_no_past():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 10, 6)) + 1.5 * rng.standard_normal((1, 4, 1, 6))
    k = rng.standard_normal((1, 2, 10, 6))
    v = rng.standard_normal((1, 2, 10, 6))
    o, steps = Q.prompt_chunks(q, k, v, 4, 2, bsa=3)
    # chunk 0: no past, attention over the chunk alone (causal)
    assert steps[0]["kidx"].shape == (1, 2, 0)
    assert np.allclose(o[:, :, :4], _causal_sdpa(q[:, :, :4], k[:, :, :4], v[:, :, :4]), atol=1e-12)
    # chunk 2 (positions 8, 9) is the one-chunk pipeline at t_past = 8
    r = Q.pipeline(q[:, :, 8:10], k, v, 8, 2, 3)
    assert np.array_equal(o[:, :, 8:10], r["o"])
    # decode steps are one-query chunks with NQ = 1 at their own position
    o2, steps2 = Q.prompt_chunks(q, k, v, 4, 2, bsa=3, n_decode=2)
    assert [st["qidx"].shape[-1] for st in steps2] == [2, 2, 1, 1]
    for t in (8, 9):
        assert np.array_equal(o2[:, :, t:t + 1], Q.pipeline(q[:, :, t:t + 1], k, v, t, 1, 3)["o"])


def test_layer_stack_reuse():
    rng = np.random.default_rng(10)
    L, b, nq, nkv, d, t, bcp = 4, 1, 4, 2, 6, 12, 3
    qs = [rng.standard_normal((b, nq, bcp, d)) + rng.standard_normal((b, nq, 1, d)) for _ in range(L)]
    ks = [rng.standard_normal((b, nkv, t + bcp, d)) for _ in range(L)]
    vs = [rng.standard_normal((b, nkv, t + bcp, d)) for _ in range(L)]
    outs, sets = Q.layer_stack(qs, ks, vs, t, 2, 5, watershed=1)
    # below the watershed: dense causal attention of the chunk
    full = np.concatenate([np.zeros((b, nq, t, d)), qs[0]], axis=2)
    assert np.allclose(outs[0], _causal_sdpa(full, ks[0], vs[0])[:, :, t:], atol=1e-12)
    # the watershed layer is the one-chunk pipeline; above it, its key sets
    r = Q.pipeline(qs[1], ks[1], vs[1], t, 2, 5)
    assert np.array_equal(outs[1], r["o"])
    for layer in (2, 3):
        o, _ = Q.attention(qs[layer], ks[layer], vs[layer], t, r["key_sets"])
        assert np.array_equal(outs[layer], o)
    # identical layers: the reused selection reproduces the watershed output
    outs2, _ = Q.layer_stack([qs[0]] * 3, [ks[0]] * 3, [vs[0]] * 3, t, 2, 5, watershed=0)
    assert np.array_equal(outs2[1], outs2[0]) and np.array_equal(outs2[2], outs2[0])
    with pytest.raises(ValueError):
        Q.layer_stack(qs, ks, vs, t, 2, 5, watershed=L)
    # round selection at the watershed: the layers above attend over the
    # positions of its chosen rounds
    off = np.array([0, 3, 7, 12])
    outs_r, sets_r = Q.layer_stack(qs, ks, vs, t, 2, 0, watershed=1, round_off=off, top_rounds=1)
    rr = Q.pipeline(qs[1], ks[1], vs[1], t, 2, 0, round_off=off, top_rounds=1)
    for j in range(nkv):
        assert np.array_equal(sets_r[0][j], rr["key_sets"][0][j])
        chosen = set(np.asarray(rr["rounds"][0][j]).tolist())
        assert 2 in chosen and len(chosen) == 2          # the latest round plus one
        want = np.concatenate([np.arange(off[r], off[r + 1]) for r in sorted(chosen)])
        assert np.array_equal(sets_r[0][j], want)
    o3, _ = Q.attention(qs[3], ks[3], vs[3], t, rr["key_sets"])
    assert np.array_equal(outs_r[3], o3)


def _pins_pass(mod):
    """Run a compact subset of the pins against a (possibly mutated) module."""
    g, env = _load_worked()
    q, k, v = (np.array(g[n], float) for n in ("q", "k", "v"))
    sh, ex = g["shape"], g["expected"]
    try:
        out = mod.pipeline(q, k, v, sh["t_past"], sh["nq_keep"], sh["bsa"])
        ok = np.allclose(out["sq"], _eval_tree(ex["sq"], env), atol=1e-14)
        ok &= out["qidx"].tolist() == ex["qidx"]
        ok &= np.allclose(out["s_agg"], _eval_tree(ex["s_agg"], env), atol=1e-14)
        ok &= out["kidx"].tolist() == ex["kidx"]
        for item in ex["attention"]:
            e = dict(env)
            e["Z"] = _eval_expr(item["Z"], e)
            ok &= np.allclose(out["o"][0, item["head"], item["row"]], _eval_tree(item["o"], e), atol=1e-13)
        rng = np.random.default_rng(4)
        qq, kk, _ = _rand_case(rng, b=1, nq=4, nkv=2, d=5, t=8, bcp=6)
        qi, _ = mod.select_queries(qq, 3)
        _, sa = mod.key_scores(mod.group_queries(qq, qi, 2), kk, 8)
        ok &= np.allclose(sa, _brute_pipeline_scores(qq.tolist(), kk.tolist(), 8, 3, 2), atol=1e-12)
        _, sd = mod.key_scores_dot(mod.group_queries_dot(qq, qi, 2), kk, 8)
        ok &= np.allclose(sd, _brute_dot_scores(qq.tolist(), kk.tolist(), qi.tolist(), 8, 2), atol=1e-12)
        ok &= mod.e4m3_decode(0x7E) == 448.0 and mod.e4m3_decode(0x01) == 2.0 ** -9
        qp = rng.standard_normal((1, 2, 9, 4))
        kp = rng.standard_normal((1, 1, 9, 4))
        vp = rng.standard_normal((1, 1, 9, 4))
        op, _ = mod.prompt_chunks(qp, kp, vp, 4, 2, bsa=9, n_decode=2)
        ok &= np.allclose(op, _causal_sdpa(qp, kp, vp), atol=1e-12)
        op2, _ = mod.prompt_chunks(qp, kp, vp, 4, 2, bsa=3, n_decode=2)
        for t in (7, 8):
            ok &= np.array_equal(op2[:, :, t:t + 1], mod.pipeline(qp[:, :, t:t + 1], kp, vp, t, 1, 3)["o"])
        srs = np.array([[[0.1, 0.5, 0.45, 0.0], [0.45, 0.1, 0.4, 0.9]]])
        ok &= [c.tolist() for c in mod.select_rounds_shared(srs, 1)[0]] == [[1, 3], [1, 3]]
        mags = mod.e4m3_decode(np.arange(0x7F))
        lo = np.arange(0x7E)
        ok &= np.array_equal(mod.e4m3_encode((mags[:-1] + mags[1:]) / 2),
                             np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8))
        return bool(ok)
    except Exception:
        return False


MUTATIONS = {
    "sq sign": ("return -dot / den", "return dot / den"),
    "mean over heads": ("return f64(q).mean(axis=2)", "return f64(q).mean(axis=1)[:, None].repeat(f64(q).shape[1], axis=1)[:, :, 0]"),
    "ties to higher index": ("order = np.lexsort((np.arange(n), -scores))", "order = np.lexsort((-np.arange(n), -scores))"),
    "ascending top-k": ("order = np.lexsort((np.arange(n), -scores))", "order = np.lexsort((np.arange(n), scores))"),
    "no query norm": ("q_norm = sel / np.maximum(_norm(sel), EPS)[..., None]", "q_norm = sel"),
    "strided grouping": ("return q_norm.reshape(b, nkv, G, n_keep, d).mean(axis=2)", "return q_norm.reshape(b, G, nkv, n_keep, d).mean(axis=1)"),
    "no key norm": ("k_norm = kp / np.maximum(_norm(kp), EPS)[..., None]", "k_norm = kp"),
    "mean instead of max": ("return s, s.max(axis=2)", "return s, s.mean(axis=2)"),
    "causal off by one": ("hidden = u[None, :] > rows[:, None]", "hidden = u[None, :] >= rows[:, None]"),
    "no causal mask": ("logits[:, n_past:][hidden] = -np.inf", "pass"),
    "scale dropped": ("sc = 1.0 / math.sqrt(d) if scale is None else float(scale)", "sc = 1.0"),
    "v transposed role": ("o[bi, hi] = (p @ vv) / l", "o[bi, hi] = (p @ kk) / l"),
    "e4m3 bias 8": ("normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))",
                    "normal = np.ldexp(1.0 + m / 8.0, (e - 8).astype(np.int64))"),
    "e4m3 ties up": ("np.where(lo % 2 == 0, lo, hi)", "hi"),
    "dot keeps key norm": ("s = np.matmul(f64(q_group), np.swapaxes(f64(k[:, :, :t_past]), -1, -2))",
                           "s = np.matmul(f64(q_group), np.swapaxes(f64(k[:, :, :t_past]) / _norm(f64(k[:, :, :t_past]))[..., None], -1, -2))"),
    "chunk past off by one": ("r = pipeline(q[:, :, t:t + n], k, v, t, keep, bsa, score=score, k_e4m3=k_e4m3)",
                              "r = pipeline(q[:, :, t:t + n], k, v, max(t - 1, 0), keep, bsa, score=score, k_e4m3=k_e4m3)"),
    "decode keeps the chunk rule": ("n = min(bcp, prompt - t) if t < prompt else 1",
                                    "n = min(bcp, total - t)"),
    "shared rounds by mean": ("shared = s_round.max(axis=1, keepdims=True)",
                              "shared = s_round.mean(axis=1, keepdims=True)"),
    "shared rounds by min": ("shared = s_round.max(axis=1, keepdims=True)",
                             "shared = s_round.min(axis=1, keepdims=True)"),
    "dot sums heads": ("return sel.reshape(b, nkv, G, sel.shape[2], d).mean(axis=2)",
                       "return sel.reshape(b, nkv, G, sel.shape[2], d).sum(axis=2)"),
}


def test_pins_catch_planted_mistakes():
    import importlib.util
    import types
    src = open(Q.__file__).read()
    assert _pins_pass(Q)
    for name, (old, new) in MUTATIONS.items():
        assert old in src, name
        mod = types.ModuleType("mutant")
        exec(compile(src.replace(old, new), "mutant", "exec"), mod.__dict__)
        assert not _pins_pass(mod), f"planted mistake not caught: {name}"
