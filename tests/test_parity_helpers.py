"""The staged GPU-vs-oracle comparison (tests/parity.py) checked on the CPU:
fed the oracle's own run it passes; fed a legitimate near-tie reordering of
kept queries it passes (the scores are recomputed on that order); fed each of
several planted mistakes it fails."""
import numpy as np
import pytest

import oracle
import workloads as W
from parity import np64, staged_attention, staged_selection


def _case():
    spec = W.spec("llama3b_32k", nq=6, nkv=2, t_past=700, bcp=64, nq_keep=12, bsa=150)
    case = W.make_case(spec, 77)
    qn, kn, vn = np64(case["q"]), np64(case["k"]), np64(case["v"])
    # head 0: the chunk's queries in mirror pairs (x, R x), R the reflection
    # about a fixed unit u.  The mean lies along u, so both queries of a pair
    # have the same cosine to it: ties (up to rounding) between different
    # vectors, which the two sides may rank either way.
    rng = np.random.default_rng(5)
    u = rng.standard_normal(spec.d)
    u /= np.linalg.norm(u)
    x = rng.standard_normal((spec.bcp // 2, spec.d)) + 0.5 * u
    qn[0, 0, 0::2] = x
    qn[0, 0, 1::2] = 2.0 * (x @ u)[:, None] * u[None, :] - x
    ref = oracle.pipeline(qn, kn, vn, spec.t_past, spec.nq_keep, spec.bsa)
    return spec, qn, kn, vn, ref


def _run(spec, qn, kn, vn, sq, qidx, s_agg, kidx, out):
    sets, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, spec.bsa, sq, qidx, s_agg, kidx)
    err = staged_attention(qn, kn, vn, spec.t_past, sets, out, "bf16")
    return st, err


def test_oracle_run_passes():
    spec, qn, kn, vn, ref = _case()
    st, err = _run(spec, qn, kn, vn, ref["sq"], ref["qidx"], ref["s_agg"], ref["kidx"], ref["o"])
    assert st["swaps"] == 0 and st["groups_differ"] == 0 and err < 1e-12


def test_near_tie_reordering_is_staged_not_skipped():
    """Swap the ranks of the two tied queries in head 0: the group means pair
    differently, the scores of that KV group change, and the staged check
    (which recomputes them on the swapped order) still passes, while the
    oracle's own scores for that group no longer match the swapped run."""
    spec, qn, kn, vn, ref = _case()
    qidx = ref["qidx"].copy()
    row = qidx[0, 0]
    # a kept pair (2m, 2m + 1) at adjacent ranks: swap their ranks
    n = next(n for n in range(spec.nq_keep - 1) if row[n] // 2 == row[n + 1] // 2)
    row[n], row[n + 1] = row[n + 1], row[n]
    assert abs(ref["sq"][0, 0, row[n]] - ref["sq"][0, 0, row[n + 1]]) < 1e-12
    qg = oracle.group_queries(qn, qidx, spec.nkv)
    _, s_agg = oracle.key_scores(qg, kn, spec.t_past)
    assert np.abs(s_agg - ref["s_agg"]).max() > 1e-4   # the pairing matters
    kidx = oracle.select_keys(s_agg, spec.bsa)
    sets = [[kidx[0, j] for j in range(spec.nkv)]]
    o, _ = oracle.attention(qn, kn, vn, spec.t_past, sets)
    st, err = _run(spec, qn, kn, vn, ref["sq"], qidx, s_agg, kidx, o)
    assert st["groups_differ"] == 1


@pytest.mark.parametrize("mistake", ["s_agg", "kidx", "order", "attention", "sq"])
def test_planted_mistakes_fail(mistake):
    spec, qn, kn, vn, ref = _case()
    sq, qidx, s_agg, kidx, out = (ref["sq"].copy(), ref["qidx"].copy(), ref["s_agg"].copy(),
                                  ref["kidx"].copy(), ref["o"].copy())
    if mistake == "s_agg":      # one group's scores off by 2e-3
        s_agg[0, 1] += 2e-3
    elif mistake == "kidx":     # a key far below the boundary replaces a selected one
        worst = int(np.argmin(ref["s_agg"][0, 0]))
        kidx[0, 0, -1] = worst
        kidx[0, 0] = np.sort(kidx[0, 0])
    elif mistake == "order":    # the first and last kept queries of a head swapped
        qidx[0, 1, [0, -1]] = qidx[0, 1, [-1, 0]]
    elif mistake == "attention":
        out[0, 3, 7, 11] += 3e-2
    else:                       # SQ of one query off by 2e-3
        sq[0, 2, 4] += 2e-3
    with pytest.raises(AssertionError):
        _run(spec, qn, kn, vn, sq, qidx, s_agg, kidx, out)
