"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (fixed by the method's statement of the target):
  * fp32 scores (SQ, S_agg, round scores): |delta| <= 1e-3
  * top-NQ / top-BSA / round index sets: identical except items whose oracle
    score lies within 2e-3 of the oracle's k-th value
  * attention output: max |delta| <= 2e-2 (bf16), <= 1e-4 (fp32)
"""
import numpy as np
import torch

SCORE_TOL = 1e-3
BOUNDARY_TOL = 2e-3
ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}
LSE_TOL = {"bf16": 2e-3, "f32": 1e-4}


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
