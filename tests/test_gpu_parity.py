"""GPU parity: the HIP library against the fp64 CPU oracle on identical seeded
inputs, through the C ABI.

Staging runs both ways.  A GPU stage may be fed the oracle's result of the
previous stage (an oracle value going into the HIP path).  An oracle stage
may be fed the GPU's previous discrete decision (its kept query positions,
its key sets): the end-to-end checks run the oracle's group queries, key
scores, selection and attention on the GPU's own choices, so that a
legitimate swap at a near-tie never hides or fakes a value difference, and
every KV group and every output row is compared.  The oracle's own full run
fixes what the choices themselves may be (the boundary rule).  No stored
expected value comes from the HIP path.  Sizes span several tiles with
ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (ATTN_TOL, BOUNDARY_TOL, LSE_TOL, SCORE_TOL, assert_set_within_boundary,
                    assert_sorted_unique, max_abs, np64, npi, staged_attention,
                    staged_selection)

pytestmark = pytest.mark.gpu

# name -> (workload, overrides, seed)
CASES = {
    "tiny_f32": ("tiny_f32", {}, 1001),
    "llama_ragged": ("llama3b_32k", dict(t_past=5000, bcp=200, bsa=1300), 1002),
    "decode_small": ("decode_64x16k", dict(b=6, t_past=3001, bsa=600), 1003),
    "d256_small": ("long_128k_d256", dict(t_past=4100, bcp=130, nq_keep=20, bsa=900), 1005),
    "d64_nq40": ("llama3b_32k", dict(d=64, nq=8, nkv=2, t_past=2000, bcp=100, nq_keep=40, bsa=500), 7),
    "g1_all_keys": ("llama3b_32k", dict(nq=4, nkv=4, t_past=700, bcp=33, nq_keep=33, bsa=700), 8),
    "f32_d128": ("tiny_f32", dict(d=128, t_past=777, bcp=45, nq_keep=9, bsa=300), 9),
    "long_chunk": ("llama3b_32k", dict(nq=6, nkv=2, t_past=1500, bcp=700, nq_keep=44, bsa=400), 10),
    "chunk_300": ("llama3b_32k", dict(nq=4, nkv=2, t_past=900, bcp=300, nq_keep=37, bsa=200), 11),
    # a batch of prefill chunks: per-sequence rows, row tiles and key splits
    "batch_prefill": ("llama3b_32k", dict(b=3, t_past=3000, bcp=128, bsa=700), 12),
    # a cache with spare rows after the chunk (kv_cap > T + bcp: every stride)
    "cache_slack": ("llama3b_32k", dict(b=2, t_past=2500, bcp=96, bsa=600, kv_extra=333), 13),
    # a past shorter than one key tile: scoring waves without blocks, one partial tile
    "tiny_past": ("llama3b_32k", dict(nq=8, nkv=2, t_past=37, bcp=40, nq_keep=8, bsa=9), 14),
    # decode steps at the other head dims
    "decode_d256": ("long_128k_d256", dict(b=4, bcp=1, nq_keep=1, t_past=3000, bsa=500), 15),
    "decode_d64": ("llama3b_32k", dict(d=64, b=4, bcp=1, nq_keep=1, t_past=2000, bsa=300), 16),
    # the fp32 kernels at decode (no outlier queries: the chunk is one query)
    "f32_decode": ("tiny_f32", dict(b=3, bcp=1, nq_keep=1, t_past=777, bsa=100, n_outliers=0), 17),
    # extremes: one kept query in a prefill chunk, one selected key, G = 64
    "nq1_prefill": ("llama3b_32k", dict(nq=4, nkv=2, t_past=1200, bcp=50, nq_keep=1, bsa=150), 19),
    "bsa1": ("llama3b_32k", dict(nq=4, nkv=2, t_past=800, bcp=40, nq_keep=8, bsa=1), 20),
    "g64": ("llama3b_32k", dict(nq=64, nkv=1, t_past=900, bcp=16, nq_keep=8, bsa=200), 21),
}
ROUND_CASES = {
    "rounds_small": ("rounds_64k", dict(nq=8, nkv=2, t_past=6000, bcp=128, n_rounds=16,
                                        top_rounds=4), 1004),
    # rounds shorter than 256 positions on average: the per-thread scan
    "rounds_short": ("rounds_64k", dict(nq=8, nkv=2, t_past=6000, bcp=128, n_rounds=48,
                                        top_rounds=6), 1006),
    # two sequences: rounds chosen (and shared by the heads) per sequence
    "rounds_batch": ("rounds_64k", dict(b=2, nq=8, nkv=2, t_past=6000, bcp=128, n_rounds=16,
                                        top_rounds=4), 1007),
    # every round chosen (top_r + latest = n_rounds); 400 rounds of 2-27 positions
    "rounds_all": ("rounds_64k", dict(nq=8, nkv=2, t_past=3000, bcp=64, n_rounds=5,
                                      top_rounds=4), 1008),
    "rounds_many": ("rounds_64k", dict(nq=8, nkv=2, t_past=3000, bcp=64, n_rounds=400,
                                       top_rounds=20), 1009),
}

_cache = {}


def _dev():
    return torch.device("cuda:0")


def _case(name, table=CASES):
    if name in _cache:
        return _cache[name]
    wname, over, seed = table[name]
    spec = W.spec(wname, **over)
    case = W.make_case(spec, seed)
    qn, kn, vn = np64(case["q"]), np64(case["k"]), np64(case["v"])
    off = case["round_off"].numpy() if case["round_off"] is not None else None
    ref = oracle.pipeline(qn, kn, vn, spec.t_past, spec.nq_keep, spec.bsa, round_off=off,
                          top_rounds=spec.top_rounds)
    dev = _dev()
    gpu = {n: case[n].to(dev) for n in ("q", "k", "v")}
    if off is not None:
        gpu["round_off"] = case["round_off"].to(dev)
    _cache[name] = (spec, case, ref, gpu)
    return _cache[name]


def _shape(spec, qk):
    return qk.shape_of(spec)


# --------------------------------------------------------------------------
# stage 1: query sub-selection and group aggregation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(CASES))
def test_qsel(gpu, name):
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    dev = _dev()
    q_idx = torch.empty((s.b, s.nq, s.nq_keep), dtype=torch.int32, device=dev)
    sq = torch.empty((s.b, s.nq, s.bcp), dtype=torch.float32, device=dev)
    qg = torch.empty((s.b, s.nkv, s.nq_keep, s.d), dtype=torch.float32, device=dev)
    qk.qk_qsel(s, g["q"], q_idx, sq, qg)
    torch.cuda.synchronize()
    err = max_abs(sq, ref["sq"])
    assert err <= SCORE_TOL and err <= 1e-5, err
    gi = npi(q_idx)
    G = s.group
    agree = np.ones((s.b, s.nkv, s.nq_keep), dtype=bool)
    for b in range(s.b):
        for h in range(s.nq):
            assert_set_within_boundary(gi[b, h], ref["qidx"][b, h], ref["sq"][b, h], s.nq_keep,
                                       what=f"qidx b{b} h{h}")
            # order: decreasing oracle SQ up to near-ties
            assert np.all(np.diff(ref["sq"][b, h][gi[b, h]]) <= BOUNDARY_TOL)
            agree[b, h // G] &= gi[b, h] == ref["qidx"][b, h]
    gq = np64(qg)
    assert np.abs(gq - ref["q_group"])[agree].max() <= 1e-5
    # slots whose picks differ at a near-tie: the group mean of the picks made
    qn = np64(case["q"])
    for b, j, n in zip(*np.nonzero(~agree)):
        rows = [qn[b, j * G + gg, gi[b, j * G + gg, n]] for gg in range(G)]
        want = np.mean([r / np.linalg.norm(r) for r in rows], axis=0)
        assert np.abs(gq[b, j, n] - want).max() <= 1e-5


@pytest.mark.parametrize("bcp", [48, 200, 256, 300, 512, 700])
def test_qsel_ties_keep_lower_positions(gpu, bcp):
    """Every chunk query of a head equal (SQ all equal): the kept queries are
    the first NQ positions in order, whatever the selection path."""
    qk = gpu
    spec = W.spec("llama3b_32k", nq=4, nkv=2, t_past=64, bcp=bcp, nq_keep=min(32, bcp), bsa=16)
    s = qk.shape_of(spec)
    g = torch.Generator().manual_seed(5)
    row = torch.randn(s.b, s.nq, 1, s.d, generator=g).to(torch.bfloat16)
    q = row.expand(s.b, s.nq, bcp, s.d).contiguous().to(_dev())
    q_idx = torch.empty((s.b, s.nq, s.nq_keep), dtype=torch.int32, device=_dev())
    qg = torch.empty((s.b, s.nkv, s.nq_keep, s.d), dtype=torch.float32, device=_dev())
    qk.qk_qsel(s, q, q_idx, None, qg)
    torch.cuda.synchronize()
    want = np.broadcast_to(np.arange(s.nq_keep), (s.b, s.nq, s.nq_keep))
    assert np.array_equal(npi(q_idx), want)


# Every layout of the query-selection kernel: d = 64 / 128 / 256 (8, 16, 32
# lanes per row), chunks held in registers four or eight rows per thread or
# read twice (bcp beyond eight rows per thread), the one-wave sort (bcp <= 64)
# and the 64- and 256-thread workgroups of short chunks.
QSEL_LAYOUTS = [(64, 8), (64, 40), (64, 500), (64, 900), (64, 1100), (128, 16), (128, 60),
                (128, 450), (128, 1000), (256, 2), (256, 7), (256, 100), (256, 200), (256, 260)]


@pytest.mark.parametrize("d,bcp", QSEL_LAYOUTS)
def test_qsel_layouts(gpu, d, bcp):
    qk = gpu
    spec = W.spec("llama3b_32k", nq=4, nkv=2, d=d, t_past=64, bcp=bcp,
                  nq_keep=min(32, bcp), bsa=16)
    s = qk.shape_of(spec)
    case = W.make_case(spec, 2000 + d + bcp)
    q = case["q"]
    q_idx = torch.empty((s.b, s.nq, s.nq_keep), dtype=torch.int32, device=_dev())
    sq = torch.empty((s.b, s.nq, bcp), dtype=torch.float32, device=_dev())
    qk.qk_qsel(s, q.to(_dev()), q_idx, sq, None)
    torch.cuda.synchronize()
    want_idx, want_sq = oracle.select_queries(np64(q), s.nq_keep)
    assert max_abs(sq, want_sq) <= 1e-5
    gi = npi(q_idx)
    for b in range(s.b):
        for h in range(s.nq):
            assert_set_within_boundary(gi[b, h], want_idx[b, h], want_sq[b, h], s.nq_keep,
                                       what=f"d{d} bcp{bcp} h{h}")
            assert np.all(np.diff(want_sq[b, h][gi[b, h]]) <= BOUNDARY_TOL)


# --------------------------------------------------------------------------
# stage 2: scoring pass, fed the oracle's group queries
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(CASES))
def test_kvscore(gpu, name):
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    qg32 = torch.from_numpy(ref["q_group"].astype(np.float32))
    s_agg = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    qk.qk_kvscore(s, qg32.to(_dev()), g["k"], s_agg)
    torch.cuda.synchronize()
    _, want = oracle.key_scores(qg32.double().numpy(), np64(case["k"]), s.t_past)
    err = max_abs(s_agg, want)
    assert err <= SCORE_TOL, err
    assert err <= 5e-5, f"precision regression: {err}"   # bf16 hi/lo split: ~1e-6


@pytest.mark.parametrize("name", list(CASES))
def test_kvscore_grouped(gpu, name):
    """Scoring with the group queries formed inside the pass, fed the oracle's
    kept positions: matches the oracle's scores of its own group queries."""
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    q_idx = torch.from_numpy(ref["qidx"].astype(np.int32)).to(_dev())
    s_agg = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    qk.qk_kvscore_grouped(s, g["q"], q_idx, g["k"], s_agg)
    torch.cuda.synchronize()
    _, want = oracle.key_scores(ref["q_group"], np64(case["k"]), s.t_past)
    err = max_abs(s_agg, want)
    assert err <= SCORE_TOL, err
    assert err <= 5e-5, f"precision regression: {err}"


# --------------------------------------------------------------------------
# scoring variants: 8-bit E4M3 keys, dot-product scores
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_keys_to_e4m3_bit_exact(gpu, dtype):
    """Key rows stored as E4M3: every byte equals the oracle's nearest-code
    encoding (ties to even, saturation above 448, signed zero), across ten
    binades of magnitudes; rows outside the converted range are untouched."""
    qk = gpu
    rng = np.random.default_rng(41)
    b, nkv, cap, d = 2, 3, 700, 128
    x = rng.standard_normal((b, nkv, cap, d)) * np.exp(rng.uniform(-12.0, 7.0, (b, nkv, cap, 1)))
    mags = oracle.e4m3_decode(np.arange(0x7F))
    mid = (mags[:-1] + mags[1:]) / 2                      # exact ties, 126 of them
    x[0, 0, 40, :126] = mid
    x[0, 0, 41, :126] = -mid
    x[1, 2, 50, :] = 0.0
    x[1, 2, 51, :] = -0.0
    x[1, 2, 52, :] = np.linspace(-2000.0, 2000.0, d)      # saturation both ways
    x[1, 1, 60, :] = np.linspace(-3e-3, 3e-3, d)          # subnormal codes
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = torch.from_numpy(x.astype(np.float32)).to(tdt).to(_dev()).contiguous()
    s = qk.Shape(b, nkv, nkv, d, 1, cap - 1, cap, 1, 1, 0.0, qk.QK_BF16 if dtype == "bf16" else qk.QK_F32)
    k8 = torch.full((b, nkv, cap, d), 0x55, dtype=torch.uint8, device=_dev())
    row0, nrows = 37, 600
    qk.qk_keys_to_e4m3(s, k, row0, nrows, k8)
    torch.cuda.synchronize()
    got = k8.cpu().numpy()
    want = oracle.e4m3_encode(np64(k)[:, :, row0:row0 + nrows])
    assert np.array_equal(got[:, :, row0:row0 + nrows], want)
    assert np.all(got[:, :, :row0] == 0x55) and np.all(got[:, :, row0 + nrows:] == 0x55)


def _variant_keys(qk, s, spec, case, g, e4m3):
    """(device keys, key format, fp64 keys the scores see)."""
    kn = np64(case["k"])
    if not e4m3:
        return g["k"], qk.QK_KEYS_DTYPE, kn
    k8 = torch.empty(g["k"].shape, dtype=torch.uint8, device=_dev())
    qk.qk_keys_to_e4m3(s, g["k"], 0, s.kv_cap, k8)
    return k8, qk.QK_KEYS_E4M3, oracle.scoring_keys_e4m3(kn)


def _dot_bound(qg, keys, t_past):
    """Per key, max over the kept slots of sum_e |q_group| |k|: the scale of the
    rounding error of a dot-product score."""
    return np.matmul(np.abs(qg), np.swapaxes(np.abs(keys[:, :, :t_past]), -1, -2)).max(axis=2)


VARIANTS = [("cosine", True), ("dot", False), ("dot", True)]


# 8-bit keys are scored with bf16 queries only (the API rejects fp32 + E4M3)
VARIANT_CASES = [(n, m, e) for n in CASES for (m, e) in VARIANTS
                 if not (e and CASES[n][0] == "tiny_f32")]


@pytest.mark.parametrize("name,mode,e4m3", VARIANT_CASES)
def test_kvscore_variant(gpu, name, mode, e4m3):
    """Scoring variants fed the oracle's kept positions.  Cosine scores of the
    decoded 8-bit keys keep the bf16 path's precision (the decode is exact);
    dot-product scores are bounded relative to sum |q_group| |k| (the group
    queries enter the matrix cores as bf16 high + low parts, about 2^-16)."""
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    assert not (e4m3 and spec.dtype != "bf16")
    q_idx = torch.from_numpy(ref["qidx"].astype(np.int32)).to(_dev())
    kin, fmt, keys = _variant_keys(qk, s, spec, case, g, e4m3)
    s_agg = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    qk.qk_kvscore_variant(s, g["q"], q_idx, kin, fmt, mode, s_agg)
    torch.cuda.synchronize()
    if mode == "cosine":
        _, want = oracle.key_scores(ref["q_group"], keys, s.t_past)
        assert max_abs(s_agg, want) <= 5e-5
    else:
        qg = oracle.group_queries_dot(np64(case["q"]), ref["qidx"], s.nkv)
        _, want = oracle.key_scores_dot(qg, keys, s.t_past)
        rel = np.abs(np64(s_agg) - want) / _dot_bound(qg, keys, s.t_past)
        assert rel.max() <= 3e-5, rel.max()


def test_kvscore_variant_cosine_dtype_is_grouped(gpu):
    """Cosine scoring of dtype keys through the variant entry point is the
    grouped scoring pass, bit for bit."""
    qk = gpu
    spec, case, ref, g = _case("llama_ragged")
    s = _shape(spec, qk)
    q_idx = torch.from_numpy(ref["qidx"].astype(np.int32)).to(_dev())
    a = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    c = torch.empty_like(a)
    qk.qk_kvscore_grouped(s, g["q"], q_idx, g["k"], a)
    qk.qk_kvscore_variant(s, g["q"], q_idx, g["k"], qk.QK_KEYS_DTYPE, qk.QK_SCORE_COSINE, c)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


@pytest.mark.parametrize("name", ["llama_ragged", "decode_small", "d64_nq40"])
@pytest.mark.parametrize("mode,e4m3", VARIANTS)
def test_pipeline_variants_end_to_end(gpu, name, mode, e4m3):
    """Whole chunk with a scoring variant, compared stage by stage with the
    oracle run with the same variant: kept queries, the scores of every KV
    group on the GPU's kept queries, key sets (near-boundary swaps only) and
    every attention row over the GPU's own selection."""
    qk = gpu
    spec, case, ref0, g = _case(name)
    s = _shape(spec, qk)
    qn, kn, vn = np64(case["q"]), np64(case["k"]), np64(case["v"])
    pipe = qk.Pipeline(s, device=_dev(), score_mode=mode, k_e4m3=e4m3)
    if e4m3:
        pipe.store_keys_e4m3(g["k"])
    pipe(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    sets, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, spec.bsa, np64(pipe.sq),
                                npi(pipe.q_idx), np64(pipe.s_agg), npi(pipe.idx), score=mode,
                                k_e4m3=e4m3, what=f"{name} {mode} e4m3={e4m3}")
    err = staged_attention(qn, kn, vn, spec.t_past, sets, pipe.out, spec.dtype,
                           what=f"{name} {mode}")
    print(f"[variant] {name} {mode} e4m3={e4m3}: {st}, attention {err:.2e}")


SELECT_CASES = ["llama_ragged", "d256_small", "decode_small", "tiny_f32", "g1_all_keys",
                "d64_nq40", "batch_prefill", "cache_slack", "tiny_past"]


# 8-bit keys are scored with bf16 queries only (the API rejects fp32 + E4M3)
SELECT_VARIANT_CASES = [(n, m, e) for n in SELECT_CASES for (m, e) in [("cosine", False)] + VARIANTS
                        if not (e and CASES[n][0] == "tiny_f32")]


@pytest.mark.parametrize("name,mode,e4m3", SELECT_VARIANT_CASES)
def test_select_equals_separate_calls(gpu, name, mode, e4m3):
    """qk_select writes what qk_qsel, qk_kvscore_variant and qk_topk write one
    by one, bit for bit: also where its scoring pass fills the histogram the
    top-k starts from (bf16 rows spread over several workgroups:
    llama_ragged, d256_small), from a workspace full of stale bytes, and on a
    second call that reuses the workspace.  With 8-bit keys the scoring pass
    also stores the chunk's own key rows, byte for byte what qk_keys_to_e4m3
    writes."""
    qk = gpu
    spec, case, ref, g = _case(name)
    assert not (e4m3 and spec.dtype != "bf16")
    s = _shape(spec, qk)
    a = qk.Pipeline(s, device=_dev(), score_mode=mode, k_e4m3=e4m3, fused_select=True)
    b = qk.Pipeline(s, device=_dev(), score_mode=mode, k_e4m3=e4m3, fused_select=False)
    assert a.fused_select and not b.fused_select
    for p in (a, b):
        if e4m3:
            p.store_keys_e4m3(g["k"])
    if a.select_ws is not None:
        a.select_ws.fill_(0x7f)
    b.select(g["q"], g["k"])
    for _ in range(2):
        for t in (a.q_idx, a.sq, a.s_agg, a.idx):
            t.fill_(-3)
        if e4m3:  # the chunk's own rows of the 8-bit copy come from the scoring pass
            a.k8[:, :, s.t_past:s.t_past + s.bcp] = 0x55
        a.select(g["q"], g["k"], append_e4m3=e4m3)
        torch.cuda.synchronize()
        assert torch.equal(a.q_idx, b.q_idx)
        assert torch.equal(a.sq, b.sq)
        assert torch.equal(a.s_agg, b.s_agg)
        assert torch.equal(a.idx, b.idx)
        if e4m3:
            assert torch.equal(a.k8, b.k8)
    # and the selection is the exact top-BSA of the scores it was taken on
    want = oracle.select_keys(np64(a.s_agg), s.bsa)
    assert np.array_equal(npi(a.idx)[..., :want.shape[-1]], want)


def test_kvscore_grouped_unsorted_positions(gpu):
    """The group means pair slot n of every head whatever the positions are:
    kept positions given in an arbitrary (unsorted, repeated) order score like
    the oracle's group queries built from the same lists."""
    qk = gpu
    spec, case, ref, g = _case("llama_ragged")
    s = _shape(spec, qk)
    rng = np.random.default_rng(31)
    pos = rng.integers(0, s.bcp, size=(s.b, s.nq, s.nq_keep)).astype(np.int32)
    qg = oracle.group_queries(np64(case["q"]), pos, s.nkv)
    s_agg = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    qk.qk_kvscore_grouped(s, g["q"], torch.from_numpy(pos).to(_dev()), g["k"], s_agg)
    torch.cuda.synchronize()
    _, want = oracle.key_scores(qg, np64(case["k"]), s.t_past)
    assert max_abs(s_agg, want) <= 5e-5


def test_kvscore_grouped_matches_split_path(gpu):
    """The fused scoring pass and qk_qsel's group means followed by qk_kvscore
    agree (same kept positions), on a case with G = 8 (two position batches)
    and 64 kept queries (two query tiles)."""
    qk = gpu
    spec = W.spec("long_128k", t_past=5000, bcp=160, nq_keep=64, bsa=512)
    case = W.make_case(spec, 21)
    s = qk.shape_of(spec)
    g = {n: case[n].to(_dev()) for n in ("q", "k")}
    q_idx = torch.empty((s.b, s.nq, s.nq_keep), dtype=torch.int32, device=_dev())
    qg = torch.empty((s.b, s.nkv, s.nq_keep, s.d), dtype=torch.float32, device=_dev())
    qk.qk_qsel(s, g["q"], q_idx, None, qg)
    a = torch.empty((s.b, s.nkv, s.t_past), dtype=torch.float32, device=_dev())
    b = torch.empty_like(a)
    qk.qk_kvscore(s, qg, g["k"], a)
    qk.qk_kvscore_grouped(s, g["q"], q_idx, g["k"], b)
    torch.cuda.synchronize()
    assert (a - b).abs().max().item() <= 1e-5


# --------------------------------------------------------------------------
# stage 3: top-BSA on the oracle's scores (fp32) -- integer result, exact
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(CASES))
def test_topk_on_oracle_scores(gpu, name):
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    scores32 = ref["s_agg"].astype(np.float32)
    rows = s.b * s.nkv
    kk = min(s.bsa, s.t_past)
    idx = torch.full((rows, kk), -1, dtype=torch.int32, device=_dev())
    qk.qk_topk(rows, s.t_past, s.bsa, torch.from_numpy(scores32).to(_dev()).reshape(rows, -1),
               s.t_past, idx, kk)
    torch.cuda.synchronize()
    want = oracle.select_keys(scores32.astype(np.float64), s.bsa).reshape(rows, kk)
    assert np.array_equal(npi(idx), want)


# --------------------------------------------------------------------------
# stage 4: attention over the oracle's selection
# --------------------------------------------------------------------------
@pytest.mark.parametrize("fused", [True, False], ids=["indexed", "gathered"])
@pytest.mark.parametrize("name", list(CASES))
def test_attention_on_oracle_selection(gpu, name, fused):
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    dev = _dev()
    kidx = torch.from_numpy(ref["kidx"].astype(np.int32)).to(dev).contiguous()
    n_sel = kidx.shape[-1]
    out = torch.empty_like(g["q"])
    lse = torch.empty((s.b, s.nq, s.bcp), dtype=torch.float32, device=dev)
    nws = qk.qk_workspace_bytes(s, "sparse_attn")
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
    if fused:
        qk.qk_sparse_attn_indexed(s, g["q"], g["k"], g["v"], kidx, n_sel, None, out, lse, ws, nws)
    else:
        ksel = torch.empty((s.b, s.nkv, n_sel, s.d), dtype=g["k"].dtype, device=dev)
        vsel = torch.empty_like(ksel)
        qk.qk_gather(s, g["k"], g["v"], kidx, n_sel, None, ksel, vsel)
        torch.cuda.synchronize()
        kn = np64(case["k"])
        want_k = np.stack([[kn[b, j, ref["kidx"][b, j]] for j in range(s.nkv)] for b in range(s.b)])
        assert np.array_equal(np64(ksel), want_k)        # a copy: bit-exact
        qk.qk_sparse_attn(s, g["q"], ksel, vsel, n_sel, None, g["k"], g["v"], out, lse, ws, nws)
    torch.cuda.synchronize()
    err = max_abs(out, ref["o"])
    assert err <= ATTN_TOL[spec.dtype], err
    assert max_abs(lse, ref["lse"]) <= LSE_TOL[spec.dtype]


@pytest.mark.parametrize("name", ["tiny_f32", "llama_ragged", "decode_small", "d256_small", "d64_nq40"])
def test_dense_attention(gpu, name):
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    dev = _dev()
    out = torch.empty_like(g["q"])
    lse = torch.empty((s.b, s.nq, s.bcp), dtype=torch.float32, device=dev)
    nws = qk.qk_workspace_bytes(s, "dense_attn")
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
    qk.qk_dense_attn(s, g["q"], g["k"], g["v"], out, lse, ws, nws)
    torch.cuda.synchronize()
    want_o, want_lse = oracle.dense_attention(np64(case["q"]), np64(case["k"]), np64(case["v"]),
                                              s.t_past)
    assert max_abs(out, want_o) <= ATTN_TOL[spec.dtype]
    assert max_abs(lse, want_lse) <= LSE_TOL[spec.dtype]


# --------------------------------------------------------------------------
# end to end: each side runs its own pipeline
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(CASES))
def test_pipeline_end_to_end(gpu, name):
    """Whole chunk, compared stage by stage with the oracle: SQ and kept
    queries against the oracle's own run, then the oracle's scores, key sets
    and attention on the GPU's kept queries and key sets, for every KV group
    and every row (the number of groups whose kept queries rank differently
    from the oracle's own run is printed)."""
    qk = gpu
    spec, case, ref, g = _case(name)
    s = _shape(spec, qk)
    pipe = qk.Pipeline(s, device=_dev())
    pipe(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    qn, kn, vn = np64(case["q"]), np64(case["k"]), np64(case["v"])
    sets, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, spec.bsa, np64(pipe.sq),
                                npi(pipe.q_idx), np64(pipe.s_agg), npi(pipe.idx), what=name)
    err = staged_attention(qn, kn, vn, spec.t_past, sets, pipe.out, spec.dtype, gpu_lse=pipe.lse,
                           what=name)
    if spec.dtype == "f32":
        assert st["swaps"] == 0
    # integer stage, exact: the key sets are the top-BSA of the GPU's own scores
    want = oracle.select_keys(np64(pipe.s_agg), spec.bsa)
    assert np.array_equal(npi(pipe.idx)[..., :want.shape[-1]], want)
    print(f"[e2e] {name}: {st}, attention {err:.2e}")


def test_sparse_equals_dense_at_full_budget(gpu):
    qk = gpu
    spec, case, ref, g = _case("g1_all_keys")
    s = _shape(spec, qk)
    pipe = qk.Pipeline(s, device=_dev())
    pipe(g["q"], g["k"], g["v"])
    out = torch.empty_like(g["q"])
    nws = qk.qk_workspace_bytes(s, "dense_attn")
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=_dev())
    qk.qk_dense_attn(s, g["q"], g["k"], g["v"], out, None, ws, nws)
    torch.cuda.synchronize()
    assert np.array_equal(npi(pipe.idx)[0, 0], np.arange(s.t_past))
    assert max_abs(pipe.out, out) <= 2e-3


# --------------------------------------------------------------------------
# round-granular selection
# --------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(ROUND_CASES))
def test_round_select_shared(gpu, name):
    """One round choice for all KV heads (QK_ROUNDS_SHARED) on the oracle's
    fp32 scores: the heads' own round scores exactly, and the chosen mask,
    lengths and position lists exactly the oracle's shared choice (maxima of
    fp32 values are exact, so both sides rank the same numbers); every head
    of a sequence gets the same rounds."""
    qk = gpu
    spec, case, ref, g = _case(name, ROUND_CASES)
    s = _shape(spec, qk)
    dev = _dev()
    scores32 = ref["s_agg"].astype(np.float32)
    idx = torch.full((s.b, s.nkv, s.t_past), -1, dtype=torch.int32, device=dev)
    sel_len = torch.empty((s.b, s.nkv), dtype=torch.int32, device=dev)
    s_round = torch.empty((s.b, s.nkv, spec.n_rounds), dtype=torch.float32, device=dev)
    chosen_mask = torch.full((s.b, s.nkv, spec.n_rounds), 7, dtype=torch.uint8, device=dev)
    qk.qk_round_select(s, torch.from_numpy(scores32).to(dev), spec.n_rounds, g["round_off"],
                       spec.top_rounds, qk.QK_ROUNDS_KEEP_LATEST | qk.QK_ROUNDS_SHARED, idx,
                       s.t_past, sel_len, s_round, chosen_mask)
    torch.cuda.synchronize()
    off = case["round_off"].numpy()
    want_sr = oracle.round_scores(scores32.astype(np.float64), off)
    assert np.array_equal(np64(s_round), want_sr)
    chosen = oracle.select_rounds_shared(want_sr, spec.top_rounds)
    sets = oracle.round_key_sets(chosen, off)
    cm, gi, gl = npi(chosen_mask), npi(idx), npi(sel_len)
    for b in range(s.b):
        for j in range(s.nkv):
            assert np.flatnonzero(cm[b, j]).tolist() == chosen[b][j].tolist()
            assert np.array_equal(cm[b, j], cm[b, 0])
            assert gl[b, j] == len(sets[b][j])
            assert np.array_equal(gi[b, j, : gl[b, j]], sets[b][j])


@pytest.mark.parametrize("name", list(ROUND_CASES))
def test_round_select_and_attention(gpu, name):
    qk = gpu
    spec, case, ref, g = _case(name, ROUND_CASES)
    s = _shape(spec, qk)
    dev = _dev()
    rows = s.b * s.nkv
    scores32 = ref["s_agg"].astype(np.float32)
    idx = torch.full((s.b, s.nkv, s.t_past), -1, dtype=torch.int32, device=dev)
    sel_len = torch.empty((s.b, s.nkv), dtype=torch.int32, device=dev)
    s_round = torch.empty((s.b, s.nkv, spec.n_rounds), dtype=torch.float32, device=dev)
    chosen_mask = torch.full((s.b, s.nkv, spec.n_rounds), 7, dtype=torch.uint8, device=dev)
    qk.qk_round_select(s, torch.from_numpy(scores32).to(dev), spec.n_rounds, g["round_off"],
                       spec.top_rounds, True, idx, s.t_past, sel_len, s_round, chosen_mask)
    torch.cuda.synchronize()
    off = case["round_off"].numpy()
    want_sr = oracle.round_scores(scores32.astype(np.float64), off)
    assert np.array_equal(np64(s_round), want_sr)      # max of fp32 values: exact
    chosen = oracle.select_rounds(want_sr, spec.top_rounds)
    sets = oracle.round_key_sets(chosen, off)
    cm = npi(chosen_mask)
    for b in range(s.b):
        for j in range(s.nkv):
            want_mask = np.zeros(spec.n_rounds, dtype=np.int64)
            want_mask[np.asarray(chosen[b][j])] = 1
            assert np.array_equal(cm[b, j], want_mask)
    gi, gl = npi(idx), npi(sel_len)
    for b in range(s.b):
        for j in range(s.nkv):
            assert gl[b, j] == len(sets[b][j])
            assert np.array_equal(gi[b, j, : gl[b, j]], sets[b][j])
    # ragged attention over the oracle's rounds, vs the oracle
    ld = max(len(x) for row in ref["key_sets"] for x in row)
    kidx = np.zeros((s.b, s.nkv, ld), dtype=np.int32)
    lens = np.zeros((s.b, s.nkv), dtype=np.int32)
    for b in range(s.b):
        for j in range(s.nkv):
            ks = ref["key_sets"][b][j]
            kidx[b, j, : len(ks)] = ks
            lens[b, j] = len(ks)
    s2 = qk.shape_of(spec, bsa=ld)
    out = torch.empty_like(g["q"])
    nws = qk.qk_workspace_bytes(s2, "sparse_attn")
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
    qk.qk_sparse_attn_indexed(s2, g["q"], g["k"], g["v"], torch.from_numpy(kidx).to(dev), ld,
                              torch.from_numpy(lens).to(dev), out, None, ws, nws)
    torch.cuda.synchronize()
    assert max_abs(out, ref["o"]) <= ATTN_TOL[spec.dtype]
    # and the whole round pipeline end to end, stage by stage on the GPU's choices
    pipe = qk.Pipeline(s2, device=dev, n_rounds=spec.n_rounds, top_rounds=spec.top_rounds)
    pipe(g["q"], g["k"], g["v"], g["round_off"])
    torch.cuda.synchronize()
    qn, kn, vn = np64(case["q"]), np64(case["k"]), np64(case["v"])
    sets2, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, s2.bsa, np64(pipe.sq),
                                 npi(pipe.q_idx), np64(pipe.s_agg), npi(pipe.idx), round_off=off,
                                 top_rounds=spec.top_rounds, gpu_sel_len=npi(pipe.sel_len), what=name)
    err = staged_attention(qn, kn, vn, spec.t_past, sets2, pipe.out, spec.dtype, what=name)
    print(f"[rounds e2e] {name}: {st}, attention {err:.2e}")


# --------------------------------------------------------------------------
# top-k edge cases (exact against the oracle's sort on the same fp32 values)
# --------------------------------------------------------------------------
def _topk_check(qk, scores32, k, ld_idx=None):
    rows, n = scores32.shape
    kk = min(k, n)
    ld_idx = ld_idx or kk
    idx = torch.full((rows, ld_idx), -7, dtype=torch.int32, device=_dev())
    qk.qk_topk(rows, n, k, torch.from_numpy(scores32).to(_dev()), n, idx, ld_idx)
    torch.cuda.synchronize()
    got = npi(idx)
    want = oracle.select_keys(scores32.astype(np.float64)[None], k)[0]
    assert np.array_equal(got[:, :kk], want)
    assert np.all(got[:, kk:] == -7)


def test_topk_edge_cases(gpu):
    qk = gpu
    rng = np.random.default_rng(3)
    _topk_check(qk, rng.standard_normal((5, 1000)).astype(np.float32), 77)
    _topk_check(qk, np.round(rng.standard_normal((4, 4099)), 1).astype(np.float32), 1500)  # ties
    _topk_check(qk, np.zeros((3, 500), np.float32), 123)                                   # all equal
    z = np.zeros((2, 64), np.float32)
    z[:, ::2] = -0.0
    _topk_check(qk, z, 10)                                                                 # -0 == +0
    _topk_check(qk, rng.standard_normal((2, 100)).astype(np.float32), 100)                 # k = n
    _topk_check(qk, rng.standard_normal((2, 100)).astype(np.float32), 150)                 # k > n
    _topk_check(qk, rng.standard_normal((3, 1)).astype(np.float32), 1)
    _topk_check(qk, rng.standard_normal((3, 333)).astype(np.float32), 1, ld_idx=5)
    _topk_check(qk, rng.uniform(-1, 1, (2, 131072)).astype(np.float32), 16384)
    # rows whose 1K blocks alternate between two very different levels: the
    # per-tile histograms of a split row differ widely
    x = rng.standard_normal((3, 32768)).astype(np.float32)
    blk = (np.arange(32768) // 1024) % 4 == 0
    x[:, blk] += 5.0
    _topk_check(qk, x, 8192)
    _topk_check(qk, x, 9000)
    x = rng.standard_normal((2, 20000)).astype(np.float32)  # partial tile
    x[:, ((np.arange(20000) // 1024) % 4) == 0] -= 4.0
    _topk_check(qk, x, 5000)


def test_topk_workspace_reuse_and_unaligned_rows(gpu):
    """One top-k workspace serves calls of different shapes (a large split
    call, a smaller one, the large one again); rows that start 4 bytes off a
    16-byte boundary take the element-wise load path.  Every result matches the
    oracle's sort."""
    qk = gpu
    rng = np.random.default_rng(29)
    big = rng.standard_normal((4, 70000)).astype(np.float32)
    small = rng.standard_normal((9, 20000)).astype(np.float32)
    nws = max(qk.topk_workspace_bytes(4, 70000), qk.topk_workspace_bytes(9, 20000))
    ws = torch.full((nws,), 0x7f, dtype=torch.uint8, device=_dev())
    for x, k in ((big, 17000), (small, 5000), (big, 17000)):
        rows, n = x.shape
        idx = torch.full((rows, k), -1, dtype=torch.int32, device=_dev())
        qk.qk_topk(rows, n, k, torch.from_numpy(x).to(_dev()), n, idx, k, ws, nws)
        torch.cuda.synchronize()
        want = oracle.select_keys(x.astype(np.float64)[None], k)[0]
        assert np.array_equal(npi(idx), want)
    # rows at an odd element offset (4-byte aligned only), leading dimension n + 1
    x = rng.standard_normal((3, 9001 * 3 + 1)).astype(np.float32)
    buf = torch.from_numpy(x.reshape(-1)).to(_dev())
    rows, n, ld, k = 3, 9000, 9001, 2500
    view = buf[1:1 + rows * ld]
    idx = torch.full((rows, k), -1, dtype=torch.int32, device=_dev())
    qk.qk_topk(rows, n, k, view, ld, idx, k)
    torch.cuda.synchronize()
    scores = x.reshape(-1)[1:1 + rows * ld].reshape(rows, ld)[:, :n]
    want = oracle.select_keys(scores.astype(np.float64)[None], k)[0]
    assert np.array_equal(npi(idx), want)


def test_topk_split_rows(gpu):
    """Rows spread over several workgroups (few rows longer than 4K scores, or
    rows longer than 32K): tiles of 4 and 8 elements per thread,
    ragged last tiles, k at both ends, and boundary bins too large for LDS
    (many copies of one value), where the candidates are re-read from the row."""
    qk = gpu
    rng = np.random.default_rng(17)
    x = rng.standard_normal((6, 12289)).astype(np.float32)
    for k in (1, 2, 4096, 12288):
        _topk_check(qk, x, k)
    _topk_check(qk, rng.standard_normal((100, 5000)).astype(np.float32), 1234)
    _topk_check(qk, rng.standard_normal((130, 16900)).astype(np.float32), 4000)   # many long rows
    _topk_check(qk, rng.standard_normal((1, 300001)).astype(np.float32), 70001)      # 37 tiles
    _topk_check(qk, rng.standard_normal((2, 70000)).astype(np.float32), 30000)       # 8 per thread
    # one value held by most of the row: its bin overflows the LDS list
    x = np.full((2, 40000), 0.25, np.float32)
    x[:, ::7] = rng.standard_normal((2, len(range(0, 40000, 7)))).astype(np.float32)
    _topk_check(qk, x, 9000)
    _topk_check(qk, np.zeros((3, 9000), np.float32), 4500)                            # all equal
    # many near-equal values: one level-1 bin, distinct low bits
    x = (1.0 + rng.integers(0, 1 << 12, (2, 30000)) * 2.0 ** -20).astype(np.float32)
    _topk_check(qk, x, 10000)
    # a boundary bin of a few thousand near-equal scores inside the cosine range
    # (more than are ranked pair by pair, few enough for LDS): radix levels
    x = np.full((2, 20000), -0.5, np.float32)
    x[:, :3000] = 2.0
    x[:, 3000:7000] = (0.3 + rng.integers(0, 2048, (2, 4000)) * 2.0 ** -24).astype(np.float32)
    x = rng.permuted(x, axis=1)
    _topk_check(qk, x, 5000)
    # -0.0 and +0.0 interleaved in a split row
    z = np.zeros((2, 8192), np.float32)
    z[:, ::3] = -0.0
    z[:, 5::11] = 1.0
    _topk_check(qk, z, 2000)
    # skewed, ragged and extreme k
    _topk_check(qk, rng.exponential(1.0, (3, 32768)).astype(np.float32), 8192)
    _topk_check(qk, rng.standard_normal((2, 12345)).astype(np.float32), 1)
    _topk_check(qk, rng.standard_normal((2, 12345)).astype(np.float32), 12344)
    _topk_check(qk, rng.standard_normal((2, 65536 + 77)).astype(np.float32), 3333)
    _topk_check(qk, np.round(rng.standard_normal((2, 32768)), 2).astype(np.float32), 8192)  # ties
    # a dense cluster at the boundary (more than fits in LDS): global fallback
    x = rng.uniform(0, 1e-6, (2, 40000)).astype(np.float32) + 0.5
    x[:, :100] = 2.0
    x[:, 100:200] = -2.0
    _topk_check(qk, x, 20000)


def test_zero_keys_and_empty_past(gpu):
    qk = gpu
    spec = W.spec("llama3b_32k", t_past=300, bcp=70, bsa=64)
    case = W.make_case(spec, 21)
    case["k"][:, :, 10:20] = 0
    g = {n: case[n].to(_dev()) for n in ("q", "k", "v")}
    s = qk.shape_of(spec)
    pipe = qk.Pipeline(s, device=_dev())
    pipe(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    assert np.all(np64(pipe.s_agg)[:, :, 10:20] == 0)
    ref = oracle.pipeline(np64(case["q"]), np64(case["k"]), np64(case["v"]), 300, spec.nq_keep, 64)
    assert max_abs(pipe.s_agg, ref["s_agg"]) <= SCORE_TOL
    # no past at all: dense attention is the chunk's causal self-attention
    s0 = qk.Shape(s.b, s.nq, s.nkv, s.d, s.bcp, 0, s.kv_cap, s.nq_keep, 1)
    kk, vv = g["k"][:, :, 300:].contiguous(), g["v"][:, :, 300:].contiguous()
    s0.kv_cap = kk.shape[2]
    out = torch.empty_like(g["q"])
    nws = qk.qk_workspace_bytes(s0, "dense_attn")
    ws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=_dev())
    qk.qk_dense_attn(s0, g["q"], kk, vv, out, None, ws, nws)
    torch.cuda.synchronize()
    want, _ = oracle.dense_attention(np64(case["q"]), np64(case["k"][:, :, 300:]),
                                     np64(case["v"][:, :, 300:]), 0)
    assert max_abs(out, want) <= ATTN_TOL["bf16"]


def test_deterministic(gpu):
    qk = gpu
    spec, case, ref, g = _case("llama_ragged")
    s = _shape(spec, qk)
    a = qk.Pipeline(s, device=_dev())
    b = qk.Pipeline(s, device=_dev())
    a(g["q"], g["k"], g["v"])
    b(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    for n in ("q_idx", "s_agg", "idx", "out", "lse"):
        assert torch.equal(getattr(a, n), getattr(b, n)), n
    c = qk.Pipeline(s, device=_dev(), fused_group=False)
    d = qk.Pipeline(s, device=_dev(), fused_group=False)
    c(g["q"], g["k"], g["v"])
    d(g["q"], g["k"], g["v"])
    torch.cuda.synchronize()
    for n in ("q_idx", "q_group", "s_agg", "idx", "out", "lse"):
        assert torch.equal(getattr(c, n), getattr(d, n)), n


def test_workspace_reuse_across_calls(gpu):
    """One workspace serves consecutive key-split attention calls of different
    sizes (a large call, a smaller one, the large one again): identical
    outputs for identical calls, each matching the oracle."""
    qk = gpu
    spec = W.spec("llama3b_32k", t_past=4096, bsa=1024, bcp=128)
    case = W.make_case(spec, 33)
    g = {n: case[n].to(_dev()) for n in ("q", "k", "v")}
    s = qk.shape_of(spec)
    nws = qk.qk_workspace_bytes(s, "dense_attn")
    assert nws > 0, "this shape is meant to use key splits"
    ws = torch.full((nws,), 0x7f, dtype=torch.uint8, device=_dev())  # contents are don't-care
    outs = []
    small = qk.Shape(s.b, s.nq, s.nkv, s.d, s.bcp, 1024, s.kv_cap, s.nq_keep, s.bsa)
    for shp in (s, small, s):
        out = torch.empty_like(g["q"])
        lse = torch.empty(s.b, s.nq, s.bcp, dtype=torch.float32, device=_dev())
        qk.qk_dense_attn(shp, g["q"], g["k"], g["v"], out, lse, ws, nws)
        outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[2][0]) and torch.equal(outs[0][1], outs[2][1])
    want, _ = oracle.dense_attention(np64(case["q"]), np64(case["k"]), np64(case["v"]), 4096)
    assert max_abs(outs[0][0], want) <= ATTN_TOL["bf16"]
    want_s, _ = oracle.dense_attention(np64(case["q"]), np64(case["k"]), np64(case["v"]), 1024)
    assert max_abs(outs[1][0], want_s) <= ATTN_TOL["bf16"]
