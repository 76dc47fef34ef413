"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (Pipeline: qsel -> kvscore -> topk / round select -> attention
with the gather fused into its loads).

Inputs are drawn on the GPU (same generator, seeded) and copied to the host for
the oracle.  The oracle recomputes every selection output of the checked
sequences (all of them when b = 1, three sampled ones for the decode batch)
and a sample of attention rows one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (ATTN_TOL, BOUNDARY_TOL, SCORE_TOL, assert_set_within_boundary,
                    assert_sorted_unique, group_agreement, np64, npi)

pytestmark = pytest.mark.gpu

FULL = {
    "llama3b_32k": 1002,
    "decode_64x16k": 1003,
    "rounds_64k": 1004,
    "long_128k": 1005,
    "long_128k_d256": 1105,
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size(gpu, name):
    qk = gpu
    dev = torch.device("cuda:0")
    spec = W.spec(name)
    seed = FULL[name]
    print(f"[full-size] {name} seed {seed}", flush=True)
    case = W.make_case(spec, seed, device=dev)
    q, k, v = case["q"], case["k"], case["v"]
    rounds = spec.n_rounds > 0
    s = qk.shape_of(spec, bsa=spec.t_past if rounds else spec.bsa)
    pipe = qk.Pipeline(s, device=dev, n_rounds=spec.n_rounds, top_rounds=spec.top_rounds)
    pipe(q, k, v, case["round_off"])
    torch.cuda.synchronize()

    rng = np.random.default_rng(seed)
    seqs = [0] if spec.b == 1 else sorted(rng.choice(spec.b, 3, replace=False).tolist())
    off = case["round_off"].cpu().numpy() if rounds else None
    for bi in seqs:
        qn = np64(q[bi:bi + 1])
        kn = np64(k[bi:bi + 1])
        vn = np64(v[bi:bi + 1])
        qidx, sq = oracle.select_queries(qn, spec.nq_keep)
        qg = oracle.group_queries(qn, qidx, spec.nkv)
        _, s_agg = oracle.key_scores(qg, kn, spec.t_past)
        g_sq = np64(pipe.sq[bi:bi + 1])
        assert np.abs(g_sq - sq).max() <= SCORE_TOL
        g_qidx = npi(pipe.q_idx[bi])
        for h in range(spec.nq):
            assert_set_within_boundary(g_qidx[h], qidx[0, h], sq[0, h], spec.nq_keep, what=f"qidx h{h}")
            assert np.all(np.diff(sq[0, h][g_qidx[h]]) <= BOUNDARY_TOL)
        # KV groups whose kept queries (and their rank order) match on both sides
        agree = group_agreement(g_qidx[None], qidx, spec.group)[0]
        assert agree.mean() >= 0.5, f"{agree.sum()} of {agree.size} groups agree"
        g_s = np64(pipe.s_agg[bi:bi + 1])
        err = max(np.abs(g_s[0, j] - s_agg[0, j]).max() for j in range(spec.nkv) if agree[j])
        assert err <= SCORE_TOL, err
        if rounds:
            chosen = oracle.select_rounds(oracle.round_scores(s_agg, off), spec.top_rounds)
            key_sets = oracle.round_key_sets(chosen, off)
            sr = oracle.round_scores(s_agg, off)[0]
            R = len(off) - 1
            lens = npi(pipe.sel_len[bi])
            g_idx = npi(pipe.idx[bi])
            for j in range(spec.nkv):
                if not agree[j]:
                    continue
                sel = g_idx[j, : lens[j]]
                assert_sorted_unique(sel, spec.t_past)
                got = np.unique(np.searchsorted(off, sel, side="right") - 1)
                assert R - 1 in got                                    # the latest round
                assert lens[j] == sum(int(off[r + 1] - off[r]) for r in got)   # whole rounds
                want = chosen[0][j]
                assert_set_within_boundary(got[got != R - 1], want[want != R - 1], sr[j, : R - 1],
                                           spec.top_rounds, what=f"rounds j{j}")
        else:
            kidx = oracle.select_keys(s_agg, spec.bsa)
            key_sets = [[kidx[0, j] for j in range(spec.nkv)]]
            g_idx = npi(pipe.idx[bi])
            for j in range(spec.nkv):
                assert_sorted_unique(g_idx[j], spec.t_past)
                if agree[j]:
                    assert_set_within_boundary(g_idx[j], kidx[0, j], s_agg[0, j], s.n_sel, what=f"kidx j{j}")
        ok_heads = np.array([h for h in range(spec.nq) if agree[h // spec.group]])
        heads = rng.choice(ok_heads, size=min(4, len(ok_heads)), replace=False)
        rows = rng.choice(spec.bcp, size=min(8, spec.bcp), replace=False)
        if spec.bcp > 1 and spec.bcp - 1 not in rows:
            rows[0] = spec.bcp - 1                                    # the last row sees the whole chunk
        o_ref, lse_ref = oracle.attention(qn, kn, vn, spec.t_past, key_sets, rows=rows, heads=heads)
        got = np64(pipe.out[bi:bi + 1])[:, heads][:, :, rows]
        err_o = np.abs(got - o_ref).max()
        assert err_o <= ATTN_TOL[spec.dtype], err_o
        got_lse = np64(pipe.lse[bi:bi + 1])[:, heads][:, :, rows]
        assert np.abs(got_lse - lse_ref).max() <= 2e-3
        print(f"[full-size] {name} b{bi}: s_agg err {err:.2e}, attention err {err_o:.2e}", flush=True)


VARIANTS_FULL = [("llama3b_32k", "cosine", True), ("long_128k", "cosine", True),
                 ("decode_64x16k", "cosine", True), ("llama3b_32k", "dot", False)]


@pytest.mark.parametrize("name,mode,e4m3", VARIANTS_FULL)
def test_full_size_scoring_variants(gpu, name, mode, e4m3):
    """The benchmarked scoring variants at full size: E4M3 key bytes (a KV
    head's rows, bit-exact), scores of one sequence against the oracle on the
    same keys, its key sets (boundary rule) and sampled attention rows."""
    qk = gpu
    dev = torch.device("cuda:0")
    spec = W.spec(name)
    seed = FULL[name]
    print(f"[full-size variant] {name} {mode} e4m3={e4m3} seed {seed}", flush=True)
    case = W.make_case(spec, seed, device=dev)
    q, k, v = case["q"], case["k"], case["v"]
    s = qk.shape_of(spec)
    pipe = qk.Pipeline(s, device=dev, score_mode=mode, k_e4m3=e4m3)
    if e4m3:
        pipe.store_keys_e4m3(k)
    pipe(q, k, v)
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed + 1)
    bi = 0 if spec.b == 1 else int(rng.integers(spec.b))
    qn, kn, vn = np64(q[bi:bi + 1]), np64(k[bi:bi + 1]), np64(v[bi:bi + 1])
    if e4m3:
        j0 = int(rng.integers(spec.nkv))
        got8 = pipe.k8[bi, j0, :spec.t_past].cpu().numpy()
        assert np.array_equal(got8, oracle.e4m3_encode(kn[0, j0, :spec.t_past]))
        keys = oracle.scoring_keys_e4m3(kn[:, :, :spec.t_past])
    else:
        keys = kn
    ref = oracle.pipeline(qn, kn, vn, spec.t_past, spec.nq_keep, spec.bsa, score=mode, k_e4m3=e4m3,
                          with_attention=False)
    agree = group_agreement(npi(pipe.q_idx[bi])[None], ref["qidx"], spec.group)[0]
    assert agree.mean() >= 0.5
    g_s = np64(pipe.s_agg[bi:bi + 1])
    g_idx = npi(pipe.idx[bi])
    if mode == "dot":
        bound = np.matmul(np.abs(ref["q_group"]), np.swapaxes(np.abs(keys[:, :, :spec.t_past]), -1, -2)).max(axis=2)
    for j in range(spec.nkv):
        assert_sorted_unique(g_idx[j], spec.t_past)
        if not agree[j]:
            continue
        err = np.abs(g_s[0, j] - ref["s_agg"][0, j])
        if mode == "dot":
            assert (err / bound[0, j]).max() <= 3e-5
            tol = max(BOUNDARY_TOL, 3e-5 * float(bound[0, j].max()))
        else:
            assert err.max() <= 5e-5
            tol = BOUNDARY_TOL
        assert_set_within_boundary(g_idx[j], ref["kidx"][0, j], ref["s_agg"][0, j], s.n_sel,
                                   tol=tol, what=f"kidx j{j}")
    # sampled attention rows over the GPU's own key sets (attention reads bf16 keys)
    sets = [[g_idx[j] for j in range(spec.nkv)]]
    heads = rng.choice(spec.nq, size=min(4, spec.nq), replace=False)
    rows = rng.choice(spec.bcp, size=min(8, spec.bcp), replace=False)
    o_ref, _ = oracle.attention(qn, kn, vn, spec.t_past, sets, rows=rows, heads=heads)
    got = np64(pipe.out[bi:bi + 1])[:, heads][:, :, rows]
    assert np.abs(got - o_ref).max() <= ATTN_TOL[spec.dtype]
