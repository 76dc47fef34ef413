"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (Pipeline: qsel -> kvscore -> topk / round select -> attention
with the gather fused into its loads).

Inputs are drawn on the GPU (same generator, seeded) and copied to the host for
the oracle.  The comparison is staged: the oracle's own run fixes what the
kept queries may be (boundary rule); its group queries, key scores, key or
round selection and attention are then recomputed on the GPU's own kept
queries and key sets, for every KV group and every attention row and head of
the checked sequences (all of them when b = 1, three sampled ones for the
decode batch).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import np64, npi, staged_attention, staged_selection

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
        sl = slice(bi, bi + 1)
        qn, kn, vn = np64(q[sl]), np64(k[sl]), np64(v[sl])
        sets, st = staged_selection(
            qn, kn, spec.t_past, spec.nq_keep, s.bsa, np64(pipe.sq[sl]), npi(pipe.q_idx[sl]),
            np64(pipe.s_agg[sl]), npi(pipe.idx[sl]), round_off=off, top_rounds=spec.top_rounds,
            gpu_sel_len=npi(pipe.sel_len[sl]) if rounds else None, what=f"{name} b{bi}")
        err = staged_attention(qn, kn, vn, spec.t_past, sets, pipe.out[sl], spec.dtype,
                               gpu_lse=pipe.lse[sl], what=f"{name} b{bi}")
        if not rounds:  # integer stage, exact: the top-BSA of the GPU's own scores
            want = oracle.select_keys(np64(pipe.s_agg[sl]), s.bsa)
            assert np.array_equal(npi(pipe.idx[sl])[..., :want.shape[-1]], want)
        print(f"[full-size] {name} b{bi}: {st}, attention err {err:.2e} (every row and head)",
              flush=True)


VARIANTS_FULL = [("llama3b_32k", "cosine", True), ("long_128k", "cosine", True),
                 ("decode_64x16k", "cosine", True), ("llama3b_32k", "dot", False)]


@pytest.mark.parametrize("name,mode,e4m3", VARIANTS_FULL)
def test_full_size_scoring_variants(gpu, name, mode, e4m3):
    """The benchmarked scoring variants at full size: E4M3 key bytes (a KV
    head's rows, bit-exact), then the staged comparison of one sequence (the
    scores of every KV group on the GPU's kept queries, key sets, and every
    attention row over the GPU's own key sets; attention reads bf16 keys)."""
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
    sl = slice(bi, bi + 1)
    qn, kn, vn = np64(q[sl]), np64(k[sl]), np64(v[sl])
    if e4m3:
        j0 = int(rng.integers(spec.nkv))
        got8 = pipe.k8[bi, j0, :spec.t_past].cpu().numpy()
        assert np.array_equal(got8, oracle.e4m3_encode(kn[0, j0, :spec.t_past]))
    sets, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, spec.bsa, np64(pipe.sq[sl]),
                                npi(pipe.q_idx[sl]), np64(pipe.s_agg[sl]), npi(pipe.idx[sl]),
                                score=mode, k_e4m3=e4m3, what=f"{name} {mode}")
    err = staged_attention(qn, kn, vn, spec.t_past, sets, pipe.out[sl], spec.dtype,
                           what=f"{name} {mode}")
    print(f"[full-size variant] {name} {mode} e4m3={e4m3} b{bi}: {st}, attention {err:.2e}",
          flush=True)


@pytest.mark.parametrize("name", ["llama3b_32k", "long_128k", "long_128k_d256", "decode_64x16k"])
def test_full_size_select_equals_separate_calls(gpu, name):
    """At full size, the one-call selection the benchmark times (qk_select: the
    scoring pass fills the histogram its top-k starts from) writes what
    qk_qsel, qk_kvscore_grouped and qk_topk write one by one, bit for bit,
    twice in a row on one workspace; and its key sets are the exact top-BSA of
    its scores."""
    qk = gpu
    dev = torch.device("cuda:0")
    spec = W.spec(name)
    print(f"[full-size select] {name}", flush=True)
    case = W.make_case(spec, FULL[name], device=dev)
    s = qk.shape_of(spec)
    a = qk.Pipeline(s, device=dev, fused_select=True)
    b = qk.Pipeline(s, device=dev, fused_select=False)
    b.select(case["q"], case["k"])
    for _ in range(2):
        a.idx.fill_(-1)
        a.select(case["q"], case["k"])
        torch.cuda.synchronize()
        for x, y in ((a.q_idx, b.q_idx), (a.sq, b.sq), (a.s_agg, b.s_agg), (a.idx, b.idx)):
            assert torch.equal(x, y)
    want = oracle.select_keys(np64(a.s_agg), s.bsa)
    assert np.array_equal(npi(a.idx)[..., :want.shape[-1]], want)


def test_million_key_row(gpu):
    """A row eight times the longest workload's: one KV head of 8 query heads
    over 2^20 past keys, a 64-row chunk, NQ = 16, BSA = 16384.  The scoring
    grid runs 512 workgroups, the top-k 128 tiles of 8192 scores, the
    attention its cap of 64 key splits.  Staged comparison of every KV group,
    row and head, and the exact top-BSA of the GPU's own scores."""
    qk = gpu
    dev = torch.device("cuda:0")
    spec = W.spec("long_128k", b=1, nq=8, nkv=1, t_past=1 << 20, bcp=64, nq_keep=16, bsa=16384)
    print("[full-size] 1M-key row seed 1201", flush=True)
    case = W.make_case(spec, 1201, device=dev)
    q, k, v = case["q"], case["k"], case["v"]
    s = qk.shape_of(spec)
    pipe = qk.Pipeline(s, device=dev)
    assert pipe.fused_select
    pipe(q, k, v)
    torch.cuda.synchronize()
    qn, kn, vn = np64(q), np64(k), np64(v)
    sets, st = staged_selection(qn, kn, spec.t_past, spec.nq_keep, spec.bsa, np64(pipe.sq),
                                npi(pipe.q_idx), np64(pipe.s_agg), npi(pipe.idx), what="1M row")
    err = staged_attention(qn, kn, vn, spec.t_past, sets, pipe.out, spec.dtype,
                           gpu_lse=pipe.lse, what="1M row")
    want = oracle.select_keys(np64(pipe.s_agg), spec.bsa)
    assert np.array_equal(npi(pipe.idx)[..., :want.shape[-1]], want)
    print(f"[full-size] 1M-key row: {st}, attention err {err:.2e} (every row and head)", flush=True)
