"""Whole prompts, decode steps and layer stacks through the driver, against the
oracle's prompt_chunks and layer_stack on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (ATTN_TOL, assert_set_within_boundary, assert_sorted_unique, group_agreement,
                    max_abs, np64, npi)

pytestmark = pytest.mark.gpu

NQ, NKV, D_HEAD = 6, 2, 128


def _dev():
    return torch.device("cuda:0")


def _sequence(n_pos, seed, layers=1):
    """Queries, keys and values of n_pos positions per layer, drawn with the
    llama3b_32k recipe (queries around a per-head mean, hot keys)."""
    out = []
    for layer in range(layers):
        spec = W.spec("llama3b_32k", nq=NQ, nkv=NKV, t_past=n_pos, bcp=n_pos, nq_keep=16,
                      bsa=n_pos)
        case = W.make_case(spec, seed + 101 * layer)
        out.append(tuple(case[n][:, :, :n_pos].contiguous().to(_dev()) for n in ("q", "k", "v")))
    return out


def test_prompt_full_budget_is_causal_attention(gpu):
    """A budget covering every past position turns the chunked prompt plus its
    decode steps into causal attention over the whole sequence: chunks of 256
    with a ragged last one, a first chunk with no past, three decode steps."""
    from sparse_kv_selection_amd import driver
    P, n_dec = 700, 3
    (q, k, v), = _sequence(P + n_dec, 3001)
    cache = driver.KVCache(1, NKV, P + n_dec + 5, D_HEAD, device=_dev())
    run = driver.PromptRunner(cache, NQ, 16, bsa=P + n_dec)
    parts = [run.prefill(q[:, :, :P], k[:, :, :P], v[:, :, :P], 256)]
    for i in range(P, P + n_dec):
        parts.append(run.decode(q[:, :, i:i + 1], k[:, :, i:i + 1], v[:, :, i:i + 1]).clone())
    torch.cuda.synchronize()
    got = torch.cat(parts, dim=2)
    want, _ = oracle.prompt_chunks(np64(q), np64(k), np64(v), 256, 16, P + n_dec, n_decode=n_dec)
    assert cache.length == P + n_dec
    assert max_abs(got, want) <= ATTN_TOL["bf16"]


@pytest.mark.parametrize("e4m3", [False, True])
def test_prompt_chunks_against_oracle(gpu, e4m3):
    """Limited budget: every step's kept queries and key set agree with the
    oracle's step (near-boundary swaps only), and every step's output equals
    the oracle's attention over the GPU's own key sets."""
    from sparse_kv_selection_amd import driver
    P, n_dec, bcp, bsa = 640, 2, 256, 150
    (q, k, v), = _sequence(P + n_dec, 3002)
    qn, kn, vn = np64(q), np64(k), np64(v)
    cache = driver.KVCache(1, NKV, P + n_dec, D_HEAD, device=_dev(), e4m3=e4m3)
    run = driver.PromptRunner(cache, NQ, 16, bsa=bsa, record=True)
    starts = list(range(0, P, bcp)) + list(range(P, P + n_dec))
    outs, qidx = [], []
    for t in starts:
        e = min(t + bcp, P) if t < P else t + 1
        if t < P:
            o = run.step(q[:, :, t:e], k[:, :, t:e], v[:, :, t:e])
        else:
            o = run.decode(q[:, :, t:e], k[:, :, t:e], v[:, :, t:e])
        outs.append(np64(o))
        qidx.append(npi(run.last.q_idx))
    torch.cuda.synchronize()
    _, steps = oracle.prompt_chunks(qn, kn, vn, bcp, 16, bsa, n_decode=n_dec, k_e4m3=e4m3)
    assert len(steps) == len(starts) == len(run.history)
    for i, (t, ref) in enumerate(zip(starts, steps)):
        t_hist, idx = run.history[i]
        idx = npi(idx)
        assert t_hist == t and idx.shape[-1] == min(bsa, t)
        e = outs[i].shape[2] + t
        agree = group_agreement(qidx[i], ref["qidx"], NQ // NKV)
        for j in range(NKV):
            if t > 0:
                assert_sorted_unique(idx[0, j], t)
            if t > 0 and agree[0, j]:
                assert_set_within_boundary(idx[0, j], ref["kidx"][0, j], ref["s_agg"][0, j],
                                           min(bsa, t), what=f"step {i} j{j}")
        sets = [[idx[0, j] for j in range(NKV)]]
        o_ref, _ = oracle.attention(qn[:, :, t:e], kn, vn, t, sets)
        assert np.abs(outs[i] - o_ref).max() <= ATTN_TOL["bf16"], (i, t)


def test_layer_stack_watershed_reuse(gpu):
    """Three layers, watershed 1: layer 0 is dense attention, layer 1 selects
    (key sets against the oracle's within the boundary rule), layer 2 attends
    over layer 1's index list with its own queries, keys and values."""
    from sparse_kv_selection_amd import driver
    t_past, bcp, bsa, L, w = 600, 128, 200, 3, 1
    layers = _sequence(t_past + bcp, 3003, layers=L)
    caches = []
    for (q, k, v) in layers:
        c = driver.KVCache(1, NKV, t_past + bcp, D_HEAD, device=_dev())
        c.k[:, :, :t_past].copy_(k[:, :, :t_past])
        c.v[:, :, :t_past].copy_(v[:, :, :t_past])
        c.advance(t_past)
        caches.append(c)
    qs = [q[:, :, t_past:].contiguous() for (q, _, _) in layers]
    krows = [k[:, :, t_past:] for (_, k, _) in layers]
    vrows = [v[:, :, t_past:] for (_, _, v) in layers]
    outs, pipe = driver.layer_stack_step(qs, caches, krows, vrows, 16, bsa, w)
    torch.cuda.synchronize()
    qn = [np64(x) for x in qs]
    kn = [np64(k) for (_, k, _) in layers]
    vn = [np64(v) for (_, _, v) in layers]
    ref_outs, _ = oracle.layer_stack(qn, kn, vn, t_past, 16, bsa, w)
    assert max_abs(outs[0], ref_outs[0]) <= ATTN_TOL["bf16"]
    ref_w = oracle.pipeline(qn[w], kn[w], vn[w], t_past, 16, bsa, with_attention=False)
    idx = npi(pipe.idx)
    agree = group_agreement(npi(pipe.q_idx), ref_w["qidx"], NQ // NKV)
    for j in range(NKV):
        assert_sorted_unique(idx[0, j], t_past)
        if agree[0, j]:
            assert_set_within_boundary(idx[0, j], ref_w["kidx"][0, j], ref_w["s_agg"][0, j], bsa)
    sets = [[idx[0, j] for j in range(NKV)]]
    for layer in (w, w + 1):
        o_ref, _ = oracle.attention(qn[layer], kn[layer], vn[layer], t_past, sets)
        assert max_abs(outs[layer], o_ref) <= ATTN_TOL["bf16"], layer
    assert all(c.length == t_past + bcp for c in caches)


def test_round_offload_matches_resident_stack(gpu):
    """Upper layers held per round in host memory: every layer's output equals
    the resident stack's bit for bit; the copies are the rounds some KV head
    chose, once per upper layer; the watershed's rounds agree with the
    oracle's (near-tie swaps only) and the upper layers with the oracle's
    attention over the GPU's key sets; the GPU holds fewer KV bytes."""
    from sparse_kv_selection_amd import driver
    L, w, T, bcp, R, top = 5, 1, 3000, 128, 12, 3
    off = W.round_offsets(T, R, 11)
    layers = _sequence(T + bcp, 4001, layers=L)
    stack = driver.RoundOffloadStack(L, w, off, 1, NKV, D_HEAD, bcp, device=_dev())
    caches = []
    for layer, (q, k, v) in enumerate(layers):
        stack.load_history(layer, k, v)
        c = driver.KVCache(1, NKV, T + bcp, D_HEAD, device=_dev())
        c.k[:, :, :T].copy_(k[:, :, :T])
        c.v[:, :, :T].copy_(v[:, :, :T])
        c.advance(T)
        caches.append(c)
    qs = [q[:, :, T:].contiguous() for (q, _, _) in layers]
    krows = [k[:, :, T:].contiguous() for (_, k, _) in layers]
    vrows = [v[:, :, T:].contiguous() for (_, _, v) in layers]
    outs, pipe = stack.step(qs, krows, vrows, 16, top, bsa_plan=T // 4)
    off_dev = torch.tensor(off, dtype=torch.int32, device=_dev())
    outs_r, pipe_r = driver.layer_stack_step(qs, caches, krows, vrows, 16, T // 4, w,
                                             round_off=off_dev, top_rounds=top)
    torch.cuda.synchronize()
    for layer in range(L):
        assert torch.equal(outs[layer], outs_r[layer]), layer
    assert torch.equal(pipe.sel_len, pipe_r.sel_len)
    chosen = npi(pipe.chosen)
    union = [r for r in range(R) if chosen[..., r].any()]
    assert stack.last_rounds == union
    lens = np.diff(np.asarray(off))
    assert stack.last_h2d_bytes == (L - w - 1) * sum(2 * NKV * int(lens[r]) * D_HEAD * 2 for r in union)
    assert stack.device_kv_bytes() < stack.resident_kv_bytes()
    # the watershed's rounds against the oracle's (the latest round is always kept)
    qn = [np64(x) for x in qs]
    kn = [np64(k) for (_, k, _) in layers]
    vn = [np64(v) for (_, _, v) in layers]
    ref = oracle.pipeline(qn[w], kn[w], vn[w], T, 16, 0, round_off=np.asarray(off), top_rounds=top,
                          with_attention=False)
    for j in range(NKV):
        got = np.flatnonzero(chosen[0, j])
        want = np.asarray(ref["rounds"][0][j])
        sr = np.asarray(ref["s_round"][0, j], dtype=np.float64).copy()
        sr[R - 1] = np.inf
        assert_set_within_boundary(got, want, sr, top + 1, what=f"rounds j{j}")
    idx, sl = npi(pipe.idx), npi(pipe.sel_len)
    sets = [[idx[0, j, :sl[0, j]] for j in range(NKV)]]
    for layer in (w, w + 1, L - 1):
        o_ref, _ = oracle.attention(qn[layer], kn[layer], vn[layer], T, sets)
        assert max_abs(outs[layer], o_ref) <= ATTN_TOL["bf16"], layer
