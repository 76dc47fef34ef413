"""Whole prompts, decode steps and layer stacks through the driver, against the
oracle's prompt_chunks and layer_stack on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from parity import (ATTN_TOL, assert_set_within_boundary, max_abs, np64, npi, staged_attention,
                    staged_selection)

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
    """Limited budget, every step compared stage by stage: kept queries
    against the oracle's run of the step, then the oracle's key scores, key
    selection and attention on the GPU's own kept queries and key sets, for
    every KV group and every row of the step."""
    from sparse_kv_selection_amd import driver
    P, n_dec, bcp, bsa = 640, 2, 256, 150
    (q, k, v), = _sequence(P + n_dec, 3002)
    qn, kn, vn = np64(q), np64(k), np64(v)
    cache = driver.KVCache(1, NKV, P + n_dec, D_HEAD, device=_dev(), e4m3=e4m3)
    run = driver.PromptRunner(cache, NQ, 16, bsa=bsa, record=True)
    starts = list(range(0, P, bcp)) + list(range(P, P + n_dec))
    outs = []
    for t in starts:
        e = min(t + bcp, P) if t < P else t + 1
        if t < P:
            o = run.step(q[:, :, t:e], k[:, :, t:e], v[:, :, t:e])
        else:
            o = run.decode(q[:, :, t:e], k[:, :, t:e], v[:, :, t:e])
        outs.append(o.clone())
    torch.cuda.synchronize()
    assert len(run.history) == len(starts)
    for i, t in enumerate(starts):
        t_hist, idx, q_idx, sq, s_agg = run.history[i]
        n = outs[i].shape[2]
        keep = min(16, n) if t < P else 1
        assert t_hist == t and idx.shape[-1] == min(bsa, t)
        qs = qn[:, :, t:t + n]
        sets, st = staged_selection(qs, kn, t, keep, bsa, np64(sq), npi(q_idx), np64(s_agg),
                                    npi(idx), k_e4m3=e4m3, what=f"step {i} at {t}")
        err = staged_attention(qs, kn, vn, t, sets, outs[i], "bf16", what=f"step {i} at {t}")
        print(f"[prompt] step {i} at {t}: {st}, attention {err:.2e}")


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
    # the watershed's selection, stage by stage on its own kept queries; the
    # layers above attend over it with their own rows
    sets, st = staged_selection(qn[w], kn[w], t_past, 16, bsa, np64(pipe.sq), npi(pipe.q_idx),
                                np64(pipe.s_agg), npi(pipe.idx), what="watershed")
    for layer in (w, w + 1):
        staged_attention(qn[layer], kn[layer], vn[layer], t_past, sets, outs[layer], "bf16",
                         what=f"layer {layer}")
    assert all(c.length == t_past + bcp for c in caches)


@pytest.mark.parametrize("shared", [False, True])
def test_round_offload_matches_resident_stack(gpu, shared):
    """Upper layers held per round in host memory: every layer's output equals
    the resident stack's bit for bit; the copies are the rounds some KV head
    chose (with the shared choice: the same rounds for every head), once per
    upper layer, into staging caches sized to them; the watershed's rounds
    agree with the oracle's (near-tie swaps only; shared: exactly the
    oracle's shared choice on the GPU's round scores) and the upper layers
    with the oracle's attention over the GPU's key sets; the GPU holds fewer
    KV bytes, by the rounds staged."""
    from sparse_kv_selection_amd import driver
    L, w, T, bcp, R, top = 5, 1, 3000, 128, 12, 3
    off = W.round_offsets(T, R, 11)
    layers = _sequence(T + bcp, 4001, layers=L)
    stack = driver.RoundOffloadStack(L, w, off, 1, NKV, D_HEAD, bcp, device=_dev(),
                                     shared_rounds=shared)
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
                                             round_off=off_dev, top_rounds=top,
                                             shared_rounds=shared)
    torch.cuda.synchronize()
    chosen = npi(pipe.chosen)
    union = [r for r in range(R) if chosen[..., r].any()]
    lens = np.diff(np.asarray(off))
    staged = sum(int(lens[r]) for r in union)
    # (the staged attention keeps the resident plan while the staging holds at
    # least the plan's keys: then the outputs agree bit for bit)
    assert staged >= T // 4
    for layer in range(L):
        assert torch.equal(outs[layer], outs_r[layer]), layer
    assert torch.equal(pipe.sel_len, pipe_r.sel_len)
    assert stack.last_rounds == union
    assert stack.last_staged == staged
    assert stack.last_h2d_bytes == (L - w - 1) * sum(2 * NKV * int(lens[r]) * D_HEAD * 2 for r in union)
    assert stack.staged_kv_bytes() < stack.resident_kv_bytes()
    assert stack.staged_kv_bytes() == (w + 1) * 2 * NKV * (T + bcp) * D_HEAD * 2 + 2 * 2 * NKV * (staged + bcp) * D_HEAD * 2
    if shared:
        assert len(union) == top + 1 and all(np.array_equal(chosen[0, j], chosen[0, 0]) for j in range(NKV))
        want = oracle.select_rounds_shared(np64(pipe.s_round), top)
        assert all(np.flatnonzero(chosen[0, j]).tolist() == want[0][j].tolist() for j in range(NKV))
    # the watershed's rounds against the oracle's (the latest round is always kept)
    qn = [np64(x) for x in qs]
    kn = [np64(k) for (_, k, _) in layers]
    vn = [np64(v) for (_, _, v) in layers]
    sets, st = staged_selection(qn[w], kn[w], T, 16, T // 4, np64(pipe.sq), npi(pipe.q_idx),
                                np64(pipe.s_agg), npi(pipe.idx), round_off=np.asarray(off),
                                top_rounds=top, gpu_sel_len=npi(pipe.sel_len),
                                shared_rounds=shared, what="watershed")
    for j in range(NKV):   # the chosen-round mask names the same rounds as the index list
        rounds_in_list = np.unique(np.searchsorted(off, sets[0][j], side="right") - 1)
        assert np.array_equal(np.flatnonzero(chosen[0, j]), rounds_in_list)
    for layer in (w, w + 1, L - 1):
        staged_attention(qn[layer], kn[layer], vn[layer], T, sets, outs[layer], "bf16",
                         what=f"layer {layer}")
