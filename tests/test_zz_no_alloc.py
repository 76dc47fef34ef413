"""The allocation-free attention entry point (for callers that cannot
allocate) against qk_sparse_attn_indexed, through the C ABI: the same kernels
with the library's fixed scratch array in place of a caller workspace, so the
outputs must be identical bit for bit.  Two calls in a row, the second on a
smaller shape (the array keeps the first call's partials)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


def _check(qk, spec, seed):
    dev = torch.device("cuda:0")
    print(f"[no-alloc] T={spec.t_past} bcp={spec.bcp} BSA={spec.bsa} seed {seed}", flush=True)
    case = W.make_case(spec, seed, device=dev)
    q, k, v = case["q"], case["k"], case["v"]
    s = qk.shape_of(spec)
    pipe = qk.Pipeline(s, device=dev)
    pipe(q, k, v)                                   # selection + the workspace entry point
    out = torch.full_like(pipe.out, 7.0)
    lse = torch.full_like(pipe.lse, 7.0)
    qk.qk_sparse_attn_indexed_noalloc(s, q, k, v, pipe.idx, pipe.ld_idx, pipe.sel_len, out, lse)
    torch.cuda.synchronize()
    assert qk.qk_workspace_bytes(s, "sparse_attn") > 0      # the partials path is exercised
    assert torch.equal(out, pipe.out)
    assert torch.equal(lse, pipe.lse)


def test_no_alloc_matches_workspace_entry(gpu):
    qk = gpu
    _check(qk, W.spec("llama3b_32k"), 1002)                                  # 15.5 MiB of partials
    _check(qk, W.spec("llama3b_32k", t_past=5000, bcp=200, bsa=1300), 1002)  # smaller, second call


def test_no_alloc_round_selection(gpu):
    """Ragged (round) selections through the same entry point."""
    qk = gpu
    dev = torch.device("cuda:0")
    spec = W.spec("rounds_64k", nq=8, nkv=2, t_past=6000, bcp=128, n_rounds=16, top_rounds=4)
    case = W.make_case(spec, 1004, device=dev)
    s = qk.shape_of(spec, bsa=spec.t_past)
    pipe = qk.Pipeline(s, device=dev, n_rounds=spec.n_rounds, top_rounds=spec.top_rounds)
    pipe(case["q"], case["k"], case["v"], case["round_off"])
    out = torch.empty_like(pipe.out)
    qk.qk_sparse_attn_indexed_noalloc(s, case["q"], case["k"], case["v"], pipe.idx, pipe.ld_idx,
                                      pipe.sel_len, out, None)
    torch.cuda.synchronize()
    assert torch.equal(out, pipe.out)
