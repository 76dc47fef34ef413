"""Seeded input generator: determinism and the structure each workload promises."""
import numpy as np
import torch

import workloads as W


def test_deterministic_and_shapes():
    s = W.spec("tiny_f32")
    a, b = W.make_case(s, 1001), W.make_case(s, 1001)
    for n in ("q", "k", "v"):
        assert torch.equal(a[n], b[n])
    assert a["q"].shape == (1, 4, 64, 64) and a["q"].dtype == torch.float32
    assert a["k"].shape == (1, 2, 1024 + 64, 64)
    c = W.make_case(s, 1101)
    assert not torch.equal(a["k"], c["k"])


def test_hot_keys_lean_toward_the_group_mean_query():
    s = W.spec("llama3b_32k", t_past=2048, bsa=512)
    case = W.make_case(s, 7)
    k = case["k"].float()
    q = case["q"].float()
    G = s.group
    u = q.mean(dim=2).reshape(s.b, s.nkv, G, s.d).mean(dim=2)
    u = u / u.norm(dim=-1, keepdim=True)
    cos = torch.einsum("bjtd,bjd->bjt", k[:, :, : s.t_past], u) / k[:, :, : s.t_past].norm(dim=-1)
    n_hot = round(s.hot_frac * s.t_past)
    hot = case["hot_pos"]
    assert hot.shape == (s.b, s.nkv, n_hot)
    mask = torch.zeros_like(cos, dtype=torch.bool)
    mask.scatter_(2, hot, True)
    # the component along the mean direction is made positive and stretched
    # four-fold: hot keys sit at cosine ~0.25, plain keys at ~N(0, 1/d)
    assert float(cos[mask].min()) > -0.02
    assert float(cos[mask].mean()) > 0.2
    assert abs(float(cos[~mask].mean())) < 0.01


def test_round_offsets():
    off = W.round_offsets(65536, 64, 1004)
    assert off[0] == 0 and off[-1] == 65536 and len(off) == 65
    lengths = np.diff(off)
    assert lengths.min() >= 1
    # lognormal(ln 1024, 0.5) renormalised: median length near T / R
    assert 400 < np.median(lengths) < 2000


def test_bf16_rounding_is_exact_widening():
    s = W.spec("llama3b_32k", t_past=256, bsa=64, bcp=16)
    case = W.make_case(s, 3)
    k = case["k"]
    assert k.dtype == torch.bfloat16
    assert torch.equal(k.float().to(torch.bfloat16), k)
