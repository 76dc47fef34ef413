"""Seeded synthetic inputs for query-oriented sparse KV selection.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests. It draws random tensors and arranges them in the shapes of the
workloads; it contains none of the selection or attention arithmetic.

Shapes (row-major, contiguous):
    q          (b, nq,  bcp,    d)   the prefill chunk (bcp = 1 for decode)
    k, v       (b, nkv, kv_cap, d)   rows [0, T) are the past keys/values,
                                      rows [T, T + bcp) are the chunk's own
    round_off  (R + 1,) int32        round boundaries, off[0] = 0, off[R] = T

Recipe (the pages print no data; these stand in for their workloads):
  * K and V entries are independent N(0, 1).
  * Each query head h of each sequence has its own mean mu_h = 2 * N(0, I);
    chunk queries are mu_h + N(0, I).  Optionally a few positions per head are
    replaced by fresh outliers 3 * N(0, I).
  * "Hot" keys: a fraction of past positions per (sequence, KV head), drawn
    without replacement.  With u the unit vector along the mean of mu over the
    query heads that share the KV head, a hot key k becomes
    k - (k.u) u + 4 |k.u| u: its component along u is made positive and
    stretched four-fold.  Stretching the whole key would change nothing,
    because the key score is a cosine.
  * Rounds: R lengths L_r = exp(ln 1024 + 0.5 z_r), z_r ~ N(0, 1), rescaled to
    sum to T; off[r] = round-half-even(T * sum(L[:r]) / sum(L)).
  * Floating point is drawn in fp32 and rounded to bf16 (round to nearest
    even) for the bf16 workloads.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

__all__ = ["CaseSpec", "CONFIGS", "make_case", "spec", "round_offsets"]


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    name: str
    b: int
    nq: int
    nkv: int
    d: int
    t_past: int
    bcp: int
    nq_keep: int
    bsa: int
    dtype: str = "bf16"          # "bf16" or "f32"
    hot_frac: float = 0.0        # fraction of past keys made "hot"
    n_outliers: int = 0          # outlier queries per head
    n_rounds: int = 0            # 0: no round structure
    top_rounds: int = 0          # rounds kept besides the latest one
    kv_extra: int = 0            # spare rows after the chunk (kv_cap slack)

    @property
    def kv_cap(self) -> int:
        return self.t_past + self.bcp + self.kv_extra

    @property
    def group(self) -> int:
        return self.nq // self.nkv

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def replace(self, **kw) -> "CaseSpec":
        return dataclasses.replace(self, **kw)


# The five workloads.  Names say what they are.
CONFIGS = {
    "tiny_f32": CaseSpec("tiny_f32", b=1, nq=4, nkv=2, d=64, t_past=1024, bcp=64,
                         nq_keep=32, bsa=256, dtype="f32", n_outliers=8),
    "llama3b_32k": CaseSpec("llama3b_32k", b=1, nq=24, nkv=8, d=128, t_past=32768,
                            bcp=256, nq_keep=32, bsa=8192, hot_frac=0.02),
    "decode_64x16k": CaseSpec("decode_64x16k", b=64, nq=32, nkv=8, d=128,
                              t_past=16384, bcp=1, nq_keep=1, bsa=2048,
                              hot_frac=0.01),
    "rounds_64k": CaseSpec("rounds_64k", b=1, nq=32, nkv=8, d=128, t_past=65536,
                           bcp=512, nq_keep=32, bsa=0, n_rounds=64, top_rounds=8),
    "long_128k": CaseSpec("long_128k", b=1, nq=64, nkv=8, d=128, t_past=131072,
                          bcp=512, nq_keep=32, bsa=16384, hot_frac=0.005),
    "long_128k_d256": CaseSpec("long_128k_d256", b=1, nq=64, nkv=8, d=256,
                               t_past=131072, bcp=512, nq_keep=32, bsa=16384,
                               hot_frac=0.005),
}


def spec(name: str, **overrides) -> CaseSpec:
    s = CONFIGS[name]
    return s.replace(**overrides) if overrides else s


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    # one independent stream per tensor role
    g.manual_seed((seed * 1_000_003 + stream * 7919) % (2**63 - 1))
    return g


def round_offsets(t_past: int, n_rounds: int, seed: int) -> np.ndarray:
    """Round boundaries for a multi-round dialogue of t_past tokens."""
    rng = np.random.Generator(np.random.PCG64(seed * 31 + 5))
    z = rng.standard_normal(n_rounds)
    lengths = np.exp(math.log(1024.0) + 0.5 * z)
    cum = np.concatenate([[0.0], np.cumsum(lengths)])
    off = np.rint(t_past * cum / cum[-1]).astype(np.int64)   # rint: half to even
    off[0], off[-1] = 0, t_past
    if np.any(np.diff(off) < 1):
        raise ValueError("a round came out empty; pick another seed")
    return off.astype(np.int32)


def make_case(s: CaseSpec, seed: int, device="cpu") -> dict:
    """Draw one workload instance.  Same (spec, seed, device) -> same bytes."""
    dev = torch.device(device)
    b, nq, nkv, d, G = s.b, s.nq, s.nkv, s.d, s.group
    f32 = torch.float32

    mu = 2.0 * torch.randn((b, nq, 1, d), generator=_gen(seed, 1, dev), device=dev, dtype=f32)
    q = mu + torch.randn((b, nq, s.bcp, d), generator=_gen(seed, 2, dev), device=dev, dtype=f32)
    if s.n_outliers:
        go = _gen(seed, 3, dev)
        for bi in range(b):
            for h in range(nq):
                pos = torch.randperm(s.bcp, generator=go, device=dev)[: s.n_outliers]
                q[bi, h, pos] = 3.0 * torch.randn((s.n_outliers, d), generator=go, device=dev, dtype=f32)

    k = torch.randn((b, nkv, s.kv_cap, d), generator=_gen(seed, 4, dev), device=dev, dtype=f32)
    v = torch.randn((b, nkv, s.kv_cap, d), generator=_gen(seed, 5, dev), device=dev, dtype=f32)
    if s.kv_extra:
        k[:, :, s.t_past + s.bcp:] = 0.0
        v[:, :, s.t_past + s.bcp:] = 0.0

    n_hot = int(round(s.hot_frac * s.t_past))
    hot_pos = None
    if n_hot > 0:
        gh = _gen(seed, 6, dev)
        hot_pos = torch.empty((b, nkv, n_hot), dtype=torch.int64, device=dev)
        u = mu[:, :, 0, :].reshape(b, nkv, G, d).mean(dim=2)
        u = u / u.norm(dim=-1, keepdim=True)
        for bi in range(b):
            for j in range(nkv):
                pos = torch.randperm(s.t_past, generator=gh, device=dev)[:n_hot]
                hot_pos[bi, j] = pos
                kk = k[bi, j, pos]
                proj = kk @ u[bi, j]
                k[bi, j, pos] = kk + (4.0 * proj.abs() - proj)[:, None] * u[bi, j][None, :]

    out = {
        "q": q.to(s.torch_dtype).contiguous(),
        "k": k.to(s.torch_dtype).contiguous(),
        "v": v.to(s.torch_dtype).contiguous(),
        "round_off": None,
        "hot_pos": hot_pos,
    }
    if s.n_rounds:
        out["round_off"] = torch.from_numpy(round_offsets(s.t_past, s.n_rounds, seed)).to(dev)
    return out
