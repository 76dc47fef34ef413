"""Whole prompts, decode steps and layer stacks over the C ABI.

QUOKA write-up, section 2.1: a prompt is processed in chunks of BCP queries;
the chunk that starts at position t attends the selected keys among positions
[0, t) and its own keys causally.  Section 5.1: generation follows the prompt,
one query at a time (BCP = NQ = 1).  Round Attention press release, section
02: past a watershed layer the layers attend to the history alike, so the
selection made at that layer serves every layer above it; the layers below
attend densely.

Every step of the path runs in the library's kernels.  This module orders the
calls, writes each step's new key and value rows into the caches (tensor
copies on the current stream; the E4M3 key copy through qk_keys_to_e4m3), and
hands the watershed layer's index list to the layers above it.
"""
from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import (QK_BF16, Pipeline, Shape, _ws, qk_dense_attn, qk_keys_to_e4m3,
               qk_sparse_attn_indexed)


class KVCache:
    """Keys and values of one layer, (b, nkv, cap, d); rows [0, length) hold
    the positions seen so far.  With ``e4m3`` it also keeps the 8-bit key copy
    the scoring pass can read, converted as rows are appended."""

    def __init__(self, b: int, nkv: int, cap: int, d: int, dtype=torch.bfloat16,
                 device="cuda", e4m3: bool = False):
        dev = torch.device(device)
        self.b, self.nkv, self.cap, self.d, self.dtype = b, nkv, cap, d, dtype
        self.k = torch.zeros((b, nkv, cap, d), dtype=dtype, device=dev)
        self.v = torch.zeros_like(self.k)
        self.k8 = torch.zeros((b, nkv, cap, d), dtype=torch.uint8, device=dev) if e4m3 else None
        self.length = 0

    def shape(self, nq: int, n: int, nq_keep: int, bsa: int, scale: float = 0.0) -> Shape:
        """Shape of a step of n queries starting at the current length."""
        return Shape(self.b, nq, self.nkv, self.d, n, self.length, self.cap, nq_keep, bsa, scale,
                     QK_BF16 if self.dtype == torch.bfloat16 else 0)

    def append(self, k_rows: torch.Tensor, v_rows: torch.Tensor, shape: Shape):
        """Write n new rows (b, nkv, n, d) at [length, length + n); the length
        itself advances in `advance`, after the step that reads them as its own
        keys."""
        t, n = self.length, k_rows.shape[2]
        if t + n > self.cap:
            raise ValueError(f"cache full: {t} + {n} rows > capacity {self.cap}")
        self.k[:, :, t:t + n].copy_(k_rows)
        self.v[:, :, t:t + n].copy_(v_rows)
        if self.k8 is not None:
            qk_keys_to_e4m3(shape, self.k, t, n, self.k8)

    def advance(self, n: int):
        self.length += n


class PromptRunner:
    """Chunks of a prompt, then decode steps, through one layer's cache.

    ``step`` runs one chunk (or, with one query, one decode step): it appends
    the chunk's key and value rows, runs selection and attention with the
    positions before the chunk as the past, and returns the chunk's output
    (b, nq, n, d).  With ``record`` the (start, index list) of every step is
    kept in ``history``."""

    def __init__(self, cache: KVCache, nq: int, nq_keep: int, bsa: int, score_mode: str = "cosine",
                 scale: float = 0.0, record: bool = False):
        self.cache, self.nq, self.nq_keep, self.bsa = cache, nq, nq_keep, bsa
        self.score_mode, self.scale, self.record = score_mode, scale, record
        self.history: List[tuple] = []
        self.last: Optional[Pipeline] = None

    def step(self, q: torch.Tensor, k_rows: torch.Tensor, v_rows: torch.Tensor,
             nq_keep: Optional[int] = None) -> torch.Tensor:
        n = q.shape[2]
        keep = min(self.nq_keep, n) if nq_keep is None else nq_keep
        shape = self.cache.shape(self.nq, n, keep, self.bsa, self.scale)
        self.cache.append(k_rows, v_rows, shape)
        pipe = Pipeline(shape, device=q.device, score_mode=self.score_mode,
                        k_e4m3=self.cache.k8 is not None)
        if self.cache.k8 is not None:
            pipe.k8 = self.cache.k8
        out = pipe(q.contiguous(), self.cache.k, self.cache.v)
        if self.record:
            self.history.append((self.cache.length, pipe.idx[..., :shape.n_sel].clone()))
        self.cache.advance(n)
        self.last = pipe
        return out

    def prefill(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, bcp: int) -> torch.Tensor:
        """The prompt's queries (b, nq, P, d) and its keys and values
        (b, nkv, P, d) in chunks of bcp (the last may be shorter)."""
        outs = []
        for t in range(0, q.shape[2], bcp):
            e = min(t + bcp, q.shape[2])
            outs.append(self.step(q[:, :, t:e], k[:, :, t:e], v[:, :, t:e]).clone())
        return torch.cat(outs, dim=2)

    def decode(self, q1: torch.Tensor, k1: torch.Tensor, v1: torch.Tensor) -> torch.Tensor:
        """One generated position: q1 (b, nq, 1, d), k1 / v1 (b, nkv, 1, d)."""
        return self.step(q1, k1, v1, nq_keep=1)


def layer_stack_step(qs: Sequence[torch.Tensor], caches: Sequence[KVCache],
                     k_rows: Sequence[torch.Tensor], v_rows: Sequence[torch.Tensor],
                     nq_keep: int, bsa: int, watershed: int, score_mode: str = "cosine",
                     scale: float = 0.0):
    """One chunk through a stack of layers with one cache each (all at the
    same length).  Layers below `watershed` attend densely; the watershed
    layer selects; the layers above attend over its index list with their own
    queries, keys and values.  Returns (outputs per layer, the Pipeline of the
    watershed layer, whose `idx` holds the shared selection)."""
    if not 0 <= watershed < len(qs):
        raise ValueError("the watershed is one of the layers")
    if len({c.length for c in caches}) != 1:
        raise ValueError("the layers' caches must hold the same positions")
    n = qs[0].shape[2]
    shape = caches[0].shape(qs[0].shape[1], n, min(nq_keep, n), bsa, scale)
    for c, kr, vr in zip(caches, k_rows, v_rows):
        c.append(kr, vr, shape)
    dev = qs[0].device
    cw = caches[watershed]
    pipe = Pipeline(shape, device=dev, score_mode=score_mode, k_e4m3=cw.k8 is not None)
    if cw.k8 is not None:
        pipe.k8 = cw.k8
    pipe.select(qs[watershed], cw.k)
    dws, dws_bytes = _ws(shape, "dense_attn", dev)
    outs = []
    for layer, (q, c) in enumerate(zip(qs, caches)):
        out = torch.empty_like(q)
        if layer < watershed:
            qk_dense_attn(shape, q, c.k, c.v, out, None, dws, dws_bytes)
        else:
            qk_sparse_attn_indexed(shape, q, c.k, c.v, pipe.idx, pipe.ld_idx, pipe.sel_len, out,
                                   None, pipe.ws, pipe.ws_bytes)
        outs.append(out)
    for c in caches:
        c.advance(n)
    return outs, pipe
