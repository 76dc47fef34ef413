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
hands the watershed layer's index list to the layers above it (for the round
offload rewritten into staging positions: host bookkeeping over the chosen
rounds, no arithmetic of the method).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
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
    (b, nq, n, d).  With ``record`` every step's (start, index list, kept
    query positions, query scores, key scores) are kept in ``history``."""

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
            t = self.cache.length
            self.history.append((t, pipe.idx[..., :shape.n_sel].clone(), pipe.q_idx.clone(),
                                 pipe.sq.clone(), pipe.s_agg[..., :t].clone()))
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
                     scale: float = 0.0, round_off: Optional[torch.Tensor] = None,
                     top_rounds: int = 0, shared_rounds: bool = False):
    """One chunk through a stack of layers with one cache each (all at the
    same length).  Layers below `watershed` attend densely; the watershed
    layer selects (top-BSA keys, or with `round_off` the latest round plus
    `top_rounds` more, per KV head or with `shared_rounds` one choice for all
    heads; `bsa` then only sizes the attention plan); the layers
    above attend over its index list with their own queries, keys and values.
    Returns (outputs per layer, the Pipeline of the watershed layer, whose
    `idx` / `sel_len` hold the shared selection)."""
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
    n_rounds = 0 if round_off is None else round_off.numel() - 1
    pipe = Pipeline(shape, device=dev, score_mode=score_mode, k_e4m3=cw.k8 is not None,
                    n_rounds=n_rounds, top_rounds=top_rounds, shared_rounds=shared_rounds)
    if cw.k8 is not None:
        pipe.k8 = cw.k8
    pipe.select(qs[watershed], cw.k, round_off)
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


class RoundOffloadStack:
    """A layer stack with round selection at a watershed layer whose upper
    layers keep their history in pinned host memory, one block per round.

    Round Attention press release, section 02: each round's KV is split at the
    watershed layer into a lower block (the layers up to it) and an upper block
    (the layers above), stored per round in host memory and moved to the GPU a
    whole round at a time, once the watershed layer has chosen its rounds.
    Here the lower layers' caches stay on the GPU (they attend densely, and
    the watershed layer scores every round); the upper block of round r for
    layer l is one pinned host tensor (2, b, nkv, len_r, d).

    After selection, the rounds to bring in -- those chosen by some KV head,
    or with `shared_rounds` the one choice all heads share -- are copied once
    per upper layer, on a copy stream, back to back into a compact staging
    cache (the chunk's own rows after them), two of which alternate between
    layers so that a layer's copies overlap the attention of the layer
    before.  The watershed's index list is rewritten into staging positions
    (bookkeeping on the host, which already waits for the chosen-round mask
    to start the copies), and the upper layers attend over it exactly as over
    resident caches.  The staging holds as many positions as the chosen
    rounds have, so the GPU memory the upper layers take follows the
    selection (it grows to the largest choice seen; `last_staged` is the
    latest)."""

    def __init__(self, n_layers: int, watershed: int, round_off: Sequence[int], b: int, nkv: int,
                 d: int, bcp: int, dtype=torch.bfloat16, device="cuda", shared_rounds: bool = False):
        if not 0 <= watershed < n_layers - 1:
            raise ValueError("the watershed has layers above it")
        dev = torch.device(device)
        self.L, self.w, self.device = n_layers, watershed, dev
        self.off = [int(x) for x in round_off]
        self.R, self.T = len(self.off) - 1, self.off[-1]
        self.b, self.nkv, self.d, self.bcp, self.dtype = b, nkv, d, bcp, dtype
        self.shared = shared_rounds
        cap = self.T + bcp
        self.round_off_dev = torch.tensor(self.off, dtype=torch.int32, device=dev)
        self.lower = [KVCache(b, nkv, cap, d, dtype, dev) for _ in range(watershed + 1)]
        self.host = [[torch.empty((2, b, nkv, self.off[r + 1] - self.off[r], d), dtype=dtype,
                                  pin_memory=True) for r in range(self.R)]
                     for _ in range(n_layers - watershed - 1)]
        self.stage: List[torch.Tensor] = []   # compact staging caches (2, b, nkv, stage_cap, d)
        self.stage_cap = 0
        self.copy_stream = torch.cuda.Stream(device=dev)
        self.chosen_host = torch.empty((b, nkv, self.R), dtype=torch.uint8, pin_memory=True)
        self.idx_host = torch.zeros((b, nkv, self.T), dtype=torch.int32, pin_memory=True)
        self.idx_stage = torch.zeros((b, nkv, self.T), dtype=torch.int32, device=dev)
        self.last_h2d_bytes = 0
        self.last_rounds: List[int] = []
        self.last_staged = 0          # past positions staged for the latest step
        self.copy_events: List[tuple] = []  # (start, end) per upper layer, on the copy stream

    def load_history(self, layer: int, k: torch.Tensor, v: torch.Tensor):
        """Keys and values (b, nkv, >= T, d) of the T past positions of a layer."""
        T = self.T
        if layer <= self.w:
            c = self.lower[layer]
            c.k[:, :, :T].copy_(k[:, :, :T])
            c.v[:, :, :T].copy_(v[:, :, :T])
            c.length = T
        else:
            for r, blk in enumerate(self.host[layer - self.w - 1]):
                blk[0].copy_(k[:, :, self.off[r]:self.off[r + 1]])
                blk[1].copy_(v[:, :, self.off[r]:self.off[r + 1]])

    def _esz(self) -> int:
        return torch.empty((), dtype=self.dtype).element_size()

    def _rows_bytes(self, rows: int) -> int:
        return 2 * self.b * self.nkv * rows * self.d * self._esz()

    def device_kv_bytes(self) -> int:
        """KV bytes this stack holds on the GPU: the lower caches and the two
        staging caches at their current size."""
        return len(self.lower) * self._rows_bytes(self.T + self.bcp) + 2 * self._rows_bytes(self.stage_cap)

    def staged_kv_bytes(self) -> int:
        """KV bytes the latest step's selection needed on the GPU: the lower
        caches and two staging caches of the chosen rounds plus the chunk."""
        return (len(self.lower) * self._rows_bytes(self.T + self.bcp)
                + 2 * self._rows_bytes(self.last_staged + self.bcp))

    def resident_kv_bytes(self) -> int:
        """KV bytes every layer's cache would take on the GPU."""
        return self.L * self._rows_bytes(self.T + self.bcp)

    def _ensure_stage(self, cap: int):
        if cap > self.stage_cap:
            self.stage = [torch.zeros((2, self.b, self.nkv, cap, self.d), dtype=self.dtype,
                                      device=self.device) for _ in range(2)]
            self.stage_cap = cap

    def step(self, qs: Sequence[torch.Tensor], k_rows: Sequence[torch.Tensor],
             v_rows: Sequence[torch.Tensor], nq_keep: int, top_rounds: int, bsa_plan: int):
        """One chunk of bcp queries at position T through every layer.  The
        chunk's own key and value rows sit at [T, T + bcp) of the lower caches
        and right after the staged rounds in the staging caches; they are not
        added to the history, so steps may repeat over one loaded history.
        Returns (outputs per layer, the watershed's Pipeline)."""
        w, T, n = self.w, self.T, qs[0].shape[2]
        if n != self.bcp:
            raise ValueError("the stack is sized for chunks of bcp queries")
        compute = torch.cuda.current_stream(self.device)
        shape = self.lower[0].shape(qs[0].shape[1], n, min(nq_keep, n), bsa_plan)
        for layer in range(w + 1):
            self.lower[layer].append(k_rows[layer], v_rows[layer], shape)
        dws, dws_bytes = _ws(shape, "dense_attn", self.device)
        outs: List[torch.Tensor] = []
        for layer in range(w):
            out = torch.empty_like(qs[layer])
            c = self.lower[layer]
            qk_dense_attn(shape, qs[layer], c.k, c.v, out, None, dws, dws_bytes)
            outs.append(out)
        cw = self.lower[w]
        pipe = Pipeline(shape, device=self.device, n_rounds=self.R, top_rounds=top_rounds,
                        shared_rounds=self.shared)
        pipe.select(qs[w], cw.k, self.round_off_dev)
        selected = torch.cuda.Event()
        selected.record(compute)
        out = torch.empty_like(qs[w])
        qk_sparse_attn_indexed(shape, qs[w], cw.k, cw.v, pipe.idx, pipe.ld_idx, pipe.sel_len, out,
                               None, pipe.ws, pipe.ws_bytes)
        outs.append(out)
        # the rounds to bring in (the host waits for the selection only; the
        # watershed's attention keeps the GPU busy)
        with torch.cuda.stream(self.copy_stream):
            self.copy_stream.wait_event(selected)
            self.chosen_host.copy_(pipe.chosen, non_blocking=True)
        self.copy_stream.synchronize()
        chosen = self.chosen_host.numpy().astype(bool)
        need = chosen.reshape(-1, self.R).any(axis=0)
        rounds = [r for r in range(self.R) if need[r]]
        base, S = {}, 0
        for r in rounds:
            base[r] = S
            S += self.off[r + 1] - self.off[r]
        self._ensure_stage(S + n)
        # the index list in staging positions: a head's rounds, ascending,
        # each at its place in the staging
        ih = self.idx_host.numpy()
        for bi in range(self.b):
            for j in range(self.nkv):
                parts = [np.arange(base[r], base[r] + self.off[r + 1] - self.off[r], dtype=np.int32)
                         for r in range(self.R) if chosen[bi, j, r]]
                lst = np.concatenate(parts) if parts else np.zeros(0, np.int32)
                ih[bi, j, :len(lst)] = lst
        self.idx_stage.copy_(self.idx_host, non_blocking=True)
        shape_s = dataclasses.replace(shape, t_past=S, kv_cap=self.stage_cap)
        done: List[torch.cuda.Event] = []
        self.copy_events = []
        h2d = 0
        for i, layer in enumerate(range(w + 1, self.L)):
            st = self.stage[i % 2]
            with torch.cuda.stream(self.copy_stream):
                if i >= 2:
                    self.copy_stream.wait_event(done[i - 2])  # that staging cache is free again
                t0 = torch.cuda.Event(enable_timing=True)
                t0.record(self.copy_stream)
                blocks = self.host[i]
                for r in rounds:  # one host-to-device copy per round
                    ln = self.off[r + 1] - self.off[r]
                    st[:, :, :, base[r]:base[r] + ln].copy_(blocks[r], non_blocking=True)
                    h2d += blocks[r].numel() * blocks[r].element_size()
                st[0, :, :, S:S + n].copy_(k_rows[layer])
                st[1, :, :, S:S + n].copy_(v_rows[layer])
                staged = torch.cuda.Event(enable_timing=True)
                staged.record(self.copy_stream)
                self.copy_events.append((t0, staged))
            for t in (k_rows[layer], v_rows[layer]):
                t.record_stream(self.copy_stream)
            compute.wait_event(staged)
            out = torch.empty_like(qs[layer])
            qk_sparse_attn_indexed(shape_s, qs[layer], st[0], st[1], self.idx_stage, self.T,
                                   pipe.sel_len, out, None, pipe.ws, pipe.ws_bytes)
            outs.append(out)
            ev = torch.cuda.Event()
            ev.record(compute)
            done.append(ev)
        self.last_h2d_bytes, self.last_rounds, self.last_staged = h2d, rounds, S
        return outs, pipe
