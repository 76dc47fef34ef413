"""Query-oriented sparse KV selection (QUOKA) and attention over the selected
keys on AMD Instinct MI355X (gfx950).

Thin ctypes binding of the C ABI in include/qk.h: every ``qk_*`` function here
has the name and argument order of its C counterpart, takes torch tensors
(device memory) and marshals their pointers and the current HIP stream.  No
step of the method runs in Python; the native library is required and its
absence is an error.

Pipeline helpers (``Shape``, ``Pipeline``) only allocate buffers with torch and
call the same entry points in order.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqk.so")

QK_F32, QK_BF16 = 0, 1
OPS = {"qsel": 0, "kvscore": 1, "topk": 2, "round_select": 3, "gather": 4,
       "sparse_attn": 5, "dense_attn": 6, "select": 7}
QK_SCORE_COSINE, QK_SCORE_DOT = 0, 1    # qk_score_mode
QK_KEYS_DTYPE, QK_KEYS_E4M3 = 0, 1      # qk_key_format
QK_ROUNDS_KEEP_LATEST, QK_ROUNDS_SHARED = 1, 2   # qk_round_select flags
SCORE_MODES = {"cosine": QK_SCORE_COSINE, "dot": QK_SCORE_DOT}
EXPORTED = ["qk_abi_version", "qk_status_string", "qk_workspace_bytes", "qk_qsel",
            "qk_kvscore", "qk_kvscore_grouped", "qk_kvscore_variant", "qk_keys_to_e4m3",
            "qk_topk", "qk_select", "qk_round_select", "qk_gather", "qk_sparse_attn",
            "qk_sparse_attn_indexed", "qk_sparse_attn_indexed_noalloc", "qk_dense_attn",
            "qk_calib_matrix_rate", "qk_calib_read_rate"]
QK_NOALLOC_SCRATCH_BYTES = 20 << 20    # the fixed scratch array of qk_sparse_attn_indexed_noalloc


class QKError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: status {code} ({text})")
        self.code = code


class _Shape(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int32), ("nq", ctypes.c_int32), ("nkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("bcp", ctypes.c_int32), ("t_past", ctypes.c_int32),
                ("kv_cap", ctypes.c_int32), ("nq_keep", ctypes.c_int32), ("bsa", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


@dataclasses.dataclass
class Shape:
    """Problem description (the C qk_shape)."""
    b: int
    nq: int
    nkv: int
    d: int
    bcp: int
    t_past: int
    kv_cap: int
    nq_keep: int
    bsa: int
    scale: float = 0.0
    dtype: int = QK_BF16

    def c(self) -> _Shape:
        return _Shape(self.b, self.nq, self.nkv, self.d, self.bcp, self.t_past, self.kv_cap,
                      self.nq_keep, self.bsa, float(self.scale), self.dtype)

    @property
    def group(self) -> int:
        return self.nq // self.nkv

    @property
    def n_sel(self) -> int:
        return min(self.bsa, self.t_past)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == QK_BF16 else torch.float32


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqk.so (built by sparse_kv_selection_amd/build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.POINTER(_Shape)
    sig = {
        "qk_abi_version": ([], I),
        "qk_status_string": ([I], ctypes.c_char_p),
        "qk_workspace_bytes": ([F, I], SZ),
        "qk_qsel": ([F, P, P, P, P, P], I),
        "qk_kvscore": ([F, P, P, P, P], I),
        "qk_kvscore_grouped": ([F, P, P, P, P, P], I),
        "qk_kvscore_variant": ([F, P, P, P, I, I, P, P], I),
        "qk_keys_to_e4m3": ([F, P, I, I, P, P], I),
        "qk_topk": ([I, I, I, P, I, P, I, P, SZ, P], I),
        "qk_select": ([F, P, P, I, I, P, P, P, P, P, I, P, SZ, P], I),
        "qk_round_select": ([F, P, I, P, I, I, P, I, P, P, P, P], I),
        "qk_gather": ([F, P, P, P, I, P, P, P, P], I),
        "qk_sparse_attn": ([F, P, P, P, I, P, P, P, P, P, P, SZ, P], I),
        "qk_sparse_attn_indexed": ([F, P, P, P, P, I, P, P, P, P, SZ, P], I),
        "qk_sparse_attn_indexed_noalloc": ([F, P, P, P, P, I, P, P, P, P], I),
        "qk_dense_attn": ([F, P, P, P, P, P, P, SZ, P], I),
        "qk_calib_matrix_rate": ([I, I, P, P], I),
        "qk_calib_read_rate": ([F, P, I, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, code: int):
    if code != 0:
        raise QKError(fn, code, qk_status_string(code))


def _sh(shape) -> ctypes.POINTER(_Shape):
    return ctypes.byref(shape.c() if isinstance(shape, Shape) else shape)


# ---------------------------------------------------------------------------
# C-ABI mirrors (same names, same argument order; tensors in, pointers out)
# ---------------------------------------------------------------------------
def qk_abi_version() -> int:
    return load_library().qk_abi_version()


def qk_status_string(code: int) -> str:
    return load_library().qk_status_string(code).decode()


def qk_workspace_bytes(shape, op) -> int:
    op = OPS[op] if isinstance(op, str) else op
    return load_library().qk_workspace_bytes(_sh(shape), op)


def qk_qsel(shape, q, q_idx, sq, q_group, stream=None):
    _check("qk_qsel", load_library().qk_qsel(_sh(shape), _ptr(q), _ptr(q_idx), _ptr(sq),
                                              _ptr(q_group), _stream(stream)))


def qk_kvscore(shape, q_group, k, s_agg, stream=None):
    _check("qk_kvscore", load_library().qk_kvscore(_sh(shape), _ptr(q_group), _ptr(k),
                                                    _ptr(s_agg), _stream(stream)))


def qk_kvscore_grouped(shape, q, q_idx, k, s_agg, stream=None):
    _check("qk_kvscore_grouped", load_library().qk_kvscore_grouped(
        _sh(shape), _ptr(q), _ptr(q_idx), _ptr(k), _ptr(s_agg), _stream(stream)))


def qk_kvscore_variant(shape, q, q_idx, k, key_format, mode, s_agg, stream=None):
    """Grouped scoring with a score mode (QK_SCORE_COSINE / QK_SCORE_DOT, or
    "cosine" / "dot") and key storage (QK_KEYS_DTYPE / QK_KEYS_E4M3)."""
    mode = SCORE_MODES[mode] if isinstance(mode, str) else int(mode)
    _check("qk_kvscore_variant", load_library().qk_kvscore_variant(
        _sh(shape), _ptr(q), _ptr(q_idx), _ptr(k), int(key_format), mode, _ptr(s_agg),
        _stream(stream)))


def qk_keys_to_e4m3(shape, k, row0, nrows, k8, stream=None):
    """Rows [row0, row0 + nrows) of every (b, KV head) block of k as E4M3 codes
    at the same positions of the uint8 tensor k8 (same shape as k)."""
    _check("qk_keys_to_e4m3", load_library().qk_keys_to_e4m3(
        _sh(shape), _ptr(k), int(row0), int(nrows), _ptr(k8), _stream(stream)))


def topk_workspace_bytes(rows: int, n: int) -> int:
    """qk_workspace_bytes(QK_OP_TOPK) for `rows` rows of `n` scores."""
    return qk_workspace_bytes(Shape(rows, 1, 1, 64, 1, n, n + 1, 1, 1), "topk")


def qk_topk(rows, n, k, scores, ld_scores, idx, ld_idx, ws=None, ws_bytes=0, stream=None):
    """ws=None: a workspace of the required size is allocated for this call."""
    if ws is None:
        ws_bytes = topk_workspace_bytes(rows, n)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device) if ws_bytes else None
    _check("qk_topk", load_library().qk_topk(rows, n, k, _ptr(scores), ld_scores, _ptr(idx),
                                              ld_idx, _ptr(ws), ws_bytes, _stream(stream)))


def qk_select(shape, q, k, key_format, mode, q_idx, sq, s_agg, idx, ld_idx, ws=None, ws_bytes=0,
              stream=None, k_new=None):
    """qk_qsel + qk_kvscore_variant + qk_topk in one call.  ws=None: a
    workspace of the required size is allocated for this call.  k_new (8-bit
    keys only): the dtype cache whose chunk rows the scoring pass also stores
    as E4M3 codes into k."""
    mode = SCORE_MODES[mode] if isinstance(mode, str) else int(mode)
    if ws is None:
        ws, ws_bytes = _ws(shape, "select", q.device)
    _check("qk_select", load_library().qk_select(
        _sh(shape), _ptr(q), _ptr(k), int(key_format), mode, _ptr(k_new), _ptr(q_idx), _ptr(sq),
        _ptr(s_agg), _ptr(idx), ld_idx, _ptr(ws), ws_bytes, _stream(stream)))


def qk_round_select(shape, s_agg, n_rounds, round_off, top_r, keep_latest, idx, ld_idx,
                    sel_len, s_round=None, chosen=None, stream=None):
    _check("qk_round_select", load_library().qk_round_select(
        _sh(shape), _ptr(s_agg), n_rounds, _ptr(round_off), top_r, int(keep_latest), _ptr(idx),
        ld_idx, _ptr(sel_len), _ptr(s_round), _ptr(chosen), _stream(stream)))


def qk_gather(shape, k, v, idx, ld_idx, sel_len, k_sel, v_sel, stream=None):
    _check("qk_gather", load_library().qk_gather(_sh(shape), _ptr(k), _ptr(v), _ptr(idx), ld_idx,
                                                  _ptr(sel_len), _ptr(k_sel), _ptr(v_sel),
                                                  _stream(stream)))


def qk_sparse_attn(shape, q, k_sel, v_sel, ld_sel, sel_len, k, v, out, lse=None, ws=None,
                   ws_bytes=0, stream=None):
    _check("qk_sparse_attn", load_library().qk_sparse_attn(
        _sh(shape), _ptr(q), _ptr(k_sel), _ptr(v_sel), ld_sel, _ptr(sel_len), _ptr(k), _ptr(v),
        _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def qk_sparse_attn_indexed(shape, q, k, v, idx, ld_idx, sel_len, out, lse=None, ws=None,
                           ws_bytes=0, stream=None):
    _check("qk_sparse_attn_indexed", load_library().qk_sparse_attn_indexed(
        _sh(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), ld_idx, _ptr(sel_len), _ptr(out),
        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def qk_sparse_attn_indexed_noalloc(shape, q, k, v, idx, ld_idx, sel_len, out, lse=None,
                                   stream=None):
    """qk_sparse_attn_indexed with the library's fixed scratch array instead of
    a workspace (no allocation; calls overlapping on one GPU race)."""
    _check("qk_sparse_attn_indexed_noalloc", load_library().qk_sparse_attn_indexed_noalloc(
        _sh(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), ld_idx, _ptr(sel_len), _ptr(out),
        _ptr(lse), _stream(stream)))


def qk_dense_attn(shape, q, k, v, out, lse=None, ws=None, ws_bytes=0, stream=None):
    _check("qk_dense_attn", load_library().qk_dense_attn(
        _sh(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws), ws_bytes,
        _stream(stream)))


def qk_calib_matrix_rate(mode, iters, out, stream=None):
    """Measurement only: the attention's matrix-core instruction mix on
    near-constant or random operands (see include/qk.h)."""
    _check("qk_calib_matrix_rate", load_library().qk_calib_matrix_rate(int(mode), int(iters),
                                                                        _ptr(out), _stream(stream)))


def qk_calib_read_rate(shape, k, key_format, sink, stream=None):
    """Measurement only: a bare read of the keys a scoring pass reads for
    `shape`, in its grid and ring, computing nothing (see include/qk.h)."""
    _check("qk_calib_read_rate", load_library().qk_calib_read_rate(
        _sh(shape), _ptr(k), int(key_format), _ptr(sink), _stream(stream)))


# ---------------------------------------------------------------------------
# Buffer-owning helpers
# ---------------------------------------------------------------------------
def _ws(shape: Shape, op: str, device) -> tuple:
    n = qk_workspace_bytes(shape, op)
    if n == 0:
        return None, 0
    return torch.zeros(n, dtype=torch.uint8, device=device), n


class Pipeline:
    """Buffers and call order for one chunk: qsel -> kvscore -> topk (or round
    select) -> attention.  Outputs are attributes; every call enqueues on the
    current stream.

    ``fused_gather``: attention reads the selected rows through the index list
    (qk_sparse_attn_indexed) instead of a qk_gather copy followed by
    qk_sparse_attn.

    ``fused_group``: the scoring pass forms the group queries itself
    (qk_kvscore_grouped); otherwise qk_qsel writes them to ``q_group`` and
    qk_kvscore reads them.

    ``score_mode``: "cosine" (the method) or "dot" (the dot-product baseline).
    ``k_e4m3``: the scoring pass reads 8-bit E4M3 keys from ``k8``, which the
    caller fills with ``store_keys_e4m3`` as rows are appended to the cache
    (attention still reads the bf16 keys).  Both variants need ``fused_group``.

    ``shared_rounds`` (round selection): one round choice for all KV heads of
    a sequence (QK_ROUNDS_SHARED).

    ``fused_select``: top-BSA selection (no rounds) with ``fused_group`` goes
    through qk_select, one call for qsel, scoring and top-k; otherwise the
    three calls are made one by one (same results, bit for bit).
    """

    def __init__(self, shape: Shape, device="cuda", n_rounds: int = 0, top_rounds: int = 0,
                 keep_latest: bool = True, fused_gather: bool = True, with_lse: bool = True,
                 fused_group: bool = True, score_mode: str = "cosine", k_e4m3: bool = False,
                 fused_select: bool = True, shared_rounds: bool = False):
        s = self.shape = shape
        if score_mode not in SCORE_MODES:
            raise ValueError("score_mode is 'cosine' or 'dot'")
        if (k_e4m3 or score_mode != "cosine") and not fused_group:
            raise ValueError("the scoring variants form their group queries (fused_group=True)")
        self.score_mode, self.k_e4m3 = score_mode, k_e4m3
        self.device = torch.device(device)
        self.n_rounds, self.top_rounds, self.keep_latest = n_rounds, top_rounds, keep_latest
        self.shared_rounds = shared_rounds
        self.fused_gather, self.fused_group = fused_gather, fused_group
        self.fused_select = (fused_select and fused_group and not n_rounds and s.t_past >= 1
                             and s.bsa >= 1)
        f32, i32 = torch.float32, torch.int32
        dev = self.device
        self.q_idx = torch.empty((s.b, s.nq, s.nq_keep), dtype=i32, device=dev)
        self.sq = torch.empty((s.b, s.nq, s.bcp), dtype=f32, device=dev)
        self.q_group = (None if fused_group else
                        torch.empty((s.b, s.nkv, s.nq_keep, s.d), dtype=f32, device=dev))
        self.s_agg = torch.empty((s.b, s.nkv, max(s.t_past, 1)), dtype=f32, device=dev)
        if n_rounds:
            self.ld_idx = max(s.t_past, 1)
            self.sel_len = torch.empty((s.b, s.nkv), dtype=i32, device=dev)
            self.s_round = torch.empty((s.b, s.nkv, n_rounds), dtype=f32, device=dev)
            self.chosen = torch.empty((s.b, s.nkv, n_rounds), dtype=torch.uint8, device=dev)
        else:
            self.ld_idx = max(s.n_sel, 1)
            self.sel_len = None
            self.s_round = None
            self.chosen = None
        self.idx = torch.empty((s.b, s.nkv, self.ld_idx), dtype=i32, device=dev)
        if not fused_gather:
            self.k_sel = torch.empty((s.b, s.nkv, self.ld_idx, s.d), dtype=s.torch_dtype, device=dev)
            self.v_sel = torch.empty_like(self.k_sel)
        self.out = torch.empty((s.b, s.nq, s.bcp, s.d), dtype=s.torch_dtype, device=dev)
        self.lse = torch.empty((s.b, s.nq, s.bcp), dtype=f32, device=dev) if with_lse else None
        self.ws, self.ws_bytes = _ws(s, "sparse_attn", dev)
        self.topk_ws_bytes = 0 if n_rounds else topk_workspace_bytes(s.b * s.nkv, s.t_past)
        self.select_ws, self.select_ws_bytes = (_ws(s, "select", dev) if self.fused_select
                                                else (None, 0))
        self.topk_ws = (torch.empty(self.topk_ws_bytes, dtype=torch.uint8, device=dev)
                        if self.topk_ws_bytes else None)
        self.k8 = (torch.empty((s.b, s.nkv, s.kv_cap, s.d), dtype=torch.uint8, device=dev)
                   if k_e4m3 else None)

    def store_keys_e4m3(self, k, row0: int = 0, nrows: Optional[int] = None):
        """Convert key rows [row0, row0 + nrows) (default: to the end of the
        cache) into the 8-bit copy read by the scoring pass."""
        nrows = self.shape.kv_cap - row0 if nrows is None else nrows
        qk_keys_to_e4m3(self.shape, k, row0, nrows, self.k8)

    def score(self, q, k):
        """Query sub-selection and key scoring: q_idx, sq and s_agg."""
        s = self.shape
        qk_qsel(s, q, self.q_idx, self.sq, self.q_group)
        if self.k_e4m3 or self.score_mode != "cosine":
            qk_kvscore_variant(s, q, self.q_idx, self.k8 if self.k_e4m3 else k,
                               QK_KEYS_E4M3 if self.k_e4m3 else QK_KEYS_DTYPE, self.score_mode,
                               self.s_agg)
        elif self.fused_group:
            qk_kvscore_grouped(s, q, self.q_idx, k, self.s_agg)
        else:
            qk_kvscore(s, self.q_group, k, self.s_agg)

    def select(self, q, k, round_off=None, append_e4m3=False):
        """append_e4m3 (8-bit keys): also store the chunk's own key rows
        [t_past, t_past + bcp) of k as E4M3 codes in k8, for later chunks (in
        the scoring pass of qk_select, else by qk_keys_to_e4m3 first)."""
        s = self.shape
        append_e4m3 = append_e4m3 and self.k_e4m3
        if self.fused_select:
            qk_select(s, q, self.k8 if self.k_e4m3 else k,
                      QK_KEYS_E4M3 if self.k_e4m3 else QK_KEYS_DTYPE, self.score_mode, self.q_idx,
                      self.sq, self.s_agg, self.idx, self.ld_idx, self.select_ws,
                      self.select_ws_bytes, k_new=k if append_e4m3 else None)
            return
        if append_e4m3:
            self.store_keys_e4m3(k, s.t_past, s.bcp)
        self.score(q, k)
        if self.n_rounds:
            flags = ((QK_ROUNDS_KEEP_LATEST if self.keep_latest else 0)
                     | (QK_ROUNDS_SHARED if self.shared_rounds else 0))
            qk_round_select(s, self.s_agg, self.n_rounds, round_off, self.top_rounds, flags,
                            self.idx, self.ld_idx, self.sel_len, self.s_round, self.chosen)
        else:
            qk_topk(s.b * s.nkv, s.t_past, s.bsa, self.s_agg, self.s_agg.shape[-1], self.idx,
                    self.ld_idx, self.topk_ws, self.topk_ws_bytes)

    def attend(self, q, k, v):
        s = self.shape
        if self.fused_gather:
            qk_sparse_attn_indexed(s, q, k, v, self.idx, self.ld_idx, self.sel_len, self.out,
                                   self.lse, self.ws, self.ws_bytes)
        else:
            qk_gather(s, k, v, self.idx, self.ld_idx, self.sel_len, self.k_sel, self.v_sel)
            qk_sparse_attn(s, q, self.k_sel, self.v_sel, self.ld_idx, self.sel_len, k, v,
                           self.out, self.lse, self.ws, self.ws_bytes)

    def __call__(self, q, k, v, round_off=None):
        self.select(q, k, round_off)
        self.attend(q, k, v)
        return self.out


def shape_of(case_spec, scale: float = 0.0, bsa: Optional[int] = None) -> Shape:
    """Shape for a workload description with the fields b, nq, nkv, d, bcp,
    t_past, kv_cap, nq_keep, bsa and dtype ("bf16"/"f32")."""
    return Shape(case_spec.b, case_spec.nq, case_spec.nkv, case_spec.d, case_spec.bcp,
                 case_spec.t_past, case_spec.kv_cap, case_spec.nq_keep,
                 case_spec.bsa if bsa is None else bsa, scale,
                 QK_BF16 if case_spec.dtype == "bf16" else QK_F32)


load_library()
