"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before launching anything.

No GPU is used: every call below fails validation, which happens on the host
before any HIP call.  Pointers are fake but aligned; should validation ever
let one through, the call would reach the HIP runtime, so these tests are
skipped where a device is present.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qk.h")

import sparse_kv_selection_amd as qk  # noqa: E402

OK, NULL, SHAPE, DTYPE, ALIGN, WS, UNSUP, HIP = range(8)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qk_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = _declared()
    assert "qk_qsel" in names and "qk_sparse_attn_indexed" in names
    out = subprocess.run(["nm", "-D", "--defined-only", qk.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (qk_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert sorted(qk.EXPORTED) == names
    lib = ctypes.CDLL(qk.LIB_PATH)
    for n in names:
        getattr(lib, n)


def test_version_and_strings():
    assert qk.qk_abi_version() == 1
    for code in range(8):
        assert qk.qk_status_string(code)
    assert qk.qk_status_string(99) == "unknown status"


nogpu = pytest.mark.skipif(torch.cuda.is_available(), reason="fake device pointers; host checks only")
FAKE = 1 << 20  # aligned, never dereferenced


def _shape(**kw):
    base = dict(b=1, nq=8, nkv=2, d=128, bcp=64, t_past=1000, kv_cap=1064, nq_keep=16, bsa=100,
                scale=0.0, dtype=qk.QK_BF16)
    base.update(kw)
    return qk.Shape(**base).c()


def _p(x=FAKE):
    return ctypes.c_void_p(x) if x else None


@nogpu
@pytest.mark.parametrize("kw,code", [
    (dict(nq=7), SHAPE), (dict(nkv=0), SHAPE), (dict(b=0), SHAPE), (dict(d=96), UNSUP),
    (dict(bcp=0), SHAPE), (dict(bcp=5000), SHAPE), (dict(kv_cap=1063), SHAPE),
    (dict(t_past=-1), SHAPE), (dict(dtype=7), DTYPE), (dict(scale=-1.0), SHAPE),
    (dict(nq_keep=0), SHAPE), (dict(nq_keep=65), SHAPE), (dict(nq_keep=300, bcp=512), SHAPE),
])
def test_qsel_rejects(kw, code):
    lib = qk.load_library()
    s = _shape(**kw)
    assert lib.qk_qsel(ctypes.byref(s), _p(), _p(), None, _p(), None) == code


@nogpu
def test_null_and_alignment():
    lib = qk.load_library()
    s = _shape()
    assert lib.qk_qsel(None, _p(), _p(), None, _p(), None) == NULL
    assert lib.qk_qsel(ctypes.byref(s), None, _p(), None, _p(), None) == NULL
    assert lib.qk_qsel(ctypes.byref(s), _p(FAKE + 8), _p(), None, _p(), None) == ALIGN
    assert lib.qk_kvscore(ctypes.byref(s), _p(), _p(FAKE + 2), _p(), None) == ALIGN
    assert lib.qk_kvscore(ctypes.byref(s), _p(), None, _p(), None) == NULL
    assert lib.qk_kvscore(ctypes.byref(s), None, _p(), _p(), None) == NULL
    assert lib.qk_kvscore_grouped(ctypes.byref(s), None, _p(), _p(), _p(), None) == NULL
    assert lib.qk_kvscore_grouped(ctypes.byref(s), _p(), None, _p(), _p(), None) == NULL
    assert lib.qk_kvscore_grouped(ctypes.byref(s), _p(), _p(), _p(), None, None) == NULL
    assert lib.qk_kvscore_grouped(ctypes.byref(s), _p(FAKE + 4), _p(), _p(), _p(), None) == ALIGN
    assert lib.qk_kvscore_grouped(ctypes.byref(s), _p(), _p(FAKE + 2), _p(), _p(), None) == ALIGN


@nogpu
def test_scoring_variants_reject():
    lib = qk.load_library()
    s = _shape()
    var = lib.qk_kvscore_variant
    assert var(ctypes.byref(s), None, _p(), _p(), 0, 0, _p(), None) == NULL
    assert var(ctypes.byref(s), _p(), None, _p(), 0, 0, _p(), None) == NULL
    assert var(ctypes.byref(s), _p(), _p(), _p(), 2, 0, _p(), None) == UNSUP    # key format
    assert var(ctypes.byref(s), _p(), _p(), _p(), 0, 2, _p(), None) == UNSUP    # score mode
    assert var(ctypes.byref(s), _p(), _p(), _p(FAKE + 8), 1, 0, _p(), None) == ALIGN
    f32 = _shape(dtype=qk.QK_F32)
    assert var(ctypes.byref(f32), _p(), _p(), _p(), qk.QK_KEYS_E4M3, 0, _p(), None) == DTYPE
    assert var(None, _p(), _p(), _p(), 0, 0, _p(), None) == NULL
    conv = lib.qk_keys_to_e4m3
    assert conv(ctypes.byref(s), None, 0, 10, _p(), None) == NULL
    assert conv(ctypes.byref(s), _p(), 0, 10, None, None) == NULL
    assert conv(ctypes.byref(s), _p(), -1, 10, _p(), None) == SHAPE
    assert conv(ctypes.byref(s), _p(), 0, -1, _p(), None) == SHAPE
    assert conv(ctypes.byref(s), _p(), 1000, 65, _p(), None) == SHAPE       # past kv_cap = 1064
    assert conv(ctypes.byref(s), _p(FAKE + 2), 0, 10, _p(), None) == ALIGN
    assert conv(ctypes.byref(s), _p(), 0, 10, _p(FAKE + 8), None) == ALIGN
    assert conv(ctypes.byref(_shape(d=96)), _p(), 0, 10, _p(), None) == UNSUP
    assert conv(ctypes.byref(s), _p(), 1064, 0, _p(), None) == OK           # nothing to do


@nogpu
def test_read_calibration_rejects():
    lib = qk.load_library()
    s = _shape()
    f = lib.qk_calib_read_rate
    assert f(None, _p(), 0, _p(), None) == NULL
    assert f(ctypes.byref(s), None, 0, _p(), None) == NULL
    assert f(ctypes.byref(s), _p(), 0, None, None) == NULL
    assert f(ctypes.byref(s), _p(), 2, _p(), None) == UNSUP                    # key format
    assert f(ctypes.byref(_shape(dtype=qk.QK_F32)), _p(), 0, _p(), None) == DTYPE
    assert f(ctypes.byref(_shape(nq_keep=0)), _p(), 0, _p(), None) == SHAPE
    assert f(ctypes.byref(_shape(nq_keep=33, d=256)), _p(), 0, _p(), None) == UNSUP
    assert f(ctypes.byref(s), _p(FAKE + 8), 0, _p(), None) == ALIGN
    assert f(ctypes.byref(s), _p(), 1, _p(FAKE + 4), None) == ALIGN
    assert f(ctypes.byref(_shape(d=96)), _p(), 0, _p(), None) == UNSUP


@nogpu
def test_kvscore_limits():
    lib = qk.load_library()
    assert lib.qk_kvscore(ctypes.byref(_shape(nq_keep=65, bcp=128, kv_cap=2000)), _p(), _p(), _p(), None) == UNSUP
    assert lib.qk_kvscore(ctypes.byref(_shape(nq_keep=33, d=256)), _p(), _p(), _p(), None) == UNSUP
    grouped = lib.qk_kvscore_grouped
    assert grouped(ctypes.byref(_shape(nq_keep=33, d=256)), _p(), _p(), _p(), _p(), None) == UNSUP
    # f32: NQ * (d + G) * 4 bytes of LDS at most 64 KiB
    f32 = dict(dtype=qk.QK_F32, d=256, bcp=128, kv_cap=2000)
    assert grouped(ctypes.byref(_shape(nq_keep=64, nq=64, nkv=2, **f32)), _p(), _p(), _p(), _p(),
                   None) == UNSUP


@nogpu
def test_topk_rejects():
    lib = qk.load_library()
    assert lib.qk_topk(4, 100, 0, _p(), 100, _p(), 10, None, 0, None) == SHAPE
    assert lib.qk_topk(4, 100, 10, _p(), 99, _p(), 10, None, 0, None) == SHAPE
    assert lib.qk_topk(4, 100, 10, _p(), 100, _p(), 9, None, 0, None) == SHAPE
    assert lib.qk_topk(-1, 100, 10, _p(), 100, _p(), 10, None, 0, None) == SHAPE
    assert lib.qk_topk(4, 100, 10, None, 100, _p(), 10, None, 0, None) == NULL
    assert lib.qk_topk(4, 100, 10, _p(FAKE + 2), 100, _p(), 10, None, 0, None) == ALIGN
    # few long rows are split over workgroups and need scratch
    need = qk.topk_workspace_bytes(8, 32768)
    assert lib.qk_topk(8, 32768, 10, _p(), 32768, _p(), 10, None, need, None) == NULL
    assert lib.qk_topk(8, 32768, 10, _p(), 32768, _p(), 10, _p(), need - 1, None) == WS
    assert lib.qk_topk(8, 32768, 10, _p(), 32768, _p(), 10, _p(FAKE + 4), need, None) == ALIGN
    assert lib.qk_topk(1, 8388609, 10, _p(), 8388609, _p(), 10, _p(), 1 << 40, None) == UNSUP
    # nothing to do is not an error
    assert lib.qk_topk(0, 100, 10, None, 100, None, 10, None, 0, None) == OK
    assert lib.qk_topk(3, 0, 10, None, 0, None, 0, None, 0, None) == OK


@nogpu
def test_round_select_rejects():
    lib = qk.load_library()
    s = _shape()
    f = lib.qk_round_select
    assert f(ctypes.byref(s), _p(), 0, _p(), 1, 1, _p(), 1000, _p(), None, None, None) == SHAPE
    assert f(ctypes.byref(s), _p(), 8, _p(), 8, 1, _p(), 1000, _p(), None, None, None) == SHAPE
    assert f(ctypes.byref(s), _p(), 8, _p(), 0, 1, _p(), 1000, _p(), None, None, None) == SHAPE
    assert f(ctypes.byref(s), _p(), 8, _p(), 2, 1, _p(), 999, _p(), None, None, None) == SHAPE
    assert f(ctypes.byref(s), _p(), 8, None, 2, 1, _p(), 1000, _p(), None, None, None) == NULL
    # the head-shared choice needs s_round (the heads' round scores meet there);
    # unknown flag bits are refused
    assert f(ctypes.byref(s), _p(), 8, _p(), 2, qk.QK_ROUNDS_KEEP_LATEST | qk.QK_ROUNDS_SHARED,
             _p(), 1000, _p(), None, None, None) == NULL
    assert f(ctypes.byref(s), _p(), 8, _p(), 2, 4, _p(), 1000, _p(), None, None, None) == UNSUP
    text = open(HEADER).read()
    assert "#define QK_ROUNDS_KEEP_LATEST 1" in text and "#define QK_ROUNDS_SHARED 2" in text


@nogpu
def test_attention_rejects():
    lib = qk.load_library()
    s = _shape()
    need = lib.qk_workspace_bytes(ctypes.byref(s), qk.OPS["sparse_attn"])
    f = lib.qk_sparse_attn_indexed
    assert f(ctypes.byref(s), _p(), _p(), _p(), _p(), 99, None, _p(), None, _p(), 1 << 30, None) == SHAPE
    assert f(ctypes.byref(s), _p(), _p(), _p(), None, 100, None, _p(), None, _p(), 1 << 30, None) == NULL
    if need:
        assert f(ctypes.byref(s), _p(), _p(), _p(), _p(), 100, None, _p(), None, _p(), need - 1, None) == WS
        assert f(ctypes.byref(s), _p(), _p(), _p(), _p(), 100, None, _p(), None, None, need, None) == NULL
    g = lib.qk_sparse_attn
    assert g(ctypes.byref(s), _p(), None, _p(), 100, None, _p(), _p(), _p(), None, _p(), 1 << 30, None) == NULL
    assert g(ctypes.byref(s), _p(), _p(), _p(), 50, None, _p(), _p(), _p(), None, _p(), 1 << 30, None) == SHAPE
    s32 = _shape(dtype=qk.QK_F32, d=256)
    assert lib.qk_dense_attn(ctypes.byref(s32), _p(), _p(), _p(), _p(), None, _p(), 1 << 30, None) == UNSUP
    assert lib.qk_gather(ctypes.byref(s), _p(), _p(), _p(), 99, None, _p(), _p(), None) == SHAPE


def test_workspace_sizes():
    # split-key partials: per split and row, d fp16 values + (lse, scale) fp32;
    # 0 when one split suffices
    s = qk.Shape(1, 24, 8, 128, 256, 32768, 33024, 32, 8192)
    n = qk.qk_workspace_bytes(s, "sparse_attn")
    rows = 1 * 24 * 256
    assert n > 0 and n % (rows * (128 * 2 + 8)) == 0
    assert qk.qk_workspace_bytes(s, "qsel") == 0
    assert qk.qk_workspace_bytes(qk.Shape(1, 4, 2, 64, 64, 1024, 1088, 32, 256, dtype=qk.QK_F32),
                                 "sparse_attn") == 0
    bad = qk.Shape(1, 7, 2, 128, 256, 32768, 33024, 32, 8192)
    assert qk.qk_workspace_bytes(bad, "sparse_attn") == 0
    # top-k of a split row (tiles of 4096 scores up to 64K, else 8192): a
    # 2048-bin histogram per tile (ints; one per row when the scoring pass
    # fills them), (B, need, count) per row, two counts per tile, and a
    # (key, position) slot for every score; each part 16-byte aligned
    def split_ws(rows, n, row_hist=False):
        tile = 4096 if n <= 65536 else 8192
        t = rows * -(-n // tile)
        up = lambda x: -(-x // 16) * 16
        return (up((rows if row_hist else t) * 2048 * 4) + up(rows * 16) + up(t * 8)
                + t * tile * 8)
    assert qk.topk_workspace_bytes(8, 32768) == split_ws(8, 32768)
    assert qk.topk_workspace_bytes(8, 131072) == split_ws(8, 131072)
    assert qk.topk_workspace_bytes(1, 300001) == split_ws(1, 300001)
    assert qk.topk_workspace_bytes(512, 16384) == 0                    # one workgroup per row
    assert qk.topk_workspace_bytes(512, 16388) == split_ws(512, 16388)
    assert qk.topk_workspace_bytes(8, 4096) == 0
    # the whole selection: what the top-k needs (bf16 rows it splits take one
    # histogram per row, filled by the scoring pass), then for bf16 the kept
    # query rows (b, nq, NQ, d) at a 256-byte boundary
    up256 = lambda x: -(-x // 256) * 256
    sel = qk.Shape(1, 24, 8, 128, 256, 32768, 33024, 32, 8192)
    assert qk.qk_workspace_bytes(sel, "select") == (up256(split_ws(8, 32768, row_hist=True))
                                                    + 24 * 32 * 128 * 2)
    sel32 = qk.Shape(1, 24, 8, 128, 256, 32768, 33024, 32, 8192, dtype=qk.QK_F32)
    assert qk.qk_workspace_bytes(sel32, "select") == split_ws(8, 32768)
    dec = qk.Shape(64, 32, 8, 128, 1, 16384, 16385, 1, 2048)
    assert qk.qk_workspace_bytes(dec, "select") == 64 * 32 * 1 * 128 * 2   # one workgroup per row
    assert qk.qk_workspace_bytes(qk.Shape(1, 24, 8, 128, 256, 32768, 33024, 32, 40000),
                                 "select") == 24 * 32 * 128 * 2        # every key kept


def test_noalloc_scratch_covers_every_plan():
    """The fixed scratch array of qk_sparse_attn_indexed_noalloc holds the
    key-split partials of every shape the attention plan produces (host-side
    sizes only), and the binding's constant is the header's."""
    text = open(HEADER).read()
    m = re.search(r"#define QK_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == qk.QK_NOALLOC_SCRATCH_BYTES
    worst = 0
    for d in (64, 128, 256):
        for nkv in (1, 2, 8):
            for G in (1, 3, 8, 16):
                for bcp in (1, 7, 64, 200, 256, 512, 1000, 4096):
                    for b in (1, 3, 64):
                        for t in (100, 5000, 32768, 131072, 500000):
                            s = qk.Shape(b, nkv * G, nkv, d, bcp, t, t + bcp, 1, t, 0.0, qk.QK_BF16)
                            worst = max(worst, qk.qk_workspace_bytes(s, "sparse_attn"))
    assert 0 < worst <= qk.QK_NOALLOC_SCRATCH_BYTES, worst


def test_noalloc_status():
    assert "fixed array" in qk.qk_status_string(8)
    lib = ctypes.CDLL(qk.LIB_PATH)
    fn = lib.qk_sparse_attn_indexed_noalloc
    fn.restype = ctypes.c_int32
    assert fn(None, None, None, None, None, 0, None, None, None, None) == NULL
