"""Host-side logic of bench.py (no GPU): the algorithmic work the roofline
figures divide by, the rule that ties stored traffic counters to the kernel
source they were taken on, and the one-GPU guard."""
import os
import subprocess
import sys

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_llama3b_32k():
    spec = W.spec("llama3b_32k")
    w = bench.algorithmic(spec, spec.bsa)
    nkv, t, d, nq, nk, bcp, bsa = 8, 32768, 128, 24, 32, 256, 8192
    # scoring: every past key once (d bf16 values) and one fp32 score per key
    # and KV head, plus the kept query rows and their positions
    assert w["score_bytes"] == nkv * t * (d * 2 + 4) + nq * nk * (d * 2 + 4)
    # attention: 4 d flops per (query row, attended key); every row sees the
    # BSA selected keys and the chunk's keys up to its own position
    rows = nq * bcp
    causal = nq * bcp * (bcp + 1) / 2
    assert w["attn_flops"] == 4 * d * (rows * bsa + causal)
    assert w["dense_flops"] == 4 * d * (rows * t + causal)
    # the figures the roofline fractions are quoted against
    assert round(w["score_bytes"] / 1e6, 1) == 68.4
    assert round(w["attn_flops"] / 1e9, 2) == 26.17


def test_algorithmic_e4m3_keys_read_one_byte_per_element():
    spec = W.spec("llama3b_32k")
    w = bench.algorithmic(spec, spec.bsa, key_bytes=1)
    assert w["score_bytes"] == 8 * 32768 * (128 + 4) + 24 * 32 * (128 * 2 + 4)


def test_measured_traffic_only_for_the_source_it_was_taken_on(monkeypatch):
    key = ("llama3b_32k", "kvscore")
    fname, digest, nbytes = bench.MEASURED_TRAFFIC[key]
    # either still valid (the stored figure) or the kernel changed since (None)
    assert bench.measured_traffic(*key) in (nbytes, None)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key, (fname, "0" * 16, nbytes))
    assert bench.measured_traffic(*key) is None
    assert bench.measured_traffic("llama3b_32k", "no_such_stage") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 2, r.stderr[-500:]
    assert "one GPU" in r.stderr
