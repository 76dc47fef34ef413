"""Benchmark: one chunk of query-oriented sparse KV selection + attention over
the selected keys, on one MI355X.

A step is the whole hot path over one chunk whose inputs are resident in HBM:
    qk_select (qk_qsel -> qk_kvscore_grouped -> qk_topk in one call) -> qk_sparse_attn_indexed
(the gather of the selected rows is fused into the attention's loads).
Steps rotate over several copies of the inputs (more bytes than the 256 MB
Infinity Cache), so each step streams its K and V from HBM.

Prints one JSON line.  `value` is the chunk latency in ms (the metric's unit;
lower is better).  `roofline` covers the kernel that dominates the step;
`roofline_scoring` covers the scoring pass (the metric's GB/s half).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import sparse_kv_selection_amd as qk  # noqa: E402
import workloads as W  # noqa: E402

METRIC = "selected-KV attention chunk ms @T=32K + scoring HBM GB/s (% of peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores

# HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by
# the plain-copy calibration (2 x FETCH_SIZE + 1 x WRITE_SIZE, KiB -> bytes),
# keyed by (workload, stage) and valid only for the kernel source they were
# taken on (first 16 hex digits of the SHA-256 of the kernel's source file
# followed by the shared device header): once either changes, the figure no
# longer describes the kernel and `traffic` is null.
MEASURED_TRAFFIC = {
    ("llama3b_32k", "kvscore"): ("kvscore.hip", "72bf584754d139ff", 70642998),
    ("llama3b_32k", "attention"): ("attention.hip", "7b63cf47e9fab0a3", 72463144),
    ("long_128k", "kvscore"): ("kvscore.hip", "72bf584754d139ff", 278068841),
    ("long_128k", "attention"): ("attention.hip", "7b63cf47e9fab0a3", 123568384),
    ("decode_64x16k", "kvscore"): ("kvscore.hip", "72bf584754d139ff", 2182091634),
    ("decode_64x16k", "attention"): ("attention.hip", "7b63cf47e9fab0a3", 542617118),
    ("rounds_64k", "kvscore"): ("kvscore.hip", "72bf584754d139ff", 138900976),
    ("rounds_64k", "attention"): ("attention.hip", "7b63cf47e9fab0a3", 95261832),
    ("long_128k_d256", "kvscore"): ("kvscore.hip", "72bf584754d139ff", 550305161),
    ("long_128k_d256", "attention"): ("attention.hip", "7b63cf47e9fab0a3", 173053928),
}


def measured_traffic(workload: str, stage: str):
    import hashlib
    entry = MEASURED_TRAFFIC.get((workload, stage))
    if entry is None:
        return None
    fname, digest, nbytes = entry
    csrc = os.path.join(ROOT, "sparse_kv_selection_amd", "csrc")
    h = hashlib.sha256()
    for name in (fname, "qk_device.h"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    current = h.hexdigest()[:16]
    return nbytes if current == digest else None


def _describe(s) -> str:
    return (f"b={s.b} nq={s.nq} nkv={s.nkv} d={s.d} T={s.t_past} bcp={s.bcp} "
            f"NQ={s.nq_keep} BSA={s.bsa}" + (f" rounds={s.n_rounds} top={s.top_rounds}+latest"
                                             if s.n_rounds else ""))


def algorithmic(spec, n_sel_per_bj, key_bytes=None):
    """Per-step algorithmic work.  n_sel_per_bj: mean selected past keys per
    (sequence, KV head); key_bytes: bytes per key element the scoring pass reads
    (default: the dtype's; 1 for E4M3 keys)."""
    esz = 2 if spec.dtype == "bf16" else 4
    kesz = esz if key_bytes is None else key_bytes
    bnkv = spec.b * spec.nkv
    # scoring: every past key read once (d*kesz) + one fp32 score written, plus the kept
    # query rows and their positions (the group queries are formed inside the pass)
    score_bytes = (bnkv * spec.t_past * (spec.d * kesz + 4)
                   + spec.b * spec.nq * spec.nq_keep * (spec.d * esz + 4))
    score_flops = 2.0 * bnkv * spec.nq_keep * spec.d * spec.t_past
    # attention: 4*d flops per (query row, attended key); causal chunk counts its half
    rows = spec.b * spec.nq * spec.bcp
    causal_pairs = spec.b * spec.nq * spec.bcp * (spec.bcp + 1) / 2
    attn_flops = 4.0 * spec.d * (rows * n_sel_per_bj + causal_pairs)
    attn_bytes = (bnkv * n_sel_per_bj * 2 * spec.d * esz + bnkv * spec.bcp * 2 * spec.d * esz
                  + 2 * rows * spec.d * esz)
    dense_flops = 4.0 * spec.d * (rows * spec.t_past + causal_pairs)
    return dict(score_bytes=score_bytes, score_flops=score_flops, attn_flops=attn_flops,
                attn_bytes=attn_bytes, dense_flops=dense_flops)


def pipe_splits(shape) -> int:
    """Key splits of the attention launch (a combine kernel follows when > 1):
    the workspace is non-empty exactly when the keys are split."""
    return 2 if qk.qk_workspace_bytes(shape, "sparse_attn") > 0 else 1


def cpu_baseline(spec, seed, budget_s: float, score: str = "cosine", k_e4m3: bool = False):
    """The fp64 oracle, as it stands, on this host: the full chunk if it fits
    the time budget, else a row sample of the attention (selection is always
    complete) scaled to one chunk."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    case = W.make_case(spec, seed)
    qn = case["q"].float().numpy().astype(np.float64)
    kn = case["k"].float().numpy().astype(np.float64)
    vn = case["v"].float().numpy().astype(np.float64)
    off = case["round_off"].numpy() if case["round_off"] is not None else None
    t0 = time.perf_counter()
    sel = oracle.pipeline(qn, kn, vn, spec.t_past, spec.nq_keep, spec.bsa, round_off=off,
                          top_rounds=spec.top_rounds, with_attention=False, score=score,
                          k_e4m3=k_e4m3)
    t_sel = time.perf_counter() - t0
    # time attention on growing row samples until the budget is used, then scale
    rows_total = spec.bcp
    n = max(1, min(rows_total, 8))
    t_att, done = 0.0, 0
    rng = np.random.default_rng(seed)
    while True:
        rows = np.sort(rng.choice(rows_total, n, replace=False))
        t1 = time.perf_counter()
        oracle.attention(qn, kn, vn, spec.t_past, sel["key_sets"], rows=rows)
        dt = time.perf_counter() - t1
        t_att, done = dt, n
        if n == rows_total or t_sel + dt * 4 > budget_s:
            break
        n = min(rows_total, n * 4)
    measured = t_sel + t_att
    if done == rows_total:
        # the whole chunk fits: repeat whole chunks until ~half the budget is spent
        reps, total = 1, measured
        while total < 0.5 * budget_s:
            t1 = time.perf_counter()
            oracle.pipeline(qn, kn, vn, spec.t_past, spec.nq_keep, spec.bsa, round_off=off,
                            top_rounds=spec.top_rounds, score=score, k_e4m3=k_e4m3)
            total += time.perf_counter() - t1
            reps += 1
        est, measured = total / reps, total
        sample = (f"{reps} whole chunks (selection over all {spec.b * spec.nkv} KV heads, "
                  f"T={spec.t_past}, + attention of all {rows_total} rows x {spec.nq} heads)")
    else:
        est = t_sel + t_att * rows_total / done
        sample = (f"full selection (all {spec.b * spec.nkv} KV heads, T={spec.t_past}) + attention "
                  f"of {done}/{rows_total} chunk rows x all {spec.nq} heads, scaled to the whole chunk")
    return {"value": est * 1e3, "unit": "ms per chunk", "cores": int(threads), "kind": "oracle",
            "sample": sample, "cpu_model": _cpu_model(),
            "host_cpus": len(os.sched_getaffinity(0)), "blas_threads": int(threads),
            "threading": ("numpy fp64: the matrix products run on the BLAS thread pool "
                          "(blas_threads); the per-row sorts and the per-head loops on one thread"),
            "selection_ms": t_sel * 1e3, "measured_s": round(measured, 2)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


CALIB_MODES = {  # qk_calib_matrix_rate modes (include/qk.h)
    "constant_registers": 0, "random_registers": 1, "constant_lds": 2, "random_lds": 3,
    "constant_lds_softmax": 6, "random_lds_softmax": 7}


def matrix_ceiling(dev, iters: int = 2048) -> dict:
    """TFLOP/s the attention's matrix-core instruction mix sustains on this GPU
    (qk_calib_matrix_rate): near-constant against random operands, from
    registers, from LDS, and with the softmax vector work.  Measured with
    events around each call on the current stream, after one warm-up call."""
    out = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    flops = 256.0 * 8 * iters * 32 * 32768
    res = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, mode in CALIB_MODES.items():
        qk.qk_calib_matrix_rate(mode, iters // 4, out)
        e0.record()
        qk.qk_calib_matrix_rate(mode, iters, out)
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    return res


def bench_offload(spec, args, dev):
    """Round workloads through a layer stack: resident (every layer's cache on
    the GPU) against round offload (the layers above the watershed held per
    round in pinned host memory, chosen rounds copied in after selection)."""
    from sparse_kv_selection_amd import driver
    if spec.n_rounds == 0:
        sys.exit("--offload-layers needs a round workload (rounds_64k)")
    L, w, T, n = args.offload_layers, args.watershed, spec.t_past, spec.bcp
    off = W.round_offsets(T, spec.n_rounds, args.seed)
    shared = args.shared_rounds
    stack = driver.RoundOffloadStack(L, w, off, spec.b, spec.nkv, spec.d, n, device=dev,
                                     shared_rounds=shared)
    caches, qs, krows, vrows = [], [], [], []
    for layer in range(L):
        case = W.make_case(spec, args.seed + 7919 * layer, device=dev)
        stack.load_history(layer, case["k"], case["v"])
        c = driver.KVCache(spec.b, spec.nkv, T + n, spec.d, device=dev)
        c.k[:, :, :T].copy_(case["k"][:, :, :T])
        c.v[:, :, :T].copy_(case["v"][:, :, :T])
        c.advance(T)
        caches.append(c)
        qs.append(case["q"])
        krows.append(case["k"][:, :, T:T + n].contiguous())
        vrows.append(case["v"][:, :, T:T + n].contiguous())
    off_dev = torch.tensor(off, dtype=torch.int32, device=dev)
    plan = T // 4

    def resident():
        for c in caches:
            c.length = T
        return driver.layer_stack_step(qs, caches, krows, vrows, spec.nq_keep, plan, w,
                                       round_off=off_dev, top_rounds=spec.top_rounds,
                                       shared_rounds=shared)

    def offload():
        return stack.step(qs, krows, vrows, spec.nq_keep, spec.top_rounds, plan)

    def timed(fn, steps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    steps = max(3, min(args.steps, 20))
    ms_res = timed(resident, steps)
    ms_off = timed(offload, steps)
    outs_o, _ = offload()
    outs_r, _ = resident()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(outs_o, outs_r))
    copy_ms = sum(s.elapsed_time(e) for s, e in stack.copy_events)
    h2d = stack.last_h2d_bytes
    result = {
        "metric": "round-offload layer stack chunk ms (host-held upper layers) + H2D GB/s",
        "value": round(ms_off, 4), "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": 2,
        "ms_per_step": round(ms_off, 4), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": f"{spec.name}: {_describe(spec)}", "layers": L, "watershed": w,
                   "round_choice": "shared by the KV heads" if shared else "per KV head",
                   "rounds_copied": len(stack.last_rounds)},
        "resident_stack_ms": round(ms_res, 4),
        "h2d_bytes_per_chunk": h2d,
        "h2d_copy_ms": round(copy_ms, 4),
        "h2d_gbps": round(h2d / (copy_ms * 1e-3) / 1e9, 2) if copy_ms > 0 else None,
        # GPU KV: the lower layers' caches plus two staging caches holding the
        # chosen rounds (and the chunk) of the last step
        "staged_past_positions": stack.last_staged,
        "gpu_kv_bytes": stack.staged_kv_bytes(), "resident_kv_bytes": stack.resident_kv_bytes(),
        "gpu_kv_saved_frac": round(1 - stack.staged_kv_bytes() / stack.resident_kv_bytes(), 4),
        "outputs_equal_resident": same,
        "timing": "wall clock over whole steps (the step waits on the host for the watershed's "
                  "selection before it schedules the copies)",
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 200 chunks take about 17 ms at llama3b_32k; 50-chunk windows varied by a few
    # per cent from run to run (clock ramp), 200 and 400 agree
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama3b_32k", choices=sorted(W.CONFIGS))
    ap.add_argument("--seed", type=int, default=1002)
    ap.add_argument("--copies", type=int, default=0, help="input copies rotated over (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--gathered", action="store_true", help="qk_gather + qk_sparse_attn instead of the fused path")
    ap.add_argument("--score", default="cosine", choices=["cosine", "dot"],
                    help="scoring: the method's cosine score or the dot-product baseline")
    ap.add_argument("--keys", default="dtype", choices=["dtype", "e4m3"],
                    help="keys the scoring pass reads: the cache dtype or an 8-bit E4M3 copy")
    ap.add_argument("--offload-layers", type=int, default=0,
                    help="round workloads: a stack of this many layers whose layers above the "
                         "watershed keep their KV per round in pinned host memory")
    ap.add_argument("--watershed", type=int, default=1)
    ap.add_argument("--shared-rounds", action="store_true",
                    help="with --offload-layers: one round choice for all KV heads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (counter calibration) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(KV heads and sequences are independent: each GPU would take its own with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # a copy of known size: 256 MiB read + 256 MiB written per dispatch
        n = 256 * 1024 * 1024 // 4
        src = torch.rand(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "dispatches": 5}), flush=True)
        return

    spec = W.spec(args.workload)
    if args.offload_layers:
        return bench_offload(spec, args, dev)
    rounds = spec.n_rounds > 0
    shape = qk.shape_of(spec, bsa=spec.t_past // 4 if rounds else spec.bsa)
    one_copy = sum(spec.b * h * r * spec.d * (2 if spec.dtype == "bf16" else 4)
                   for h, r in ((spec.nq, spec.bcp), (spec.nkv, spec.kv_cap), (spec.nkv, spec.kv_cap)))
    copies = args.copies or max(2, min(16, int(np.ceil(1.0e9 / one_copy))))
    inputs = []
    for c in range(copies):
        case = W.make_case(spec, args.seed + 7919 * c, device=dev)
        inputs.append(case)
    e4m3 = args.keys == "e4m3"
    variant = e4m3 or args.score != "cosine"
    pipe = qk.Pipeline(shape, device=dev, n_rounds=spec.n_rounds, top_rounds=spec.top_rounds,
                       fused_gather=not args.gathered, score_mode=args.score, k_e4m3=e4m3)
    if e4m3:
        # every copy's cache also held as E4M3 (written once, as the rows were
        # appended); the timed step converts the chunk's own rows, the append
        for c in inputs:
            pipe.k8 = torch.empty(c["k"].shape, dtype=torch.uint8, device=dev)
            pipe.store_keys_e4m3(c["k"])
            c["k8"] = pipe.k8
    torch.cuda.synchronize()

    def step(i):
        c = inputs[i % copies]
        if e4m3:
            # the chunk's own key rows become E4M3 codes too (the append):
            # inside qk_select's scoring pass
            pipe.k8 = c["k8"]
        pipe.select(c["q"], c["k"], c["round_off"], append_e4m3=e4m3)
        pipe.attend(c["q"], c["k"], c["v"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # Per-stage kernel time: each stage is launched `reps` times back to back
    # over the rotating input copies, between two events on the current stream
    # (the launches are enqueued ahead, so host gaps between calls do not
    # count).  A stage reads the previous stage's outputs as they stand, which
    # are valid inputs of the same shape.
    stages = ((["store_keys"] if e4m3 else []) + ["qsel", "kvscore", "select", "attention"]
              + (["select_one_call"] if pipe.fused_select else []))

    read_sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def run_stage(name, c):
        if name == "read_keys":
            # measurement only: the scoring pass's key loads with nothing
            # computed (its floor over these bytes on this GPU)
            qk.qk_calib_read_rate(shape, c["k8"] if e4m3 else c["k"],
                                  qk.QK_KEYS_E4M3 if e4m3 else qk.QK_KEYS_DTYPE, read_sink)
        elif name == "store_keys":
            qk.qk_keys_to_e4m3(shape, c["k"], spec.t_past, spec.bcp, c["k8"])
        elif name == "qsel":
            qk.qk_qsel(shape, c["q"], pipe.q_idx, pipe.sq, pipe.q_group)
        elif name == "kvscore" and variant:
            qk.qk_kvscore_variant(shape, c["q"], pipe.q_idx, c["k8"] if e4m3 else c["k"],
                                  qk.QK_KEYS_E4M3 if e4m3 else qk.QK_KEYS_DTYPE, args.score,
                                  pipe.s_agg)
        elif name == "kvscore":
            qk.qk_kvscore_grouped(shape, c["q"], pipe.q_idx, c["k"], pipe.s_agg)
        elif name == "select_one_call":
            # qk_select: query selection, scoring (with the histogram the
            # top-k starts from) and top-k in one call, as the timed step runs
            if e4m3:
                pipe.k8 = c["k8"]
            pipe.select(c["q"], c["k"], append_e4m3=e4m3)
        elif name == "select":
            if rounds:
                qk.qk_round_select(shape, pipe.s_agg, spec.n_rounds, c["round_off"],
                                   spec.top_rounds, True, pipe.idx, pipe.ld_idx, pipe.sel_len,
                                   pipe.s_round)
            else:
                qk.qk_topk(shape.b * shape.nkv, shape.t_past, shape.bsa, pipe.s_agg,
                           shape.t_past, pipe.idx, pipe.ld_idx, pipe.topk_ws, pipe.topk_ws_bytes)
        else:
            pipe.attend(c["q"], c["k"], c["v"])

    reps = max(10, args.steps)
    stage_ms = {}
    read_floor = spec.dtype == "bf16"
    for sname in stages + (["read_keys"] if read_floor else []):
        for i in range(2):
            run_stage(sname, inputs[i % copies])
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            run_stage(sname, inputs[i % copies])
        e1.record()
        torch.cuda.synchronize()
        stage_ms[sname] = e0.elapsed_time(e1) / reps

    read_ms = stage_ms.pop("read_keys", None)
    n_sel = float(pipe.sel_len.float().mean()) if rounds else float(shape.n_sel)
    work = algorithmic(spec, n_sel, key_bytes=1 if e4m3 else None)
    score_gbs = work["score_bytes"] / (stage_ms["kvscore"] * 1e-3) / 1e9
    attn_tflops = work["attn_flops"] / (stage_ms["attention"] * 1e-3) / 1e12
    score_kernel = ("qk_kvscore_variant (kvscore_bf16_kernel, "
                    + ("E4M3 keys, " if e4m3 else "") + f"{args.score} score)" if variant
                    else "qk_kvscore_grouped (kvscore_bf16_kernel)")
    roof_score = {"kernel": score_kernel, "bound": "hbm",
                  "achieved": round(score_gbs, 1),
                  "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(score_gbs / HBM_PEAK_GBS, 4),
                  # counters were taken on the default path only
                  "traffic": None if variant else measured_traffic(spec.name, "kvscore"),
                  "algorithmic_bytes": work["score_bytes"],
                  "ms": round(stage_ms["kvscore"], 5)}
    if read_ms:
        # beside the published peak, the floor this GPU sets for these bytes:
        # a bare read of the same keys in the pass's grid and ring
        key_bytes = spec.b * spec.nkv * spec.t_past * spec.d * (1 if e4m3 else 2)
        roof_score["ceiling"] = {"bare_read_ms": round(read_ms, 5),
                                 "bare_read_gbps": round(key_bytes / (read_ms * 1e-3) / 1e9, 1),
                                 "frac": round(read_ms / stage_ms["kvscore"], 4)}
    # the attention plan's choice: the eight-wave ping-pong kernel at d = 128
    # when a KV head has more than 128 query rows
    pp = spec.d == 128 and (spec.nq // spec.nkv) * spec.bcp > 128
    attn_kernels = ("qk_sparse_attn_indexed (" + ("attn_pp_kernel" if pp else "attn_bf16_kernel")
                    + (" + attn_combine_kernel)" if pipe_splits(shape) > 1 else ")"))
    if spec.bcp == 1:
        attn_gbs = work["attn_bytes"] / (stage_ms["attention"] * 1e-3) / 1e9
        roof_attn = {"kernel": attn_kernels, "bound": "hbm", "achieved": round(attn_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(spec.name, "attention"),
                     "algorithmic_bytes": work["attn_bytes"],
                     "ms": round(stage_ms["attention"], 5)}
    else:
        roof_attn = {"kernel": attn_kernels, "bound": "mfma", "achieved": round(attn_tflops, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic(spec.name, "attention"),
                     "algorithmic_flops": work["attn_flops"], "ms": round(stage_ms["attention"], 5)}
    if spec.bcp > 1:
        # the published peak stays the denominator; beside it, what the same
        # instruction mix reaches on this GPU with random operands (power-bound)
        ceil = matrix_ceiling(dev)
        roof_attn["ceiling"] = {"tflops_random_operands": ceil["random_lds_softmax"],
                                "frac": round(attn_tflops / ceil["random_lds_softmax"], 4),
                                "calibration_tflops": ceil}
    dominant = roof_attn if stage_ms["attention"] >= stage_ms["kvscore"] else roof_score

    result = {
        "metric": METRIC, "value": round(ms, 5), "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if spec.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{spec.name}: {_describe(spec)}", "input_copies": copies,
                   "gather": "gathered" if args.gathered else "fused into attention",
                   "score": args.score, "scoring_keys": "e4m3" if e4m3 else spec.dtype},
        "roofline": dominant, "roofline_scoring": roof_score, "roofline_attention": roof_attn,
        "scoring_gbps": round(score_gbs, 1), "scoring_frac_of_peak": round(score_gbs / HBM_PEAK_GBS, 4),
        "keys_scored_per_s": spec.b * spec.nkv * spec.t_past / (stage_ms["kvscore"] * 1e-3),
        "stages_ms": {k: round(v, 5) for k, v in stage_ms.items()},
        # the one-call selection less its query and scoring stages: what the
        # top-k costs after a scoring pass that fills its histogram
        "topk_in_one_call_ms": (round(stage_ms["select_one_call"] - stage_ms["qsel"]
                                      - stage_ms["kvscore"], 5)
                                if "select_one_call" in stage_ms else None),
        "chunks_per_s": round(1e3 / ms, 1),
    }

    if not args.no_dense:
        dout = torch.empty_like(inputs[0]["q"])
        nws = qk.qk_workspace_bytes(shape, "dense_attn")
        dws = torch.zeros(max(nws, 1), dtype=torch.uint8, device=dev)
        for i in range(3):
            c = inputs[i % copies]
            qk.qk_dense_attn(shape, c["q"], c["k"], c["v"], dout, None, dws, nws)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nd = max(5, args.steps // 5)
        d0.record()
        for i in range(nd):
            c = inputs[i % copies]
            qk.qk_dense_attn(shape, c["q"], c["k"], c["v"], dout, None, dws, nws)
        d1.record()
        torch.cuda.synchronize()
        dms = d0.elapsed_time(d1) / nd
        result["dense_attention_ms"] = round(dms, 5)
        result["dense_attention_tflops"] = round(work["dense_flops"] / (dms * 1e-3) / 1e12, 1)
        result["chunk_vs_dense_attention"] = round(dms / ms, 3)
        result["dense_over_sparse_attention"] = round(dms / stage_ms["attention"], 3)
        if spec.bcp == 1:
            # memory-bound decode: dense moves K and V, the method K once plus
            # the selected K and V rows, so the chunk can beat dense attention
            # by at most 2 / (1 + 2 BSA / T)
            f = shape.n_sel / spec.t_past
            result["decode_ceiling_vs_dense"] = round(2.0 / (1.0 + 2.0 * f), 3)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(spec, args.seed, args.cpu_budget, args.score, e4m3)
        result["cpu_baseline"]["value"] = round(result["cpu_baseline"]["value"], 2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
