#!/usr/bin/env python3
"""Benchmark of the SLA2 sparse-linear attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload video95]

One step is one full forward (router, linear summaries, complement, sparse attention with
the fused linear apply and mix) over the workload's synthetic inputs, which are resident in
HBM before timing starts. Each timed step is preceded by a 512 MB write that evicts L2 and
the 256 MB MALL (--no-cold: no flush); the library records HIP events around every stage on
its stream, and `value` is the median step (first stage start to last stage end). Prints ONE
JSON line with the latency, the roofline of the dominant kernel (the sparse-attention
kernel, from the same events), the dense-attention baselines on the same GPU, the backward
at the forward's selection (sla_backward) beside torch's SDPA backward, and the CPU oracle
baseline. Outside the timed region it also reports the spread (p10 / median / p90) of K warm
back-to-back forwards and what the GPU reaches on a 1 GiB copy and an 8192^3 bf16 GEMM
(achievable peaks next to the published ones).

Other modes:
    --profile            only warm-up + K plain forward calls and a 1 GiB copy (short runs
                         under rocprofv3; the copy calibrates the memory counters)
    --backward-only      one forward for the selection, then W + K sla_backward calls
    --cached             the decode path (sla_forward_cached against a prebuilt summary cache)
    --summarize-pmc FETCH_DIR WRITE_DIR
                         turn two rocprofv3 --pmc CSV outputs (FETCH_SIZE, WRITE_SIZE) into
                         profiles/sparse_attn_<workload>_traffic.json
    --summarize-trace DIR OUT "COMMAND"
                         turn rocprofv3 --kernel-trace --stats CSV output into a short text
                         summary (per-kernel calls and average duration) with its command
    --summarize-mfma DIR OUT "COMMAND"
                         the same for one rocprofv3 --pmc pass over the matrix-core counters
                         (executed MFMA FLOPs and MFMA-busy fraction per kernel)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-linear attn fwd latency (ms) + effective TFLOP/s and % MFMA/HBM peak"
PEAK_BF16 = 2.5e15
PEAK_FP8 = 5.0e15
PEAK_HBM = 8.0e12
SPARSE_SOURCES = ["sparse_linear_hybrid_amd/csrc/sparse.hip", "sparse_linear_hybrid_amd/csrc/common.h"]
TRAFFIC_FILE = "profiles/sparse_attn_{workload}_traffic.json"
COPY_BYTES = 1 << 30
FLUSH_BYTES = 512 << 20      # written before each cold-cache step: more than L2 + MALL


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


# --------------------------------------------------------------------------- algorithmic work
def work(p, fp8=False):
    """Algorithmic FLOPs / bytes of each stage for problem p: FLOPs of the executed MFMA
    work, bytes each stage must move at least (per-unit figures times the units)."""
    BH, d, b = p.batch * p.heads, p.head_dim, 64
    pairs = BH * p.nbq * p.top_k
    qk_flops = pairs * 2 * b * b * d
    pv_flops = pairs * 2 * b * b * d
    apply_flops = BH * p.nbq * 2 * b * d * d
    sparse_flops = qk_flops + pv_flops + apply_flops
    # MFMA-time floor of the sparse kernel: the quantised branch runs P.V at the fp8 rate and
    # Q K^T and the linear apply at the bf16 rate
    if fp8:
        floor_s = (qk_flops + apply_flops) / PEAK_BF16 + pv_flops / PEAK_FP8
    else:
        floor_s = sparse_flops / PEAK_BF16
    elt = 2 if p.dtype == "bf16" else 4
    kv_bytes = (2 * BH * p.n_kv * d * elt                  # read K, V
                + BH * p.nbk * d * d * 2                  # write S_j (bf16)
                + BH * p.nbk * b * d * 2)                 # write f16 V
    # HBM bytes each stage has to move, by what the method needs (SLA2 router, SPLA linear
    # state): the key/value pass reads K and V once and writes S_j (bf16), z_j (fp32) and k~
    # (fp64); its f16 copy of V is the exact branch's operand, reported apart. The router
    # reads Q once, writes and reads its fp64 score rows once and writes the indices. The
    # complement reads every S_j once and writes S_c (bf16) once per query block.
    v16_bytes = BH * p.nbk * b * d * 2
    hbm = {
        "kv_summary": 2 * BH * p.n_kv * d * elt + BH * p.nbk * (d * d * 2 + d * 4 + d * 8),
        "route": BH * p.n_q * d * elt + 2 * BH * p.nbq * p.nbk * 8 + BH * p.nbq * p.top_k * 4,
        "complement": BH * p.nbk * d * d * 2 + BH * p.nbq * (d * d * 2 + d * 4),
    }
    dense_flops = 4 * BH * p.n_q * p.n_kv * d
    return {"pairs": pairs, "sparse_flops": sparse_flops, "kv_summary_bytes": kv_bytes,
            "hbm_bytes": hbm, "v16_bytes": v16_bytes,
            "dense_flops": dense_flops, "sparse_peak": sparse_flops / floor_s}


# --------------------------------------------------------------------------- measured peaks
def spread(vals):
    """p10 / median / p90 of a list of per-step times (ms)."""
    import numpy as np
    v = np.asarray(vals, dtype=np.float64)
    return {"p10": float(np.percentile(v, 10)), "median": float(np.median(v)),
            "p90": float(np.percentile(v, 90))}


def achievable_peaks(torch, dev, sla=None):
    """What this GPU reaches in practice: a 1 GiB device-to-device copy (bytes read plus
    written per second), an 8192^3 bf16 GEMM through torch (dense MFMA work) and, with the
    library, its matrix-instruction throughput loop (independent 32x32x16 bf16 products on
    every SIMD: the rate of the matrix cores at the clock they run under that load)."""
    def timed(fn, n):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_copy = timed(lambda: dst.copy_(src), 5)
    del src, dst
    n = 8192
    a = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    b = torch.randn(n, n, dtype=torch.bfloat16, device=dev)
    t_mm = timed(lambda: torch.mm(a, b), 5)
    del a, b
    out = {"copy_GBps": 2 * COPY_BYTES / t_copy / 1e9,
           "bf16_gemm_TFLOPs": 2 * n ** 3 / t_mm / 1e12,
           "how": "1 GiB device copy (read + write bytes); 8192^3 bf16 torch.mm"}
    if sla is not None:
        out["mfma_bf16_TFLOPs"] = sla.sla_diag_mfma_rate(dev)
        out["how"] += "; sla_diag_mfma_rate (bf16 32x32x16 products, 512 workgroups)"
    return out


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(x, min_seconds=10.0):
    """The oracle, as it stands, on a bounded sample: complete (batch, head) pairs in turn
    until at least ``min_seconds`` of CPU work (or the whole workload) is done; scaled to
    all pairs, in ms."""
    from oracle import sla_oracle as so
    blas = None
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        blas = "; ".join(f"{i.get('internal_api')} {i.get('version')} "
                         f"({i.get('threading_layer', '')}, {i.get('architecture', '')})"
                         for i in info if i.get("user_api") == "blas") or None
    except Exception:   # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    p = x.problem
    pairs = [(b, h) for b in range(p.batch) for h in range(p.heads)]
    done = 0
    t0 = time.perf_counter()
    while done < len(pairs) and (done == 0 or time.perf_counter() - t0 < min_seconds):
        so.forward(x, heads=[pairs[done]])
        done += 1
    dt = time.perf_counter() - t0
    total = len(pairs)
    what = ("the whole workload" if done == total else
            f"{done} of {total} (batch, head) pairs computed in full, scaled to all pairs")
    return {"value": dt * 1e3 * total / done, "unit": "ms", "cores": int(threads),
            "kind": "oracle", "sample": f"{what} ({dt:.1f} s)", "cpu_model": cpu_model,
            "host_cpus": len(os.sched_getaffinity(0)), "blas": blas}


# --------------------------------------------------------------------------- traffic summary
def read_traffic(workload):
    path = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != sources_sha(SPARSE_SOURCES):
        return None          # the kernel changed since the counters were taken
    return rec.get("traffic_bytes_per_launch")


def short_name(name):
    """Kernel name without the return type, anonymous namespace and parameter list."""
    return name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").strip()


def summarize_pmc(fetch_dir, write_dir, workload):
    """profiles/sparse_attn_<workload>_traffic.json from two rocprofv3 --pmc runs."""
    def rows(d):
        out = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(fn) as f:
                out += list(csv.DictReader(f))
        return out

    def per_kernel(rs, counter):
        acc = {}
        for r in rs:
            if r.get("Counter_Name") != counter:
                continue
            name = r.get("Kernel_Name", "")
            acc.setdefault(name, []).append(float(r["Counter_Value"]))
        return acc

    def pick(acc, needle, how="mean"):
        vals = [x for k, v in acc.items() if needle in k for x in v]
        if not vals:
            return None
        return max(vals) if how == "max" else sum(vals) / len(vals)

    f = per_kernel(rows(fetch_dir), "FETCH_SIZE")
    w = per_kernel(rows(write_dir), "WRITE_SIZE")
    kname = "sparse_attn_fp8_kernel" if workload.endswith("_fp8") else "sparse_attn_kernel"
    sp_f, sp_w = pick(f, kname), pick(w, kname)
    # the calibration copy is the largest copy dispatch of the run (1 GiB device to device)
    cp_f = pick(f, "copy", "max")
    cp_w = pick(w, "copy", "max")
    sf = (cp_f * 1024) / COPY_BYTES if cp_f else None       # KiB counted per real byte read
    sw = (cp_w * 1024) / COPY_BYTES if cp_w else None
    rec = {
        "workload": workload, "kernel": kname,
        "source_sha256": sources_sha(SPARSE_SOURCES),
        "fetch_kib_per_launch": sp_f, "write_kib_per_launch": sp_w,
        "copy_fetch_kib": cp_f, "copy_write_kib": cp_w, "copy_bytes": COPY_BYTES,
        "fetch_scale": sf, "write_scale": sw,
        "traffic_bytes_per_launch": (sp_f * 1024 / sf + sp_w * 1024 / sw)
        if (sp_f and sp_w and sf and sw) else None,
        "per_kernel_fetch_kib": {short_name(k): sum(v) / len(v) for k, v in f.items()},
        "per_kernel_write_kib": {short_name(k): sum(v) / len(v) for k, v in w.items()},
    }
    path = os.path.join(ROOT, TRAFFIC_FILE.format(workload=workload))
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec))


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4          # MI355X: 256 compute units with 4 SIMDs each
XCDS = 8


def summarize_mfma(d, out, command):
    """Matrix-core utilisation per kernel from one rocprofv3 --pmc pass over MFMA_COUNTERS:
    executed MFMA FLOPs (each MOPS unit is 512 FLOPs), the MFMA-busy fraction of the SIMD
    cycles (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs) and, where the dispatch
    timestamps are present, the executed rate."""
    rows = []
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for r in rows:
        key = (r.get("Kernel_Name", ""), r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        rec = per.setdefault(key, {})
        rec[r["Counter_Name"]] = rec.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            rec["_ns"] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
    kern = {}
    for (name, _), rec in per.items():
        kern.setdefault(short_name(name), []).append(rec)
    lines = ["# rocprofv3 matrix-core counters (one --pmc pass)", f"# command: {command}",
             "# mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) "
             "(GRBM_GUI_ACTIVE comes summed over the 8 XCDs); clock_GHz = GRBM_GUI_ACTIVE / 8 / "
             "duration; exec_TF = (MOPS_BF16 + MOPS_F16 + MOPS_F8) x 512 / duration", "#",
             f"{'kernel':58s} {'calls':>5s} {'GFLOP_exec':>11s} {'mfma_busy':>9s} "
             f"{'exec_TF':>8s} {'clock_GHz':>9s} {'mfma_insts':>11s} {'valu_insts':>11s}"]
    for name, recs in sorted(kern.items(), key=lambda kv: -sum(r.get("SQ_VALU_MFMA_BUSY_CYCLES", 0)
                                                                for r in kv[1])):
        n = len(recs)
        mean = lambda c: sum(r.get(c, 0.0) for r in recs) / n          # noqa: E731
        flops = 512 * (mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") + mean("SQ_INSTS_VALU_MFMA_MOPS_F16")
                       + mean("SQ_INSTS_VALU_MFMA_MOPS_F8"))
        gui = mean("GRBM_GUI_ACTIVE") / XCDS
        busy = mean("SQ_VALU_MFMA_BUSY_CYCLES") / (gui * SIMDS) if gui else float("nan")
        ns = [r["_ns"] for r in recs if "_ns" in r]
        tf = flops / (sum(ns) / len(ns)) / 1e3 if ns else float("nan")
        ghz = gui / (sum(ns) / len(ns)) if ns else float("nan")
        lines.append(f"{name[:58]:58s} {n:5d} {flops / 1e9:11.2f} {busy:9.3f} {tf:8.1f} "
                     f"{ghz:9.2f} {mean('SQ_INSTS_MFMA'):11.0f} {mean('SQ_INSTS_VALU'):11.0f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(d, out, command, timed=None, bench_log=None):
    """Short text summary of rocprofv3 --kernel-trace --stats CSV output: per kernel the
    calls and average duration. timed = "W,K": also the average over the dispatches W ..
    W + K - 1 of each kernel, which for a profiled `bench.py --warmup W --steps K` run are the
    calls of its timed region (bench.py's HIP-event average of the same run covers exactly
    those); bench_log: the run's output, whose JSON line is quoted for comparison."""
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(files[0])))
    per = {}
    tr = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if tr:
        for r in csv.DictReader(open(tr[0])):
            per.setdefault(short_name(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    w0, k0 = (int(x) for x in timed.split(",")) if timed else (0, 0)
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", "#",
             f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'total_%':>8s}"
             + (f" {'timed_avg_us':>12s}" if timed else "")]
    for r in rows:
        name = r.get("Name", "")
        short = short_name(name)[:70]
        line = (f"{short:70s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                f"{float(r['Percentage']):8.2f}")
        if timed:
            ds = per.get(short_name(name), [])[w0:w0 + k0]
            line += f" {sum(ds) / len(ds):12.2f}" if len(ds) == k0 else f" {'':12s}"
        lines.append(line)
    if timed:
        lines.append(f"# timed_avg_us: mean duration of dispatches {w0} .. {w0 + k0 - 1} of each "
                     "kernel (the timed steps of the profiled run)")
    if bench_log and os.path.exists(bench_log):
        for l in open(bench_log):
            if l.startswith("{") and '"roofline"' in l:
                rec = json.loads(l)
                rf = rec["roofline"]
                lines.append(f"# the run's own line: value {rec['value']:.4f} ms/step, "
                             f"{rf['kernel']} avg_launch_ms {rf['avg_launch_ms']:.4f} "
                             f"(HIP events), roofline frac {rf['frac']:.4f}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# --------------------------------------------------------------------------- decode path
def bench_cached(args, sla, x, q, k, v, pq, pk, al, out):
    """sla_forward_cached against a cache built before timing (the key/value summary lives
    with the KV cache); one step = one cached forward."""
    import numpy as np
    import torch
    from workloads import sha256_of
    p = x.problem
    dev = q.device
    kprob = sla.make_problem(k, k, 0)
    cache = torch.empty(sla.kv_cache_size(kprob), dtype=torch.uint8, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sla.sla_kv_cache_update(k, v, pk, cache)                   # warm-up build
    torch.cuda.synchronize()
    a.record()
    sla.sla_kv_cache_update(k, v, pk, cache)
    b.record()
    torch.cuda.synchronize()
    build_ms = a.elapsed_time(b)
    ws = torch.empty(sla.cached_workspace_size(sla.make_problem(q, k, p.top_k)),
                     dtype=torch.uint8, device=dev)

    def fwd():
        sla.sla_forward_cached(q, k, v, pq, al, p.top_k, cache, return_idx=False, workspace=ws,
                               out=out)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    if args.profile:
        for _ in range(args.steps):
            fwd()
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": args.workload, "cached": True, "steps": args.steps}))
        return 0
    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record()
        fwd()
        e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / K
    call_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    BH, d = p.batch * p.heads, p.head_dim
    # bytes the method has to move: the selected K/V tiles, Q, O, the cached k~ (router)
    # and S_tot, z_tot
    sel_bytes = BH * p.nbq * p.top_k * 2 * 64 * d * 2
    alg_bytes = (sel_bytes + BH * p.n_q * d * (2 + 4) + p.nbk * BH * d * 8 + BH * (d * d + d) * 4)
    achieved = alg_bytes / (call_ms * 1e-3)
    dense = None
    if not args.no_dense:
        f = torch.nn.functional.scaled_dot_product_attention
        for _ in range(2):
            f(q, k, v)
        torch.cuda.synchronize()
        a.record()
        for _ in range(3):
            f(q, k, v)
        b.record()
        torch.cuda.synchronize()
        sdpa = a.elapsed_time(b) / 3
        dense = {"sdpa_bf16_ms": sdpa, "speedup_vs_sdpa": sdpa / ms}
    line = {
        "metric": METRIC, "value": ms, "unit": "ms", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": p.name, "path": "sla_forward_cached", "batch": p.batch,
                   "heads": p.heads, "n_q": p.n_q, "n_kv": p.n_kv, "head_dim": d,
                   "block": p.block, "top_k": p.top_k, "sparsity": round(p.sparsity, 4),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": PEAK_HBM / 1e9,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM, "traffic": None,
                     "kernel": "sla_forward_cached (whole call: route, decode, combine)",
                     "bytes_per_call": alg_bytes, "avg_call_ms": call_ms},
        "cpu_baseline": None,
        "kv_cache_build_ms": build_ms,
        "dense": dense,
        "inputs_sha256": sha256_of(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha),
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))
    return 0


# --------------------------------------------------------------------------- main
def bench_backward(args, sla, torch, p, q, k, v, pq, pk, al, ws, out, skip_dense=False):
    """Outside the timed forward region: sla_backward at the forward's selection for a
    random upstream gradient (fp32), K timed calls after the warm-up ones, and torch's SDPA
    backward (bf16) on the same shapes for comparison. Sparse-branch FLOPs follow the
    FlashAttention convention (2.5 x the forward's 4 b^2 d per routed pair: recomputed
    scores, dP, dV, dK, dQ)."""
    _, idx = sla.sla_forward(q, k, v, pq, pk, al, p.top_k, workspace=ws, out=out)
    gen = torch.Generator(device=q.device).manual_seed(11)
    dout = torch.randn(q.shape, device=q.device, dtype=torch.float32, generator=gen)
    need = sla.sla_backward_workspace_size(sla.make_problem(q, k, p.top_k))
    bws = torch.empty(need, dtype=torch.uint8, device=q.device)
    for _ in range(max(1, args.warmup)):
        sla.sla_backward(q, k, v, al, dout, idx, workspace=bws)
    torch.cuda.synchronize()
    K = args.steps
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(K):
        sla.sla_backward(q, k, v, al, dout, idx, workspace=bws)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / K
    pairs = p.batch * p.heads * p.nbq * p.top_k
    flops = 2.5 * 4 * p.block * p.block * p.head_dim * pairs
    res = {"ms": ms, "workspace_bytes": need, "sparse_flops": flops,
           "sparse_TFLOPs_effective": flops / (ms * 1e-3) / 1e12}
    del bws
    if not skip_dense:
        try:
            f = torch.nn.functional.scaled_dot_product_attention
            qd, kd, vd = (t.detach().clone().requires_grad_(True) for t in (q, k, v))
            g16 = dout.to(torch.bfloat16)
            for _ in range(2):
                f(qd, kd, vd).backward(g16)
            torch.cuda.synchronize()
            n = 3
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record()
            for _ in range(n):
                f(qd, kd, vd)
            e[1].record()
            for _ in range(n):
                f(qd, kd, vd).backward(g16)
            e[2].record()
            torch.cuda.synchronize()
            fwd_ms = e[0].elapsed_time(e[1]) / n
            res["sdpa_bf16_fwd_bwd_ms"] = e[1].elapsed_time(e[2]) / n
            res["sdpa_bf16_bwd_ms"] = res["sdpa_bf16_fwd_bwd_ms"] - fwd_ms
            res["speedup_vs_sdpa_bwd"] = res["sdpa_bf16_bwd_ms"] / ms
            del qd, kd, vd
        except Exception as ex:  # noqa: BLE001
            res["sdpa_error"] = str(ex)[:200]
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="video95")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache pass (512 MB written before each forward)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured copy and GEMM peaks")
    ap.add_argument("--cached", action="store_true",
                    help="time sla_forward_cached against a prebuilt key/value summary cache "
                         "(the decode path); the cache build is timed separately")
    ap.add_argument("--router", choices=("learnable", "taylor"), default="learnable",
                    help="taylor: time sla_forward_taylor (training-free second-order router)")
    ap.add_argument("--pisa", action="store_true",
                    help="time sla_forward_pisa (exact routed blocks + Taylor tail, one "
                         "normalisation) instead of sla_forward")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward leg (sla_backward at the forward's selection)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only the backward leg (one forward for the selection, then "
                         "W + K sla_backward calls); prints its own JSON line")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-trace", nargs=3, metavar=("DIR", "OUT", "COMMAND"))
    ap.add_argument("--timed", default=None, metavar="W,K",
                    help="with --summarize-trace: also average dispatches W .. W+K-1")
    ap.add_argument("--bench-log", default=None,
                    help="with --summarize-trace: the profiled run's output (its JSON line)")
    ap.add_argument("--summarize-mfma", nargs=3, metavar=("DIR", "OUT", "COMMAND"))
    args = ap.parse_args()

    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, timed=args.timed, bench_log=args.bench_log)
        return 0
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (every "
              "(batch, head) is independent, so heads would shard across GPUs without "
              "communication). Run with --gpus 1.", file=sys.stderr)
        return 2

    import ctypes
    import numpy as np
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import sparse_linear_hybrid_amd as sla
    from workloads import make_inputs, sha256_of

    fp8 = args.workload.endswith("_fp8")
    dev = torch.device("cuda:0")
    x = make_inputs(args.workload)
    p = x.problem

    def t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v, pq, pk, al = (t(a) for a in (x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha))
    prob = sla.make_problem(q, k, p.top_k)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    if args.cached:
        return bench_cached(args, sla, x, q, k, v, pq, pk, al, out)
    taylor = args.router == "taylor"
    pisa = args.pisa
    if int(taylor) + int(pisa) + int(fp8) > 1:
        print("--router taylor, --pisa and the fp8 workload are separate paths", file=sys.stderr)
        return 2
    variant = (sla.VARIANT_FP8 if fp8 else sla.VARIANT_PISA if pisa else
               sla.VARIANT_TAYLOR if taylor else sla.VARIANT_FORWARD)
    ws = torch.empty(sla.workspace_size(prob, variant), dtype=torch.uint8, device=dev)
    if args.backward_only:
        if fp8 or taylor or pisa or p.dtype != "bf16":
            print("the backward takes the bf16 forward's selection", file=sys.stderr)
            return 2
        res = bench_backward(args, sla, torch, p, q, k, v, pq, pk, al, ws, out,
                             skip_dense=args.no_dense)
        print(json.dumps({"backward": res, "workload": p.name, "steps": args.steps,
                          "warmup": args.warmup}))
        return 0

    def fwd():
        if pisa:
            sla.sla_forward_pisa(q, k, v, pq, pk, p.top_k, return_idx=False, workspace=ws, out=out)
        elif taylor:
            sla.sla_forward_taylor(q, k, v, al, p.top_k, return_idx=False, workspace=ws, out=out)
        elif fp8:
            sla.sla_forward_fp8(q, k, v, pq, pk, al, p.top_k, return_idx=False, workspace=ws,
                                out=out)
        else:
            sla.sla_forward(q, k, v, pq, pk, al, p.top_k, return_idx=False, workspace=ws, out=out)

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    if args.profile:
        for _ in range(args.steps):
            fwd()
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile_run": args.workload, "steps": args.steps}))
        return 0

    # ---------------------------------------------------------------- timed region
    # K forwards, each preceded by a 512 MB write that evicts L2 and the 256 MB MALL (so the
    # inputs come from HBM); every stage of every forward is bracketed by HIP events on the
    # library's stream, and a step's time runs from its first stage's start to its last
    # stage's end (the flush is outside it). value = the median step.
    K = args.steps
    nst = len(sla.STAGES)
    flush = None if args.no_cold else torch.empty(FLUSH_BYTES // 4, dtype=torch.float32,
                                                   device=dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)] for _ in range(K)]
    for row in evs:
        for e in row:
            e.record()
    torch.cuda.synchronize()
    handles = [(ctypes.c_void_p * (2 * nst))(*[e.cuda_event for e in row]) for row in evs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        if flush is not None:
            flush.fill_(float(s))
        sla.sla_forward_profiled(q, k, v, pq, pk, al, p.top_k, handles[s], fp8=fp8,
                                 workspace=ws, out=out, taylor=taylor, pisa=pisa)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / K
    stage_ms = {name: float(np.mean([evs[s][2 * i].elapsed_time(evs[s][2 * i + 1])
                                     for s in range(K)]))
                for i, name in enumerate(sla.STAGES)}
    steps = [evs[s][0].elapsed_time(evs[s][2 * nst - 1]) for s in range(K)]
    ms = float(np.median(steps))
    cold_steps = steps if flush is not None else None

    # Warm caches (outside the timed region): K back-to-back forwards, no flush.
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(K)]
    for s in range(K):
        marks[s][0].record()
        fwd()
        marks[s][1].record()
    torch.cuda.synchronize()
    warm_steps = [a.elapsed_time(b) for a, b in marks]
    del flush
    peaks = None if args.no_peaks else achievable_peaks(torch, dev, sla)

    w = work(p, fp8)
    sparse_s = stage_ms["sparse"] * 1e-3
    peak = w["sparse_peak"]
    achieved = w["sparse_flops"] / sparse_s
    roofline = {"bound": "mfma", "achieved": achieved / 1e12, "peak": peak / 1e12,
                "unit": "TFLOP/s", "frac": achieved / peak, "traffic": read_traffic(args.workload),
                "kernel": "sparse_attn_fp8_kernel" if fp8 else "sparse_attn_kernel",
                "flops_per_launch": w["sparse_flops"],
                "avg_launch_ms": stage_ms["sparse"]}
    if peaks and not fp8:
        roofline["achievable_peak"] = peaks["bf16_gemm_TFLOPs"]
        roofline["frac_of_achievable"] = achieved / 1e12 / peaks["bf16_gemm_TFLOPs"]
        roofline["mfma_rate"] = peaks["mfma_bf16_TFLOPs"]
        roofline["frac_of_mfma_rate"] = achieved / 1e12 / peaks["mfma_bf16_TFLOPs"]
    # algorithmic HBM rate of the memory-bound stages (the key/value pass, the router, the
    # complement), against the 8 TB/s peak; the f16 V copy is shown apart
    hbm = {}
    # sla_forward's cache path (bf16, at most 8 query blocks per head over at least 256 key
    # blocks): the key/value stage is the cache build, which writes only k~ per key block,
    # and there is no complement stage
    cache_path = (p.dtype == "bf16" and p.nbq <= 8 and p.nbk >= 256
                  and not (fp8 or taylor or pisa))
    if cache_path:
        BH, d = p.batch * p.heads, p.head_dim
        w["hbm_bytes"] = {"kv_summary": 2 * BH * p.n_kv * d * 2 + BH * p.nbk * d * 8,
                          "route": w["hbm_bytes"]["route"]}
        w["v16_bytes"] = 0
    if fp8:
        # the quantised path's key/value pass writes K8 (E4M3 values held as bf16) and the V8
        # tiles instead of the f16 copy of V; the "with_v16" figures below count those
        BH, d = p.batch * p.heads, p.head_dim
        k8v8 = BH * p.nbk * 64 * d * 3
        w["kv_summary_bytes"] += k8v8 - w["v16_bytes"]
        w["v16_bytes"] = k8v8
    for stg, nbytes in w["hbm_bytes"].items():
        t_s = stage_ms[stg] * 1e-3
        if t_s > 0 and not (pisa and stg == "complement"):
            hbm[stg] = {"bytes": nbytes, "GBps": nbytes / t_s / 1e9, "frac": nbytes / t_s / PEAK_HBM}
    if "kv_summary" in hbm:
        hbm["kv_summary"]["with_v16_copy_frac"] = ((w["hbm_bytes"]["kv_summary"] + w["v16_bytes"])
                                                   / (stage_ms["kv_summary"] * 1e-3) / PEAK_HBM)
    kernels = {
        "stage_ms": stage_ms,
        "hbm": hbm,
        # the key/value pass including its f16 copy of V (the exact branch's operand; the
        # method's own bytes are in hbm["kv_summary"])
        "kv_summary_with_v16_GBps": w["kv_summary_bytes"] / (stage_ms["kv_summary"] * 1e-3) / 1e9,
        "step_ms_warm": spread(warm_steps),
        "step_ms_cold": spread(cold_steps) if cold_steps else None,
        "wall_ms_per_step": wall_ms,
        "timing": ("value = median over the timed steps of the HIP-event time from the first "
                   "stage's start to the last stage's end"
                   + (", each step after a 512 MB cache-flush write" if cold_steps else
                      ", warm caches (--no-cold)")),
        "achievable": peaks,
    }
    if peaks:
        kernels["kv_summary_with_v16_frac_of_copy"] = (kernels["kv_summary_with_v16_GBps"]
                                                       / peaks["copy_GBps"])
    kernels["kv_summary_operand_copies"] = ("K8 (bf16-held) and V8 tiles" if fp8 else
                                            "none" if cache_path else "f16 copy of V")
    if pisa:
        # tail kernel (timed as the complement stage): Q K_bar^T and P Vsum over the
        # unrouted centroids, 4 d FLOP per (query row, centroid)
        tail_flops = p.batch * p.heads * p.n_q * (p.nbk - p.top_k) * 4 * p.head_dim
        kernels["tail_TFLOPs"] = tail_flops / (stage_ms["complement"] * 1e-3) / 1e12

    # ---------------------------------------------------------------- dense baselines
    dense = None
    if not args.no_dense:
        dense = {}
        try:
            f = torch.nn.functional.scaled_dot_product_attention
            if p.dtype == "bf16":
                for _ in range(2):
                    f(q, k, v)
                torch.cuda.synchronize()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                n = 5
                a.record()
                for _ in range(n):
                    f(q, k, v)
                b.record()
                torch.cuda.synchronize()
                dense["sdpa_bf16_ms"] = a.elapsed_time(b) / n
        except Exception as ex:  # noqa: BLE001
            dense["sdpa_error"] = str(ex)[:200]
        try:
            all_k = p.nbk
            ones = torch.ones_like(al)
            ws2 = torch.empty(sla.workspace_size(sla.make_problem(q, k, all_k), False),
                              dtype=torch.uint8, device=dev)
            sla.sla_forward(q, k, v, pq, pk, ones, all_k, return_idx=False, workspace=ws2, out=out)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            n = 3
            a.record()
            for _ in range(n):
                sla.sla_forward(q, k, v, pq, pk, ones, all_k, return_idx=False, workspace=ws2,
                                out=out)
            b.record()
            torch.cuda.synchronize()
            dense["own_all_blocks_ms"] = a.elapsed_time(b) / n
            del ws2
        except Exception as ex:  # noqa: BLE001
            dense["own_error"] = str(ex)[:200]
        best = min([v_ for k_, v_ in dense.items() if k_.endswith("_ms")] or [float("nan")])
        dense["best_dense_ms"] = best
        dense["speedup_vs_best_dense"] = best / ms
        # the dense baselines run back to back (warm caches): the same against the warm
        # forwards
        dense["speedup_vs_best_dense_warm"] = best / float(np.median(warm_steps))

    backward = None
    if not (args.no_backward or fp8 or taylor or pisa or p.dtype != "bf16"):
        backward = bench_backward(args, sla, torch, p, q, k, v, pq, pk, al, ws, out,
                                  skip_dense=args.no_dense)

    cpu = None if args.no_cpu else cpu_baseline(x)

    line = {
        "metric": METRIC, "value": ms, "unit": "ms", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": ("fp8-e4m3/bf16" if fp8 else "bf16" if p.dtype == "bf16"
                  else "f32 (bf16 three-term split products)"),
        "data": "synthetic",
        "config": {"workload": p.name, "batch": p.batch, "heads": p.heads, "n_q": p.n_q,
                   "n_kv": p.n_kv, "head_dim": p.head_dim, "block": p.block,
                   "top_k": p.top_k, "sparsity": round(p.sparsity, 4),
                   "grid": "x".join(map(str, p.grid)) if p.grid else None,
                   "router": args.router, "path": "sla_forward_pisa" if pisa else None,
                   "parallelism": "single GPU"},
        # dense-equivalent: what full attention on the same shape would compute, over this
        # forward's time (it exceeds the MFMA peak whenever the speedup over dense does);
        # executed: the sparse kernel's FLOPs (Q K^T, P.V, linear apply) plus the complement's
        # masked product, over the same time
        "effective_tflops": w["dense_flops"] / (ms * 1e-3) / 1e12,
        "effective_tflops_kind": "dense-equivalent FLOPs / forward time",
        "executed_tflops": (w["sparse_flops"] + 2 * p.batch * p.heads * p.nbq * p.nbk
                            * p.head_dim ** 2) / (ms * 1e-3) / 1e12,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense": dense,
        "kernels": kernels,
        "backward": backward,
        "inputs_sha256": sha256_of(x.q, x.k, x.v, x.proj_q, x.proj_k, x.alpha),
        "gpu": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
