#!/usr/bin/env python3
"""Benchmark of the lightning-indexer backward on one MI355X.

One step = one full backward call (row kernel, dK range kernel, slab sum on
the default route) over the anchor workload B=1, H=64, D=128, S_q=8192,
S_k=4096, topk=1024 (2% of slots padded), inputs resident in HBM before
timing starts.  Prints ONE JSON line.  Throughput counts 6*H*D*topk FLOP per
query (three GEMMs of 2*H*D per slot: score recompute, dQ, dK), the count used
for the pages' own anchor figure.  Every kernel of the call is also timed with
HIP events on the kernels' stream (through the library's stage hook); the
roofline object describes the kernel that takes longest.
"""
import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer-bwd µs + TFLOP/s (frac of MFMA peak) at S_q=8192,S_k=4096,topk=1024"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
COMPUTE_DTYPE = "bf16"      # MFMA operands bf16, fp32 accumulation and outputs


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--workload", default="anchor")
    ap.add_argument("--topk", type=int, default=0,
                    help="override the sparse workload's topk (a topk sweep at its other shapes)")
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--atomic-dk", action="store_true",
                    help="the single-pass route with fp32 atomic dK (not bitwise reproducible)")
    ap.add_argument("--dk-route", choices=("auto", "key_ranges", "slot_rows"), default="auto",
                    help="deterministic dK route: by selection density (auto), or forced")
    ap.add_argument("--bf16-out", action="store_true",
                    help="d_q, d_w and d_k written as bf16 (the fp32 results rounded)")
    ap.add_argument("--forward", action="store_true",
                    help="time the step before the backward instead: indexer scores over every "
                         "key plus the top-k selection, at the workload's shapes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=18.0,
                    help="target wall time of the oracle sample (three timed runs)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before timing, copy a buffer of this many MiB once (a kernel of "
                         "known traffic, read by the HBM counter runs to scale them)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.forward:
        forward_main(args)
        return
    import numpy as np
    import torch

    import dsa_lightning_indexer_bwd_amd as ibwd
    from synth import WORKLOADS, make_inputs

    ibwd.library()  # fails loudly when the HIP library is missing
    wl = WORKLOADS[args.workload]
    if args.topk:
        if wl.dense or args.topk > wl.S_k:
            print("--topk applies to sparse workloads, at most S_k", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, topk=args.topk)
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    x = make_inputs(wl, device=dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k = bf16(x.q), bf16(x.k)
    w = torch.from_numpy(x.w).to(dev)
    I = torch.from_numpy(x.index_score).to(dev)
    p = torch.from_numpy(x.attn_score).to(dev)
    ids = None if x.ids is None else torch.from_numpy(x.ids).to(dev)
    B, S_q, H, D = x.q.shape
    S_k = x.k.shape[1]
    odt = torch.bfloat16 if args.bf16_out else torch.float32
    dq = torch.empty((B, S_q, H, D), dtype=odt, device=dev)
    dw = torch.empty((B, S_q, H), dtype=odt, device=dev)
    dk = torch.empty((B, S_k, D), dtype=odt, device=dev)
    if args.atomic_dk and (args.deterministic or args.bf16_out):
        print("--atomic-dk excludes --deterministic and --bf16-out", file=sys.stderr)
        sys.exit(2)
    flags = (ibwd.IBWD_FLAG_DETERMINISTIC if args.deterministic else 0) | \
        (ibwd.IBWD_FLAG_ATOMIC_DK if args.atomic_dk else 0) | \
        (ibwd.IBWD_FLAG_BF16_OUT if args.bf16_out else 0) | \
        ({"auto": 0, "key_ranges": ibwd.IBWD_FLAG_DK_KEY_RANGES,
          "slot_rows": ibwd.IBWD_FLAG_DK_SLOT_ROWS}[args.dk_route] if ids is not None else 0)
    ws_bytes = ibwd.indexer_bwd_workspace_bytes(wl.dense, B, S_q, S_k, H, D, wl.topk, flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.Stream(device=dev)

    def step():
        if ids is None:
            ibwd.indexer_bwd_dense(q, k, w, I, p, dq, dw, dk, q_offset=wl.q_offset,
                                   deterministic=args.deterministic, atomic_dk=args.atomic_dk,
                                   bf16_out=args.bf16_out, workspace=ws, stream=stream)
        else:
            ibwd.indexer_bwd_sparse(q, k, w, ids, I, p, dq, dw, dk,
                                    deterministic=args.deterministic, atomic_dk=args.atomic_dk,
                                    bf16_out=args.bf16_out, dk_route=args.dk_route, workspace=ws,
                                    stream=stream)

    if args.calibration_copy_mib:
        n = args.calibration_copy_mib << 18  # fp32 elements
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    clk_before = read_gfx_clock()
    print("bench: clock under load", file=sys.stderr, flush=True)
    clk_load = clocks_under_load(step, torch.cuda.synchronize)
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    # HIP events recorded on the stream the kernels run on: one pair around
    # every call, and one after every kernel of the call (the library's stage
    # hook runs on the host right after each kernel is enqueued)
    stage_events = []

    def hook(stage, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        stage_events[-1].append((stage, name, e))

    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    ibwd.set_stage_hook(hook)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for e0, e1 in calls:
        e0.record(stream)
        stage_events.append([])
        step()
        e1.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    clk_after = read_gfx_clock()
    ibwd.set_stage_hook(None)
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in calls]
    total_ms = t_all0.elapsed_time(t_all1)
    med_us = statistics.median(per_call_ms) * 1e3
    mean_us = statistics.fmean(per_call_ms) * 1e3
    flops = wl.flops()
    tflops = flops / (med_us * 1e-6) / 1e12
    ms_per_step = total_ms / args.steps

    # per-kernel durations: event after kernel i minus event after kernel i-1
    # (the call's first event for i = 0)
    per_kernel = {}
    for (e0, _), evs in zip(calls, stage_events):
        prev = e0
        for stage, name, e in evs:
            per_kernel.setdefault((stage, name), []).append(prev.elapsed_time(e) * 1e3)
            prev = e
    kernels = []
    slot_rows = any(name == "dk_rows_kernel" for (_, name) in per_kernel)
    for (stage, name), ts in sorted(per_kernel.items()):
        bound, work = kernel_model(name, wl, B, H, D, S_q, S_k, 2 if args.bf16_out else 4, slot_rows)
        mean_k = statistics.fmean(ts)
        if bound == "mfma":
            ach, peak, unit = work / (mean_k * 1e-6) / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            ach, peak, unit = work / (mean_k * 1e-6) / 1e9, PEAK_HBM_GBS, "GB/s"
        kernels.append({"stage": stage, "kernel": name, "us_mean": round(mean_k, 2),
                        "us_median": round(statistics.median(ts), 2), "bound": bound,
                        "algorithmic_work": work, "achieved": round(ach, 3), "peak": peak,
                        "unit": unit, "frac": round(ach / peak, 4)})
    dom = max(kernels, key=lambda k: k["us_mean"])
    # the stored counters are for the workloads' own shapes only
    traffic = None if (args.topk or args.bf16_out) else measured_traffic(
        dom["kernel"], wl.name, bool(args.deterministic))

    # algorithmic HBM bytes of one call (inputs read once, outputs written once)
    row = wl.S_k if wl.dense else wl.topk
    ob = 2 if args.bf16_out else 4
    hbm_bytes = (B * S_q * H * D * 2 + B * S_k * D * 2 + B * S_q * H * 4
                 + B * S_q * row * (4 + 4 + (0 if wl.dense else 4))
                 + (B * S_q * H * D + B * S_q * H + B * S_k * D) * ob)

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": COMPUTE_DTYPE,
        "data": "synthetic (seeded PCG64; q,k ~N(0,1) bf16, w ~N(0,1)/8, per-row distinct ids, "
                "index_score recomputed fp32, attn_score softmax of N(0,1) logits)",
        "config": {"workload": wl.name, "B": B, "H": H, "D": D, "S_q": S_q, "S_k": S_k,
                   "topk": None if wl.dense else wl.topk, "pad_frac": wl.pad_frac,
                   "sorted_ids": wl.sorted_ids, "dense": wl.dense,
                   "deterministic": bool(args.deterministic), "atomic_dk": bool(args.atomic_dk),
                   "bf16_out": bool(args.bf16_out),
                   "dk_route": "atomic" if args.atomic_dk else ("slot_rows" if slot_rows else "key_ranges")},
        "us_per_call_median": round(med_us, 2),
        "us_per_call_mean": round(mean_us, 2),
        "us_per_call_min": round(min(per_call_ms) * 1e3, 2),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flop_per_call": flops,
        "roofline": {
            "bound": dom["bound"],
            "achieved": dom["achieved"],
            "peak": dom["peak"],
            "unit": dom["unit"],
            "frac": dom["frac"],
            "traffic": traffic,
            "kernel": dom["kernel"],
            "us_mean": dom["us_mean"],
            "algorithmic_work": dom["algorithmic_work"],
        },
        "kernels": kernels,
        "clocks": clock_report(clk_before, clk_load, clk_after, tflops, dom),
        "call_hbm_algorithmic_bytes": hbm_bytes,
        "pages_context": {"kernel_gemm_us_B200_anchor": 1688.8,
                          "note": "NVIDIA B200 figure from the pages; context only"},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def forward_main(args):
    """The indexer forward scores (every key; causal for the dense workload) and
    the top-k selection of the workload's topk (S_k/2 for the dense workload),
    timed like the backward: W untimed steps, K timed steps on one stream with
    HIP events around each step and after each kernel."""
    import numpy as np
    import torch

    import dsa_lightning_indexer_bwd_amd as ibwd
    from synth import WORKLOADS, make_inputs

    ibwd.library()
    wl = WORKLOADS[args.workload]
    if args.topk:
        wl = dataclasses.replace(wl, topk=args.topk)
    topk = wl.S_k // 2 if wl.dense else wl.topk
    dev = torch.device("cuda:0")
    print("bench: generating %s inputs" % wl.name, file=sys.stderr, flush=True)
    x = make_inputs(wl, device=dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k = bf16(x.q), bf16(x.k)
    w = torch.from_numpy(x.w).to(dev)
    B, S_q, H, D = x.q.shape
    S_k = x.k.shape[1]
    causal = bool(wl.dense)
    scores = torch.empty((B, S_q, S_k), dtype=torch.float32, device=dev)
    ids = torch.empty((B, S_q, topk), dtype=torch.int32, device=dev)
    vals = torch.empty((B, S_q, topk), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)

    def step():
        ibwd.indexer_fwd_scores(q, k, w, scores, causal=causal, q_offset=wl.q_offset, stream=stream)
        ibwd.indexer_topk(scores, topk, ids, vals, stream=stream)

    if args.calibration_copy_mib:
        src = torch.ones(args.calibration_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stage_events = []

    def hook(stage, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        stage_events[-1].append((name, e))

    calls = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    ibwd.set_stage_hook(hook)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for e0, e1 in calls:
        e0.record(stream)
        stage_events.append([])
        step()
        e1.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    ibwd.set_stage_hook(None)
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in calls]
    med_us = statistics.median(per_call_ms) * 1e3
    # (query, key) pairs scored: every key, or the causal triangle
    t = np.arange(S_q, dtype=np.int64)
    pairs = B * int(np.clip(t + wl.q_offset + 1, 0, S_k).sum()) if causal else B * S_q * S_k
    flops = 2 * pairs * H * D
    per_kernel = {}
    for (e0, _), evs in zip(calls, stage_events):
        prev = e0
        for name, e in evs:
            per_kernel.setdefault(name, []).append(prev.elapsed_time(e) * 1e3)
            prev = e
    kernels = []
    for name in ("fwd_scores_kernel", "topk_kernel"):
        ts = per_kernel[name]
        mean_k = statistics.fmean(ts)
        if name == "fwd_scores_kernel":
            work, unit, peak = flops, "TFLOP/s", PEAK_BF16_TFLOPS
            ach = work / (mean_k * 1e-6) / 1e12
        else:
            # scores read once, ids and values written once
            work, unit, peak = B * S_q * (S_k * 4 + topk * 8), "GB/s", PEAK_HBM_GBS
            ach = work / (mean_k * 1e-6) / 1e9
        kernels.append({"kernel": name, "us_mean": round(mean_k, 2),
                        "us_median": round(statistics.median(ts), 2),
                        "bound": "mfma" if unit == "TFLOP/s" else "hbm", "algorithmic_work": work,
                        "achieved": round(ach, 3), "peak": peak, "unit": unit,
                        "frac": round(ach / peak, 4)})
    dom = max(kernels, key=lambda r: r["us_mean"])
    tflops = flops / (med_us * 1e-6) / 1e12
    out = {
        "metric": "indexer forward scores + top-k: TFLOP/s of the score GEMM over the whole step",
        "value": round(tflops, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t_all0.elapsed_time(t_all1) / args.steps, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": COMPUTE_DTYPE,
        "data": "synthetic (seeded PCG64; q,k ~N(0,1) bf16, w ~N(0,1)/8)",
        "config": {"workload": wl.name + "-forward", "B": B, "H": H, "D": D, "S_q": S_q, "S_k": S_k,
                   "topk": topk, "causal": causal, "q_offset": wl.q_offset},
        "us_per_call_median": round(med_us, 2),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {"bound": dom["bound"], "achieved": dom["achieved"], "peak": dom["peak"],
                     "unit": dom["unit"], "frac": dom["frac"],
                     "traffic": None if args.topk else measured_traffic(dom["kernel"],
                                                                       wl.name + "-forward", False),
                     "kernel": dom["kernel"], "us_mean": dom["us_mean"],
                     "algorithmic_work": dom["algorithmic_work"]},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_forward(x, wl, topk, causal, flops, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def cpu_baseline_forward(x, wl, topk, causal, flops, seconds):
    """The oracle's forward scores and top-k on the first rows of the workload,
    grown until they take about `seconds`, scaled to the whole step."""
    import numpy as np

    import oracle

    q = oracle.widen_bf16(x.q)
    k = oracle.widen_bf16(x.k)
    S_q = q.shape[1]
    n, spent = 16, 0.0
    while True:
        n = min(n, S_q)
        t0 = time.perf_counter()
        sc = oracle.forward_scores(q[:, :n], k, x.w[:, :n], wl.q_offset if causal else None,
                                   np.arange(n))
        oracle.select_topk(sc, topk)
        spent = time.perf_counter() - t0
        if spent * 4 > seconds or n == S_q:
            break
        n *= 4
    full_s = spent * S_q / n
    return {"value": round(flops / full_s / 1e12, 6), "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
            "sample": "first %d of %d query rows (scores over every key, then top-%d), %.2f s wall"
                      % (n, S_q, topk, spent),
            "us_per_call_extrapolated": round(full_s * 1e6, 1)}


def clock_report(before, load, after, tflops, dom):
    """amd-smi GFX clocks around the timed region, and the bf16 peak rescaled
    from its 2.4 GHz rating to the clock measured under load."""
    rep = {"before_timing": before, "under_load": load, "after_timing": after,
           "source": "amd-smi metric -c (mean of the accelerator dies' GFX clocks)"}
    if load and load.get("mhz"):
        peak = PEAK_BF16_TFLOPS * load["mhz"] / 2400.0
        rep["bf16_peak_at_load_clock_tflops"] = round(peak, 1)
        rep["frac_of_bf16_peak_at_load_clock"] = round(tflops / peak, 4)
        if dom["unit"] == "TFLOP/s":
            rep["roofline_frac_at_load_clock"] = round(dom["achieved"] / peak, 4)
    return rep


def read_gfx_clock():
    """GFX clock of the GPU as amd-smi reports it now: {"mhz": mean over the
    accelerator dies' current clocks, "max_mhz": their rated maximum}, or None
    when amd-smi is unavailable.  The clocks drop to a few hundred MHz when the
    GPU idles, so a sample means something only while kernels run."""
    import shutil
    import subprocess

    try:
        # amd-smi is a Python script started through `env`; running it with this
        # interpreter directly keeps the child from replacing itself once more
        # (a profiler's preloaded library may have initialised the GPU in it)
        tool = shutil.which("amd-smi")
        if tool is None:
            return None
        tool = os.path.realpath(tool)
        with open(tool, "rb") as f:
            head = f.readline()
        cmd = [sys.executable, tool] if b"python" in head else [tool]
        res = subprocess.run(cmd + ["metric", "-c", "--json"], capture_output=True, text=True,
                             timeout=20)
        start = res.stdout.find("{")
        data = json.loads(res.stdout[start:]) if start >= 0 else None
        gpus = data["gpu_data"] if isinstance(data, dict) else data
        clocks = gpus[0]["clock"]
        cur = [v["clk"]["value"] for key, v in clocks.items()
               if key.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        mx = [v["max_clk"]["value"] for key, v in clocks.items()
              if key.startswith("gfx_") and isinstance(v.get("max_clk"), dict)]
        cur = [float(c) for c in cur if isinstance(c, (int, float))]
        mx = [float(c) for c in mx if isinstance(c, (int, float))]
        if not cur:
            return None
        return {"mhz": round(sum(cur) / len(cur), 1), "max_mhz": max(mx) if mx else None}
    except Exception:
        return None


def clocks_under_load(step, sync, samples=3, spacing=1.0):
    """GFX clock under load: amd-smi sampled `samples` times, `spacing` seconds
    apart after a first second of load, from a thread while the main thread
    keeps running calls (untimed).  The driver's clock figures are refreshed
    about once a second, so samples of a shorter run repeat one stale value.
    Returns {"mhz": mean of the samples, "samples_mhz": [...], "max_mhz": ...}."""
    import threading

    got = []

    def sample():
        for _ in range(samples):
            time.sleep(spacing)
            got.append(read_gfx_clock())

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while th.is_alive() and time.perf_counter() - t0 < samples * spacing + 30.0:
        for _ in range(8):
            step()
        sync()
    th.join(timeout=30.0)
    sync()
    vals = [g for g in got if g]
    if not vals:
        return None
    mhz = [g["mhz"] for g in vals]
    return {"mhz": round(sum(mhz) / len(mhz), 1), "samples_mhz": mhz,
            "max_mhz": vals[0].get("max_mhz")}


def query_blocks(B, S_q, S_k):
    """Query blocks as the library lays them out: 128-key ranges, about 512
    range workgroups, at most 512 queries per block."""
    nr = (S_k + 127) // 128
    nqb = max(-(-512 // (nr * B)), -(-S_q // 512))
    nqb = max(1, min(nqb, S_q))
    qbs = -(-S_q // nqb)
    return -(-S_q // qbs)


def kernel_model(name, wl, B, H, D, S_q, S_k, out_bytes=4, slot_rows=False):
    """(bound, algorithmic work per launch) of one kernel of the call.

    Work units per query row are the row's slots (topk, or t+1 for the dense
    variant): the prep kernel reads the slot inputs and writes one 8-byte
    {position, dI} per slot, the row kernels do GEMM1 + GEMM2 (4*H*D FLOP per slot), the range
    kernel the dK GEMM (2*H*D per slot), the atomic-route row kernel all three, and
    so does the row kernel of the slot-row route (its third product is the slot's
    dK row).  The slot-row sum reads each slot's dK row and key once and writes
    the query blocks' partial dK; the slab sum reads every query block's partial
    dK once and writes d_k (out_bytes per element)."""
    slots = wl.flops() // (6 * H * D)
    if name == "row_prep_kernel":
        # ids (sparse), I and p read once, {position, dI} written per slot
        return "hbm", (16 if wl.dense else 20) * slots
    if name == "row_export_kernel":
        return "mfma", (6 if slot_rows else 4) * H * D * slots
    if name == "dk_range_kernel":
        return "mfma", 2 * H * D * slots
    if name == "dk_rows_kernel":
        return "hbm", (D * 4 + 4) * slots + query_blocks(B, S_q, S_k) * B * S_k * D * 4
    if name == "row_kernel":
        return "mfma", 6 * H * D * slots
    if name == "dk_sum_kernel":
        return "hbm", (query_blocks(B, S_q, S_k) * 4 + out_bytes) * B * S_k * D
    if name == "zero_u32_kernel":
        return "hbm", B * S_k * D * 4
    raise KeyError(name)


def source_digest():
    """sha256 over the HIP library sources (the key of a stored counter run)."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dsa_lightning_indexer_bwd_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload, deterministic):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known size),
    or None when there is none for this kernel and workload or the library
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % workload)
    if not os.path.exists(path):
        return None
    want = source_digest()
    for line in open(path):
        if not line.startswith("traffic:"):
            continue
        kv = dict(t.split("=", 1) for t in line.split()[1:])
        if kv.get("kernel") == kernel and kv.get("src") == want:
            return int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    return None


def cpu_baseline(x, wl, target_s):
    """The fp64 oracle, as it stands, on the first n query rows of the same
    workload (the same per-row work, including the dK scatter of those rows)."""
    import dataclasses

    import oracle
    from synth import Inputs

    def sub(n):
        w2 = dataclasses.replace(wl, S_q=n)
        return Inputs(w2, x.q[:, :n], x.k, x.w[:, :n], None if x.ids is None else x.ids[:, :n],
                      x.index_score[:, :n], x.attn_score[:, :n], x.sm_scale, x.grad_loss)

    print("bench: cpu baseline calibration", file=sys.stderr, flush=True)
    n0 = min(wl.S_q, 64)
    t0 = time.perf_counter()
    oracle.Problem.from_inputs(sub(n0)).backward()
    t_cal = time.perf_counter() - t0
    # three timed runs of about target_s / 3 each; the median is reported
    n = int(min(wl.S_q, max(n0, n0 * target_s / 3.0 / max(t_cal, 1e-3))))
    xs = sub(n)
    prob = oracle.Problem.from_inputs(xs)
    runs = []
    for _ in range(3):
        t0 = time.perf_counter()
        prob.backward()
        runs.append(time.perf_counter() - t0)
    dt = statistics.median(runs)
    fl = xs.wl.flops()
    return {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "first %d of %d query rows of the %s workload (full backward of those rows incl. "
                  "their dK scatter); median of 3 runs: %s s wall"
                  % (n, wl.S_q, wl.name, ", ".join("%.2f" % r for r in runs)),
        "runs_s": [round(r, 3) for r in runs],
        "us_per_call_extrapolated": round(dt * wl.S_q / n * 1e6, 1),
        "nproc": os.cpu_count(),
    }


if __name__ == "__main__":
    main()
