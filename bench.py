#!/usr/bin/env python3
"""Benchmark of the lightning-indexer backward on one MI355X.

One step = one full backward call (dK fill + main kernel [+ deterministic
passes]) over the anchor workload B=1, H=64, D=128, S_q=8192, S_k=4096,
topk=1024 (2% of slots padded), inputs resident in HBM before timing starts.
Prints ONE JSON line.  Throughput counts 6*H*D*topk FLOP per query (three
GEMMs of 2*H*D per slot: score recompute, dQ, dK), the count used for the
pages' own anchor figure.
"""
import argparse
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
    ap.add_argument("--deterministic", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the oracle sample")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dsa_lightning_indexer_bwd_amd as ibwd
    from synth import WORKLOADS, make_inputs

    ibwd.library()  # fails loudly when the HIP library is missing
    wl = WORKLOADS[args.workload]
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
    dq = torch.empty((B, S_q, H, D), dtype=torch.float32, device=dev)
    dw = torch.empty((B, S_q, H), dtype=torch.float32, device=dev)
    dk = torch.empty((B, S_k, D), dtype=torch.float32, device=dev)
    flags = ibwd.IBWD_FLAG_DETERMINISTIC if args.deterministic else 0
    ws_bytes = ibwd.indexer_bwd_workspace_bytes(wl.dense, B, S_q, S_k, H, D, wl.topk, flags)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev) if ws_bytes else None
    stream = torch.cuda.Stream(device=dev)

    def step():
        if ids is None:
            ibwd.indexer_bwd_dense(q, k, w, I, p, dq, dw, dk, q_offset=wl.q_offset,
                                   deterministic=args.deterministic, workspace=ws, stream=stream)
        else:
            ibwd.indexer_bwd_sparse(q, k, w, ids, I, p, dq, dw, dk,
                                    deterministic=args.deterministic, workspace=ws, stream=stream)

    torch.cuda.synchronize()
    print("bench: warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    # events recorded on the stream the kernels run on
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(args.steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for e0, e1 in pairs:
        e0.record(stream)
        step()
        e1.record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in pairs]
    total_ms = t_all0.elapsed_time(t_all1)
    med_us = statistics.median(per_call_ms) * 1e3
    mean_us = statistics.fmean(per_call_ms) * 1e3
    flops = wl.flops()
    tflops = flops / (med_us * 1e-6) / 1e12
    ms_per_step = total_ms / args.steps

    # algorithmic HBM bytes of one call (inputs read once, outputs written once)
    row = wl.S_k if wl.dense else wl.topk
    hbm_bytes = (B * S_q * H * D * 2 + B * S_k * D * 2 + B * S_q * H * 4
                 + B * S_q * row * (4 + 4 + (0 if wl.dense else 4))
                 + B * S_q * H * D * 4 + B * S_q * H * 4 + B * S_k * D * 4)

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
                   "deterministic": bool(args.deterministic)},
        "us_per_call_median": round(med_us, 2),
        "us_per_call_mean": round(mean_us, 2),
        "us_per_call_min": round(min(per_call_ms) * 1e3, 2),
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "flop_per_call": flops,
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "kernel": "full call (dK fill + main kernel), median of per-call HIP events on the "
                      "kernels' stream",
            "hbm_algorithmic_bytes": hbm_bytes,
            "hbm_GBs_at_this_time": round(hbm_bytes / (med_us * 1e-6) / 1e9, 1),
        },
        "pages_context": {"kernel_gemm_us_B200_anchor": 1688.8,
                          "note": "NVIDIA B200 kernel-2-only figure from the pages; context only"},
    }

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(x, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


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
    n = int(min(wl.S_q, max(n0, n0 * target_s / max(t_cal, 1e-3))))
    xs = sub(n)
    prob = oracle.Problem.from_inputs(xs)
    t0 = time.perf_counter()
    prob.backward()
    dt = time.perf_counter() - t0
    fl = xs.wl.flops()
    return {
        "value": round(fl / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "first %d of %d query rows of the %s workload (full backward of those rows incl. "
                  "their dK scatter), %.2f s wall" % (n, wl.S_q, wl.name, dt),
        "us_per_call_extrapolated": round(dt * wl.S_q / n * 1e6, 1),
        "nproc": os.cpu_count(),
    }


if __name__ == "__main__":
    main()
