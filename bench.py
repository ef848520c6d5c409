#!/usr/bin/env python3
"""Benchmark of the LaCT fast-weight layer on one MI355X.

One step = one whole sequence of the workload through lact_sequence (every
chunk read, every chunk but the last written with momentum, Muon, step and
row renorm), starting from the initial fast weights, inputs already resident
in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload lm-causal] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
F32_PEAK_TFLOPS = 157.3     # MI355X dense fp32 MFMA
HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="lm-causal")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-heads", type=int, default=32, help="heads of the oracle sample (10-30 s of host work)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a plain device copy of BYTES (counter calibration)")
    return p.parse_args()


def copy_probe(nbytes):
    """A plain device-to-device copy of a known size, to calibrate the
    FETCH_SIZE / WRITE_SIZE counters against a kernel whose traffic is
    known exactly (nbytes read, nbytes written)."""
    import torch
    x = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)


def measured_traffic(kernel_src, workload):
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile (FETCH_SIZE / WRITE_SIZE, copy-calibrated), or None when the
    profile is for another workload or the kernel source changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_grad_{workload}_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, rec["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
                return None
        return rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, W, inp, heads):
    """The float64 oracle as it stands, on the host cores, on `heads` of the
    workload's heads over the whole sequence; scaled to all heads."""
    import threadpoolctl
    from oracle import lact_oracle as O
    heads = min(heads, w.bh)
    t0 = time.perf_counter()
    for b in range(heads):
        e = inp["eta"][b]
        m = None if inp["mom"] is None else inp["mom"][b]
        O.sequence(W[0][b], W[1][b], W[2][b], inp["q"][b], inp["k"][b], inp["v"][b], e, e, e, w.chunk,
                   mom=m, order=w.order, subset=w.subset, update_last=w.update_last,
                   use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
    dt = time.perf_counter() - t0
    full = dt * w.bh / heads
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {
        "value": w.batch * w.T / full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{heads} of {w.bh} (batch, head) states over the whole {w.T}-token sequence, "
                  f"{dt:.1f} s, scaled by {w.bh}/{heads}; numpy float64, BLAS threads={threads}",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    import numpy as np
    import torch

    from chunk_test_head_amd import _lib as L
    from chunk_test_head_amd import workloads as WL

    w = WL.get(args.workload)
    dev = torch.device("cuda:0")
    W = WL.weights(w)
    inp = WL.tokens(w, threads=16)
    bf = w.dtype == "bf16"

    def up(name):
        if bf:
            return torch.from_numpy(inp[name + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(inp[name]).to(dev)

    q, k, v = up("q"), up("k"), up("v")
    eta = torch.from_numpy(inp["eta"]).to(dev)
    mom = torch.from_numpy(inp["mom"]).to(dev) if inp["mom"] is not None else None
    out = torch.empty_like(q)
    shape = L.Shape(w.bh, w.d, w.dh, L.BF16 if bf else L.F32)
    W0 = [torch.from_numpy(x).to(dev) for x in W]
    fw = L.FastWeights(shape, *W0, momentum=w.use_momentum)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
    writes = w.writes()
    max_upd = max((z - a for _, a, z in writes), default=0)
    ws = torch.empty(L.workspace_bytes(shape, max_upd, o), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        # sequence start: fast weights back to their initial values
        fw.w1.copy_(W0[0])
        fw.w3.copy_(W0[1])
        fw.w2.copy_(W0[2])
        L.lact_init_state(shape, fw, stream)
        L.lact_sequence(shape, fw, q, k, v, out, eta, eta, eta, mom, w.T, w.chunk, w.order, w.subset,
                        int(w.update_last), o, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region; the dominant kernel (k_grad) is bracketed by HIP events on
    # the same stream to give its average launch duration.  Only the launches
    # of the first timed step are bracketed: each event record costs a few us
    # of queue bubble, which would otherwise be charged to every step.
    n_grad = len(writes)
    L.lact_prof_begin(L.PROF_GRAD, max(1, n_grad))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches, grad_ms, grad_min, grad_max = L.lact_prof_end()
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps

    tokens = w.batch * w.T
    flops = WL.algorithmic_flops(w)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if bf else F32_PEAK_TFLOPS

    # roofline of the dominant kernel: 12 d dh flops per written token
    # (forward on keys 6 d dh + gradient contractions 6 d dh), bh heads
    n_written = max_upd
    grad_flops = 12.0 * w.d * w.dh * n_written * w.bh
    grad_avg_ms = grad_ms / max(1, launches)
    achieved = grad_flops / (grad_avg_ms * 1e-3) / 1e12
    line = {
        "metric": "fast-weight chunk-step tokens/s (LaCT SwiGLU layer, whole sequence)",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf else "f32",
        "data": "synthetic (seeded q/k/v/eta/W0 with the workload's shapes and distributions)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "d": w.d, "dh": w.dh,
                   "T": w.T, "chunk": w.chunk, "muon": w.use_muon,
                   "momentum": w.momentum if w.use_momentum else None, "renorm": w.renorm,
                   "subset": list(w.subset) if w.subset else None},
        "tflops_algorithmic": tflops,
        "pct_of_peak": 100.0 * tflops / peak,
        "tflops_page_convention": WL.page_convention_flops(w) / (ms_per_step * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "kernel": "k_grad", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic("k_mlp.hip", w.name),
                     "launch_ms_avg": grad_avg_ms, "launch_ms_min": grad_min,
                     "launch_ms_max": grad_max, "launches": launches,
                     "flops_per_launch": grad_flops},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, W, inp, args.cpu_heads)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
