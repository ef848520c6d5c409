#!/usr/bin/env python3
"""Benchmark of the LaCT fast-weight layer on one MI355X.

One step = one whole sequence of the workload through lact_sequence (every
chunk read, every chunk but the last written with momentum, Muon, step and
row renorm), starting from the initial fast weights, inputs already resident
in HBM.  The headline workload is the largest one that fits one GPU
(long-context: 1,048,576 tokens, 4 heads, d 256, dh 1024); the other bf16
workloads are timed the same way and reported beside it.  Prints one JSON
line.

  python bench.py [--steps K] [--warmup W] [--workload long-context] [--gpus 1]
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
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="long-context")
    p.add_argument("--ns-prec", default="bf16-shifted", choices=["bf16-shifted", "bf16", "f32"],
                   help="Newton-Schulz operand precision")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-others", action="store_true", help="time only the headline workload")
    p.add_argument("--backward-only", default=None, metavar="WORKLOAD",
                   help="only time lact_sequence_backward on WORKLOAD (one JSON line)")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="host time budget of the oracle sample (about 10-30 s)")
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


def measured_traffic(workload):
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


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, W, inp, budget_s):
    """The float64 oracle as it stands, on the host cores: head 0 of the
    workload, chunk by chunk from the start of the sequence (the oracle's
    own state carried from chunk to chunk), until about `budget_s` seconds of
    host time are spent; scaled to the whole workload by the number of
    (head, chunk) steps."""
    import threadpoolctl
    from oracle import lact_oracle as O
    from chunk_test_head_amd import workloads as WL
    bounds = w.chunk_bounds()
    b = 0
    st = O.HeadState(W[0][b], W[1][b], W[2][b])
    e = inp["eta"][b]
    m = None if inp["mom"] is None else inp["mom"][b]
    t0 = time.perf_counter()
    done = 0
    for ci, (s0, e0) in enumerate(bounds):
        kw = dict(mom=None if m is None else m[s0:e0], order=w.order, subset=w.subset,
                  update_last=w.update_last or ci < len(bounds) - 1, use_muon=w.use_muon,
                  use_momentum=w.use_momentum, renorm=w.renorm, state=st)
        _, st = O.sequence(W[0][b], W[1][b], W[2][b], WL.token_values(inp, "q", b, s0, e0),
                           WL.token_values(inp, "k", b, s0, e0), WL.token_values(inp, "v", b, s0, e0),
                           e[s0:e0], e[s0:e0], e[s0:e0], w.chunk, **kw)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    full = dt * w.bh * len(bounds) / done
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    return {
        "value": w.batch * w.T / full,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"head 0 of {w.bh}, the first {done} of {len(bounds)} chunks of the {w.T}-token "
                  f"sequence, {dt:.1f} s, scaled by {w.bh} x {len(bounds)} / {done} (head, chunk) steps; "
                  f"numpy float64 with {threads} BLAS threads on a host with {os.cpu_count()} logical "
                  f"CPUs ({cpu_model()})",
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model(),
    }


# The pages' own throughput figures for this layer, with their hardware
# (context only: another machine, whole-layer or whole-model numbers).
PAGE_CONTEXT = {
    "ttt_layer_flops_utilization": "about 70% of peak on an NVIDIA A100 with large chunks in plain "
                                   "PyTorch (summary page, section 1, Fig. 1a)",
    "lm_training_tokens_per_s": "4.3K and 5.0K tokens/s for the Muon LM variant and its comparison model, "
                                "A100-40GB training runs (summary page, section 5.2, Table 3)",
}


def time_workload(w, steps, warmup, ns_prec, profile, values=False):
    """Times `steps` whole sequences of workload w (after `warmup`); with
    profile, also the mean launch time of the gradient kernel over the writes
    of the first timed sequence.  Returns a dict (and the inputs)."""
    import numpy as np
    import torch

    from chunk_test_head_amd import _lib as L
    from chunk_test_head_amd import workloads as WL

    dev = torch.device("cuda:0")
    W = WL.weights(w)
    inp = WL.tokens(w, threads=16, values=values or w.dtype != "bf16")
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
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm, ns_prec=ns_prec)
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region; the dominant kernel (the gradient launch) is bracketed by
    # HIP events on the same stream to give its average launch duration.
    # Only the launches of the first timed step are bracketed: each event
    # record costs a few us of queue bubble, which would otherwise be charged
    # to every step.
    n_grad = len(writes)
    if profile:
        L.lact_prof_begin(L.PROF_GRAD, max(1, n_grad))
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = max(gpu_ms, wall * 1e3) / steps
    flops = WL.algorithmic_flops(w)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = BF16_PEAK_TFLOPS if bf else F32_PEAK_TFLOPS
    res = {"ms_per_step": ms_per_step, "tokens_per_s": w.batch * w.T / (ms_per_step * 1e-3),
           "tflops_algorithmic": tflops, "pct_of_peak": 100.0 * tflops / peak,
           "tflops_page_convention": WL.page_convention_flops(w) / (ms_per_step * 1e-3) / 1e12,
           "peak": peak, "max_upd": max_upd}
    if profile:
        launches, grad_ms, grad_min, grad_max = L.lact_prof_end()
        res.update(launches=launches, grad_ms=grad_ms, grad_min=grad_min, grad_max=grad_max)
    del fw, q, k, v, out, ws
    torch.cuda.empty_cache()
    return res, W, inp


def time_decode(w, calls=200, warmup=20):
    """Streaming decode of workload w's shape: one new token per head per
    step through lact_decode_apply (weight-streaming read), timed over
    `calls` steps; the write that follows every `chunk` tokens is timed too
    (lact_update on one chunk), and the amortised per-token cost reported."""
    import numpy as np
    import torch

    from chunk_test_head_amd import _lib as L
    from chunk_test_head_amd import workloads as WL

    dev = torch.device("cuda:0")
    W = WL.weights(w)
    shape = L.Shape(w.bh, w.d, w.dh, L.BF16)
    fw = L.FastWeights(shape, *(torch.from_numpy(x).to(dev) for x in W), momentum=w.use_momentum)
    L.lact_init_state(shape, fw)
    g = torch.Generator(device="cpu").manual_seed(w.index)
    q = torch.randn(w.bh, calls, w.d, generator=g).to(dev, torch.bfloat16)
    out = torch.empty_like(q)
    ws = torch.zeros(L.decode_workspace_bytes(shape, 1), dtype=torch.uint8, device=dev)
    lay = L.layout_of(q)
    stream = torch.cuda.current_stream()
    for t in range(warmup):
        L.lact_decode_apply(shape, fw, q[:, t:t + 1], out[:, t:t + 1], ws, n_tok=1, q_layout=lay,
                            o_layout=lay, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for t in range(calls):
        L.lact_decode_apply(shape, fw, q[:, t:t + 1], out[:, t:t + 1], ws, n_tok=1, q_layout=lay,
                            o_layout=lay, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    # the same steps captured once into a HIP graph and replayed (a serving
    # loop would replay a captured step: launches then cost less)
    gs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            for t in range(calls):
                L.lact_decode_apply(shape, fw, q[:, t:t + 1], out[:, t:t + 1], ws, n_tok=1, q_layout=lay,
                                    o_layout=lay, stream=gs)
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(3):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us_graph = e0.elapsed_time(e1) * 1e3 / (3 * calls)
    # the write of one full chunk
    C = w.chunk
    k = torch.randn(w.bh, C, w.d, generator=g).to(dev, torch.bfloat16)
    v = torch.randn(w.bh, C, w.d, generator=g).to(dev, torch.bfloat16)
    eta = torch.full((w.bh, C), 0.01, device=dev)
    mom = torch.full((w.bh, C), w.momentum, device=dev) if w.use_momentum else None
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
    wsu = torch.empty(L.workspace_bytes(shape, C, o), dtype=torch.uint8, device=dev)
    for _ in range(3):
        L.lact_update(shape, fw, k, v, eta, eta, eta, mom, o, wsu, stream=stream)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        L.lact_update(shape, fw, k, v, eta, eta, eta, mom, o, wsu, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    write_us = e0.elapsed_time(e1) * 1e3 / 5
    wbytes = 3.0 * w.d * w.dh * 2 * w.bh
    return {"heads": w.bh, "d": w.d, "dh": w.dh, "weight_bytes_per_step": wbytes,
            "us_per_token_step": us, "tokens_per_s": w.batch / (us * 1e-6),
            "weight_gbs": wbytes / (us * 1e-6) / 1e9, "pct_of_hbm": 100.0 * wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "graph_us_per_token_step": us_graph, "graph_tokens_per_s": w.batch / (us_graph * 1e-6),
            "graph_weight_gbs": wbytes / (us_graph * 1e-6) / 1e9,
            "write_us_per_chunk": write_us, "chunk": C,
            "amortised_us_per_token_step": us + write_us / C}


def backward_gemm_flops(w):
    """GEMM flops that lact_sequence_backward executes for workload w (all
    heads), recomputation included: per write of n tokens the forward
    recompute (12 n d dh, twice: the forward pass and again in the reverse
    pass) and the write's VJP (30 n d dh); per read of n tokens 16 n d dh;
    with Muon, per matrix and Newton-Schulz step 4 d^2 dh + 2 d^3 forward
    (twice) and 8 d^2 dh + 6 d^3 for the VJP."""
    d, dh = w.d, w.dh
    per_head = 0.0
    for _, a, z in w.writes():
        n = z - a
        per_head += (2 * 12 + 30) * n * d * dh
        if w.use_muon:
            per_head += 3 * 5 * (2 * (4 * d * d * dh + 2 * d ** 3) + (8 * d * d * dh + 6 * d ** 3))
    for s0, e0 in w.chunk_bounds():
        per_head += 16 * (e0 - s0) * d * dh
    return per_head * w.bh


def time_backward(w, reps=3):
    """lact_sequence_backward over the whole sequence of workload w (bf16
    activations, fp32 compute), seeded random cotangent dO."""
    import numpy as np
    import torch

    from chunk_test_head_amd import _lib as L
    from chunk_test_head_amd import workloads as WL

    dev = torch.device("cuda:0")
    W = [torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in WL.weights(w)]
    inp = WL.tokens(w, threads=16, values=False)
    up = lambda n: torch.from_numpy(inp[n + "_bits"].view(np.int16)).to(dev).view(torch.bfloat16)
    q, k, v = up("q"), up("k"), up("v")
    eta = torch.from_numpy(inp["eta"]).to(dev)
    mom = torch.from_numpy(inp["mom"]).to(dev) if inp["mom"] is not None else None
    g = torch.Generator(device=dev).manual_seed(w.index)
    dout = torch.randn(w.bh, w.T, w.d, device=dev, generator=g)
    shape = L.Shape(w.bh, w.d, w.dh, L.BF16)
    o = L.opts(use_muon=w.use_muon, use_momentum=w.use_momentum, renorm=w.renorm)
    grads = {"dq": torch.empty(w.bh, w.T, w.d, device=dev), "dk": torch.empty(w.bh, w.T, w.d, device=dev),
             "dv": torch.empty(w.bh, w.T, w.d, device=dev), "deta1": torch.empty(w.bh, w.T, device=dev),
             "dmom": torch.empty(w.bh, w.T, device=dev) if mom is not None else None,
             "dw1": torch.empty_like(W[0]), "dw3": torch.empty_like(W[1]), "dw2": torch.empty_like(W[2])}
    grads["deta3"] = grads["deta2"] = grads["deta1"]  # one rate for the three matrices: the terms add
    ws = torch.empty(L.backward_workspace_bytes(shape, w.T, w.chunk, o), dtype=torch.uint8, device=dev)

    def run():
        L.lact_sequence_backward(shape, W[0], W[1], W[2], q, k, v, dout, eta, eta, eta, mom, w.T, w.chunk,
                                 w.order, w.subset, int(w.update_last), o, grads, ws)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    fl = backward_gemm_flops(w)
    return {"workload": w.name, "ms_per_sequence": ms, "tokens_per_s": w.batch * w.T / (ms * 1e-3),
            "gemm_tflops_executed": fl / (ms * 1e-3) / 1e12,
            "pct_of_fp32_peak": 100.0 * fl / (ms * 1e-3) / 1e12 / F32_PEAK_TFLOPS,
            "workspace_bytes": ws.numel(), "compute": "fp32 (forward recomputed chunk by chunk)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only (one process, one device); "
                                   "--gpus must be 1"}))
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.backward_only:
        from chunk_test_head_amd import workloads as WL
        print(json.dumps({"outer_loop_backward": time_backward(WL.get(args.backward_only))}), flush=True)
        return
    from chunk_test_head_amd import _lib as L
    from chunk_test_head_amd import workloads as WL

    prec = {"bf16-shifted": L.NS_BF16_SHIFTED, "bf16": L.NS_BF16, "f32": L.NS_F32}[args.ns_prec]
    w = WL.get(args.workload)
    bf = w.dtype == "bf16"
    r, W, inp = time_workload(w, args.steps, args.warmup, prec, profile=True)
    ms_per_step = r["ms_per_step"]
    peak = r["peak"]

    # roofline of the dominant kernel: 12 d dh flops per written token
    # (forward on keys 6 d dh + gradient contractions 6 d dh), bh heads
    grad_flops = 12.0 * w.d * w.dh * r["max_upd"] * w.bh
    launches = r["launches"]
    grad_avg_ms = r["grad_ms"] / max(1, launches)
    achieved = grad_flops / (grad_avg_ms * 1e-3) / 1e12
    line = {
        "metric": "fast-weight chunk-step tokens/s (LaCT SwiGLU layer, whole sequence)",
        "value": r["tokens_per_s"],
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
                   "subset": list(w.subset) if w.subset else None,
                   "ns_prec": args.ns_prec if w.use_muon else None},
        "tflops_algorithmic": r["tflops_algorithmic"],
        "pct_of_peak": r["pct_of_peak"],
        "tflops_page_convention": r["tflops_page_convention"],
        "roofline": {"bound": "mfma",
                     "kernel": "k_grad" if not bf else ("k_grad_solo" if w.d == 256 else "k_grad_bf16"),
                     "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": measured_traffic(w.name),
                     "launch_ms_avg": grad_avg_ms, "launch_ms_min": r["grad_min"],
                     "launch_ms_max": r["grad_max"], "launches": launches,
                     "flops_per_launch": grad_flops},
        "page_context": PAGE_CONTEXT,
    }
    if not args.no_others:
        others = {}
        for name in ("lm-causal", "nvs-bidirectional", "ar-video", "long-context"):
            if name == w.name:
                continue
            ro, _, _ = time_workload(WL.get(name), args.steps, args.warmup, prec, profile=False)
            others[name] = {k: ro[k] for k in ("tokens_per_s", "ms_per_step", "tflops_algorithmic",
                                               "pct_of_peak", "tflops_page_convention")}
        line["other_workloads"] = others
        line["streaming_decode"] = {name: time_decode(WL.get(name)) for name in ("lm-causal", "long-context")}
        line["outer_loop_backward"] = time_backward(WL.get("lm-causal"))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, W, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
