#!/usr/bin/env python3
"""Throughput of the MoE FFN layer forward on one MI355X.

A step is one whole-layer forward (RMSNorm + gate, top-k, sort, grouped
expert GEMMs, reduce, shared expert, residual) over one batch of seeded
synthetic tokens already resident in HBM. Eight layer instances with
distinct weights run round-robin, as consecutive layers of a model would,
so the weight stream cannot sit in the 256 MB Infinity Cache. Each step has
its own input buffer (the forward is in place), prepared before timing.

The K timed forwards are captured into one HIP graph and the step time comes
from one replay of it (a forward enqueues no allocation, host sync or
readback, so it captures whole, side-stream fork/join included), after one
untimed replay that absorbs the graph's first-launch set-up; --eager times K
plain forward calls instead.

Prints ONE JSON line. The roofline object covers the dominant kernel (the
slower of the grouped up / grouped down GEMMs), timed with HIP events on the
stream it runs on, over the K forwards: in graph mode over an eager pass of
the same K restored inputs right after the replay (events cannot sit inside
the graph). The cpu_baseline object times the float64 oracle on a bounded
token sample of the same workload on the host. `layer.ms_per_step_p10_p50_p90`
is the spread over --replays replays of the same K steps (inputs restored).
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
GEMV_MAX_N = 16  # token counts served by the decode-sized (GEMV) arm
BF16_PEAK_TFLOPS = 2500.0
METRIC = ("MoE-layer prefill tokens/s at N=1024 bf16; % MFMA peak (GEMM) / "
          "% HBM peak (N≤16)")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="nemotron_direct_bf16")
    ap.add_argument("--tokens", type=int, default=None, help="override N of the workload")
    ap.add_argument("--experts", type=int, default=None,
                    help="override E of the workload (e.g. one GPU's expert shard)")
    ap.add_argument("--instances", type=int, default=8)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="repeat the oracle forward until this much CPU time has passed")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="copy a buffer of this size once before timing (counter calibration "
                         "for rocprofv3 --pmc runs)")
    ap.add_argument("--all-stages", action="store_true",
                    help="record every stage (adds event markers to the timed region)")
    ap.add_argument("--eager", action="store_true",
                    help="time K eager forward calls instead of one HIP graph replay of them")
    ap.add_argument("--replays", type=int, default=5,
                    help="graph replays of the K steps for the reported spread (the first "
                         "replay gives value)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the layer's tokens shard across GPUs with no exchange, so the figure to "
              "measure is one GPU's throughput; no multi-GPU path is implemented",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    from mixture_experts_ffn_gate_amd import workloads as wlm
    from mixture_experts_ffn_gate_amd import moe_layer as ml

    wl = wlm.WORKLOADS[args.workload]
    if args.tokens:
        wl = wl.with_(N=args.tokens)
    if args.experts:
        wl = wl.with_(E=args.experts)
    N = wl.N
    torch.cuda.init()
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name} N={N} instances={args.instances} "
        f"steps={args.steps} warmup={args.warmup}")

    # Layers (weights generated on the device, copied into each layer, freed)
    # and one input batch per layer instance.
    layers, base = [], []
    host_w0 = None
    for i in range(args.instances):
        W = wlm.make_weights(wl, seed=args.seed + i, device=dev)
        layers.append(ml.layer_from_workload(wl, W, max_tokens=N))
        base.append(wlm.make_hidden(wl, N, seed=args.seed + i, device=dev, gate=W["gate"])[0])
        if i == 0 and not args.no_cpu_baseline:
            host_w0 = {k: wlm.to_numpy_f32(v) for k, v in W.items()}
        del W
    torch.cuda.synchronize()
    log("[bench] layers built")

    total = args.warmup + args.steps
    inputs = [base[j % args.instances].clone() for j in range(total)]
    residual = torch.empty_like(inputs[0])
    x0_host = wlm.to_numpy_f32(base[0]) if host_w0 is not None else None
    torch.cuda.synchronize()

    if args.calibrate_copy_mib:
        ca = torch.ones(args.calibrate_copy_mib << 20, dtype=torch.uint8, device=dev)
        cb = torch.empty_like(ca)
        torch.cuda.synchronize()
        cb.copy_(ca)
        torch.cuda.synchronize()
        del ca, cb

    for j in range(args.warmup):
        layers[j % args.instances].forward(inputs[j], residual)
    torch.cuda.synchronize()

    stages = ml.STAGES if args.all_stages else ("grouped_up", "grouped_down")
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    graph = None
    if not args.eager:
        # One graph holds the K forwards, each on its own (not yet used) input.
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for j in range(args.warmup, total):
                    layers[j % args.instances].forward(inputs[j], residual, stream=cap)
        torch.cuda.synchronize()
        # One untimed replay: the first launch of a new executable graph does
        # one-time set-up work on the device (measured ~0.7 ms for 50 forwards,
        # the slowest of every set of replays). The forward is in place, so
        # the inputs are restored before the timed replay.
        graph.replay()
        torch.cuda.synchronize()
        for j in range(args.warmup, total):
            inputs[j].copy_(base[j % args.instances])
        torch.cuda.synchronize()
    else:
        for L in layers:
            L.timing_begin(stages, max_forwards=args.steps)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for j in range(args.warmup, total):
            layers[j % args.instances].forward(inputs[j], residual)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    # Spread: more replays of the same K steps, each on restored inputs.
    spread = [ms_step]
    if graph is not None:
        for _ in range(args.replays - 1):
            for j in range(args.warmup, total):
                inputs[j].copy_(base[j % args.instances])
            torch.cuda.synchronize()
            ev0.record(stream)
            graph.replay()
            ev1.record(stream)
            torch.cuda.synchronize()
            spread.append(ev0.elapsed_time(ev1) / args.steps)
    spread_sorted = sorted(spread)

    def pct(q):
        return spread_sorted[min(len(spread_sorted) - 1, int(round(q * (len(spread_sorted) - 1))))]
    if graph is not None:
        # Kernel timing pass (eager, event markers) over the same K inputs,
        # restored first (the forward is in place).
        del graph
        for j in range(args.warmup, total):
            inputs[j].copy_(base[j % args.instances])
        torch.cuda.synchronize()
        for L in layers:
            L.timing_begin(stages, max_forwards=args.steps)
        for j in range(args.warmup, total):
            layers[j % args.instances].forward(inputs[j], residual)
        torch.cuda.synchronize()

    # Per-stage event times, summed over all instances.
    st_tot = {}
    for L in layers:
        for st, (ms, cnt) in L.timing_end().items():
            a = st_tot.setdefault(st, [0.0, 0])
            a[0] += ms
            a[1] += cnt
    stage_us = {st: 1000.0 * v[0] / v[1] for st, v in st_tot.items() if v[1]}
    log("[bench] stage averages (us): " + ", ".join(f"{k}={v:.1f}" for k, v in stage_us.items()))

    # Routing statistics of each instance (touched experts drive the weight bytes).
    touched = []
    max_load = []
    for L in layers[:min(total, args.instances)]:  # instances that ran a forward
        c = torch.empty(wl.E, dtype=torch.int32, device=dev)
        L.debug_read("counts", c)
        c = c.cpu().numpy()
        touched.append(int((c > 0).sum()))
        max_load.append(int(c.max()))
    E_t = float(np.mean(touched))
    R = N * wl.k
    D, I = wl.D, wl.I
    wb = 0.5625 if wl.expert_dtype == "nvfp4" else 2.0   # bytes per expert weight
    ab = 2.0 if wl.act_dtype == "bf16" else 4.0          # bytes per activation
    wbytes = E_t * I * D * wb
    # Algorithmic bytes of one launch: the touched experts' weights once, the
    # unique input rows once, the output rows once.
    algo = {
        "grouped_up": wbytes + N * D * ab + R * I * ab,
        "grouped_down": wbytes + R * I * ab + R * D * ab,
    }
    flops = {"grouped_up": 2.0 * R * D * I, "grouped_down": 2.0 * R * D * I}
    if N <= GEMV_MAX_N and wl.act_dtype == "bf16":
        # Decode-sized arm: the shared expert is a second segment of the same
        # launches (its weights once, its activations once).
        sb = wl.S * wl.H * wb
        algo["grouped_up"] += sb + N * wl.S * ab + (N * wl.H * ab if wl.L else 0)
        algo["grouped_down"] += sb + N * wl.S * ab + N * wl.H * ab
        flops["grouped_up"] += 2.0 * N * wl.S * wl.H
        flops["grouped_down"] += 2.0 * N * wl.S * wl.H
    dom = max(("grouped_up", "grouped_down"), key=lambda s: stage_us.get(s, 0.0))
    dom_s = stage_us[dom] * 1e-6
    ai = flops[dom] / algo[dom]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if ai < ridge:
        achieved = algo[dom] / dom_s / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = flops[dom] / dom_s / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roofline.update({"traffic": measured_traffic(wl, dom), "kernel": dom, "avg_us": round(stage_us[dom], 2),
                     "algorithmic_bytes": int(algo[dom]), "flops": flops[dom],
                     "arith_intensity": round(ai, 1),
                     "hbm_gbs": round(algo[dom] / dom_s / 1e9, 1),
                     "mfma_tflops": round(flops[dom] / dom_s / 1e12, 1)})

    tokens_per_s = N * args.steps / (ms_total / 1000.0)
    layer_flops = wl.flops(N)
    layer_bytes = (E_t * I * D * wb * 2 + wl.S * wl.H * wb * 2 + wl.E * wl.H * ab
                   + (wl.L * wl.H * ab * 2 if wl.L else 0) + N * wl.H * ab * 3)
    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.act_dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1/fan_in) weights, N(0,1) tokens)",
        "config": {"workload": wl.name, "hidden": wl.H, "experts": wl.E, "top_k": wl.k,
                   "moe_inter": wl.I, "shared_inter": wl.S, "latent": wl.L, "tokens": N,
                   "expert_dtype": wl.expert_dtype, "layer_instances": args.instances,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "layer": {"tflops": round(layer_flops / (ms_step * 1e-3) / 1e12, 1),
                  "gbs": round(layer_bytes / (ms_step * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "mfma_frac": round(layer_flops / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                     4),
                  "experts_touched": E_t, "max_expert_load": int(max(max_load)),
                  "stage_us": {k: round(v, 2) for k, v in stage_us.items()},
                  "wall_s": round(t_wall, 3),
                  "ms_per_step_p10_p50_p90": [round(pct(0.1), 4), round(pct(0.5), 4),
                                              round(pct(0.9), 4)],
                  "replays": len(spread),
                  "timed": "eager" if args.eager else "graph replay"},
        "cpu_baseline": None,
    }

    if host_w0 is not None:
        out["cpu_baseline"] = cpu_baseline(wl, host_w0, x0_host, args.cpu_min_seconds)
    print(json.dumps(out), flush=True)
    return 0


def measured_traffic(wl, stage):
    """HBM bytes per launch of ``stage`` from the committed rocprofv3 counter
    record of this workload (FETCH_SIZE + WRITE_SIZE, each scaled by a
    known-size copy), or None if there is none or the kernels changed since."""
    from mixture_experts_ffn_gate_amd import profiling

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        f"traffic_{wl.name}_n{wl.N}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != profiling.source_hash():
        return None
    role = "relu2" if stage == "grouped_up" else "store"
    wq = "nvfp4" if wl.expert_dtype == "nvfp4" else "bf16"
    prefix = (f"gemv[{role},{wq}]" if wl.N <= GEMV_MAX_N and wl.act_dtype == "bf16"
              else f"gemm[grouped,{role},{wq},")
    if wl.N == 1 and wl.L == 0 and wl.act_dtype == "bf16" and stage == "grouped_down":
        prefix = "gemv_down_reduce"  # one token: down projection fused with the reduce
    if rec.get("tokens") != wl.N:
        return None
    cands = [(v.get("dispatches", 0), v) for k, v in rec["kernels"].items()
             if k.startswith(prefix)]
    if not cands:
        return None
    v = max(cands, key=lambda c: c[0])[1]
    if "fetch_size_bytes" not in v or "write_size_bytes" not in v:
        return None
    return int(v["fetch_size_bytes"] + v["write_size_bytes"])


def host_cpu():
    """Model name (lscpu, else /proc/cpuinfo) and CPU counts of the host."""
    import subprocess

    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    try:
        usable = len(os.sched_getaffinity(0))
    except OSError:
        usable = os.cpu_count()
    return {"model": model, "cpus": os.cpu_count(), "usable": usable}


def cpu_baseline(wl, Wn, x, min_seconds):
    """The float64 oracle forward over layer instance 0's whole token batch, on
    the host, repeated until ``min_seconds`` of CPU time have passed."""
    import threadpoolctl

    from oracle import moe_oracle as mo

    if wl.expert_dtype == "nvfp4":
        from oracle import nvfp4 as onv
        Wn = dict(Wn)
        for k in ("up", "down", "shared_up", "shared_down"):
            if k in Wn:
                w = Wn[k] if Wn[k].ndim == 3 else Wn[k][None]
                deq = onv.dequantize_stack(*onv.quantize_stack(w))
                Wn[k] = deq if Wn[k].ndim == 3 else deq[0]
    xs = x.astype("float64")
    info = threadpoolctl.threadpool_info()
    threads = max([d.get("num_threads", 1) for d in info] or [1])
    reps, t = 0, time.perf_counter()
    while True:
        mo.layer_forward(xs, Wn, wl.oracle_cfg())
        reps += 1
        dt = time.perf_counter() - t
        if dt >= min_seconds:
            break
    tokens = reps * xs.shape[0]
    log(f"[bench] oracle: {reps} x {xs.shape[0]} tokens in {dt:.2f} s with {threads} BLAS threads")
    host = host_cpu()
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": host["model"], "host_cpus": host["cpus"],
            "host_cpus_usable": host["usable"],
            "sample": f"{reps} float64 oracle forward(s) of layer instance 0's {xs.shape[0]} "
                      f"tokens ({wl.name}), {dt:.1f} s of host time"}


if __name__ == "__main__":
    sys.exit(main())
