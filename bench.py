#!/usr/bin/env python3
"""Decode-step benchmark: one tensor-parallel rank's share of a decode step.

A step is one pass of the whole path over one batch: for each of the L
layers, the mixer output projection and the FFN down projection of this
rank's weight slice (bf16, fp32 accumulation), each followed by the
ring-ordered sum of the N ranks' partials plus the residual. The default
workload is the 27B specimen of "Interconnects e clusters" (lesson 9.9,
section 01 · Conceito): hidden 5120, FFN 17408, 64 layers (128 reductions
per token), 4 ranks, batch 1; rank 0's slice is timed, the other ranks'
partials are inputs already in HBM.

Prints one JSON line: decode tokens/s per rank-shard, plus the achieved HBM
bandwidth of the dominant kernel against the MI355X peak (8 TB/s) and the
CPU oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s per rank-shard; achieved HBM GB/s as % of MI355X peak"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_inputs(w, rank, seed=0):
    import numpy as np
    import torch

    from row_gemv_reduction_amd import synth
    L, b, H = w.layers, w.batch, w.hidden
    kw = dict(seed=seed, workload=w.name, rank=rank)
    xa = synth.device_normal((L, b, w.ka_r), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, w.ka_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, b, w.ki_r), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, w.ki_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    sig = synth.WEIGHT_STD * math.sqrt(w.ki_r)
    slots = synth.device_normal((L, 2, w.n_ranks, b, H), sig, torch.float32, tensor="slots",
                                seed=seed, workload=w.name)
    h0 = synth.device_normal((b, H), 1.0, torch.float32, tensor="residual", seed=seed,
                             workload=w.name)
    torch.cuda.synchronize()
    return xa, wo, xf, wd, slots, h0


def cpu_baseline(w, rank, xa, wo, xf, wd, slots, h0, budget_s):
    """Time the CPU oracle on a bounded sample of the same workload: whole
    steps over the first Ls layers of the stack (the same per-point work as
    the GPU step), repeated until about budget_s of CPU time has passed,
    scaled to the L-layer step."""
    import numpy as np
    import torch

    import oracle

    cores = len(os.sched_getaffinity(0))

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def run(nl):
        a = bits(xa[:nl]); o = bits(wo[:nl]); f = bits(xf[:nl]); d = bits(wd[:nl])
        s = slots[:nl].cpu().numpy()
        h = h0.cpu().numpy()
        t0 = time.perf_counter()
        oracle.decode_layers(rank, a, o, f, d, s, h, nthreads=cores)
        return time.perf_counter() - t0

    t1 = run(1)
    nl = int(max(1, min(w.layers, math.ceil(budget_s / max(t1, 1e-6)))))
    reps, total = 0, 0.0
    while total < budget_s or reps == 0:
        total += run(nl)
        reps += 1
    per_layer = total / (reps * nl)
    tok_s = w.batch / (per_layer * w.layers)
    return {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "%d run(s) of the first %d of %d layers of the same stack (rank %d, both "
                      "points, ring reductions), %.1f s in all, scaled linearly to %d layers"
                      % (reps, nl, w.layers, rank, total, w.layers)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, help="workload name (default: page-1 stack, N=4, b=1)")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune", action="append", default=[], help="key=value plan knob")
    ap.add_argument("--layout", choices=["auto", "packed", "rowmajor"], default="auto",
                    help="weight layout: strip-packed (packed once at load, untimed) or row-major")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the N virtual ranks are emulated on a single "
              "MI355X, so --gpus %d is not supported (use --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    import row_gemv_reduction_amd as tp
    from row_gemv_reduction_amd import workloads

    w = workloads.ALL[args.workload] if args.workload else workloads.PAGE1
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    tune = {}
    for kv in args.tune:
        k, v = kv.split("=")
        tune[k] = int(v)
    plan = tp.Plan(w.hidden, w.inter, w.n_ranks, w.batch, k_attn=w.k_attn, tune=tune)
    info = plan.info()
    log("workload %s: K_r = %s, splits %s, path %s" % (w.name, info["k_rank"], info["splits"],
                                                      info["path"]))
    xa, wo, xf, wd, slots, h0 = build_inputs(w, args.rank)
    ws = plan.new_workspace()
    hidden = h0.clone()
    stream = torch.cuda.current_stream()
    layout = args.layout
    if layout == "auto":
        layout = "packed" if w.batch <= 8 else "rowmajor"
    if layout == "packed":
        # load-time layout change, outside the timed region
        po = torch.empty(tp.packed_shape(plan, 0, w.layers), dtype=torch.bfloat16, device="cuda")
        pd = torch.empty(tp.packed_shape(plan, 1, w.layers), dtype=torch.bfloat16, device="cuda")
        tp.tp_pack_weights(plan, 0, wo, po)
        tp.tp_pack_weights(plan, 1, wd, pd)
        torch.cuda.synchronize()

        def step():
            tp.tp_decode_layers_packed(plan, w.layers, args.rank, xa, po, xf, pd, slots, hidden, ws)
    else:
        def step():
            tp.tp_decode_layers(plan, w.layers, args.rank, xa, wo, xf, wd, slots, hidden, ws)
    log("weight layout: %s" % layout)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / args.steps
    log("timed %d steps: %.4f ms/step (events), wall %.4f ms/step" % (args.steps, ms,
                                                                       wall * 1e3 / args.steps))

    tok_s = w.batch / (ms * 1e-3)
    step_bytes = w.algorithmic_bytes_per_step()
    achieved = step_bytes / (ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
        "kernel": "decode step, %s weights (%d reconciliation points, one launch)" % (layout, 2 * w.layers),
        "algorithmic_bytes_per_launch": step_bytes,
    }
    out = {
        "metric": METRIC, "value": round(tok_s, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": {"workload": w.name, "hidden": w.hidden, "inter": w.inter, "k_attn": w.k_attn,
                   "layers": w.layers, "n_ranks": w.n_ranks, "rank": args.rank,
                   "batch": w.batch, "reductions_per_token": 2 * w.layers, "weight_layout": layout,
                   "weight_bytes_per_step": w.weight_bytes_per_step()},
        "roofline": roofline,
        "context": {"pages_collective_latency_us": {"fast": 10, "slow": 50},
                    "pages_comm_ms_per_token": {"fast": 1.28, "slow": 6.4},
                    "pages_peer_bandwidth_gbs_gb200": 1800},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.rank, xa, wo, xf, wd, slots, h0,
                                           args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
