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

Other workloads (--workload NAME, see row_gemv_reduction_amd/workloads.py)
print the same line for that shape; the MoE decode share times one layer's
share (the 8192->4096 attention output slice at 64 tokens, its ring sum,
routing, the rank's experts and their ring sum) and rotates weight copies
so that the weights stream from HBM rather than from the 256 MB cache.
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
    out = {"value": tok_s, "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": "%d run(s) of the first %d of %d layers of the same stack (rank %d, both "
                     "points, ring reductions), %.1f s in all, scaled linearly to %d layers"
                     % (reps, nl, w.layers, rank, total, w.layers)}
    # the same oracle on one thread: a bounded sample of layers, scaled
    t0 = time.perf_counter()
    oracle.decode_layers(rank, bits(xa[:1]), bits(wo[:1]), bits(xf[:1]), bits(wd[:1]),
                         slots[:1].cpu().numpy(), h0.cpu().numpy(), nthreads=1)
    t_one = time.perf_counter() - t0
    n1 = int(max(1, min(w.layers, math.floor(budget_s / 2 / max(t_one, 1e-6)))))
    t0 = time.perf_counter()
    oracle.decode_layers(rank, bits(xa[:n1]), bits(wo[:n1]), bits(xf[:n1]), bits(wd[:n1]),
                         slots[:n1].cpu().numpy(), h0.cpu().numpy(), nthreads=1)
    t_n1 = time.perf_counter() - t0
    out["single_thread"] = {
        "value": w.batch / (t_n1 / n1 * w.layers), "unit": "tokens/s", "cores": 1,
        "sample": "the first %d of %d layers on one thread, %.1f s, scaled linearly" % (n1, w.layers, t_n1)}
    return out


WEIGHT_NAMES = {0: "bf16", 1: "mxfp8", 2: "mxfp4"}


def cpu_baseline_mx(w, rank, fmt, xa, wo, xf, wd, slots, h0, budget_s):
    """The oracle's MX decode step on a bounded sample of layers: per layer
    both points' MX projections (the oracle's own static conversion of the
    same bf16 weights, untimed) and their ring sums, threaded over columns;
    scaled to the L-layer step."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    h = h0.cpu().numpy()
    spent, nl = 0.0, 0
    wall0 = time.perf_counter()
    # the sample is bounded by wall time: the oracle's conversion (untimed)
    # takes seconds per layer
    while nl < w.layers and (time.perf_counter() - wall0 < budget_s or nl == 0):
        q = [oracle.mx_quantize(fmt, bits(W[nl])) for W in (wo, wd)]
        log("cpu baseline: layer %d converted" % nl)
        xs = (bits(xa[nl]), bits(xf[nl]))
        s = slots[nl].cpu().numpy()
        t0 = time.perf_counter()
        for pt in range(2):
            _, p32 = oracle.mx_partial(fmt, xs[pt], q[pt][0], q[pt][1], nthreads=cores)
            s[pt, rank] = p32
            h = oracle.ring_reduce(s[pt], h)
        spent += time.perf_counter() - t0
        nl += 1
    return {"value": w.batch / (spent / nl * w.layers), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "the first %d of %d layers (both points' %s projections and ring sums), "
                      "%.1f s, scaled linearly" % (nl, w.layers, WEIGHT_NAMES[fmt], spent)}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def tiny_single_thread(budget_s=2.0):
    """The oracle on one thread over the tiny config (hidden 512, FFN 1376,
    N = 2, b = 1, one layer: both points and their ring sums), repeated for
    about budget_s seconds."""
    import numpy as np

    import oracle
    from row_gemv_reduction_amd import synth, workloads
    w = workloads.TINY
    kw = dict(seed=0, workload=w.name, rank=0)
    xa = synth.normal_bf16((1, w.batch, w.ka_r), 1.0, tensor="x_attn", **kw)
    wo = synth.normal_bf16((1, w.ka_r, w.hidden), synth.WEIGHT_STD, tensor="w_o", **kw)
    xf = synth.normal_bf16((1, w.batch, w.ki_r), 1.0, tensor="x_ffn", **kw)
    wd = synth.normal_bf16((1, w.ki_r, w.hidden), synth.WEIGHT_STD, tensor="w_down", **kw)
    slots = synth.normal_f32((1, 2, w.n_ranks, w.batch, w.hidden), synth.WEIGHT_STD * np.sqrt(w.ki_r),
                             tensor="slots", seed=0, workload=w.name)
    h0 = synth.normal_f32((w.batch, w.hidden), 1.0, tensor="residual", seed=0, workload=w.name)
    reps, t = 0, 0.0
    while t < budget_s:
        t0 = time.perf_counter()
        oracle.decode_layers(0, xa, wo, xf, wd, slots, h0, nthreads=1)
        t += time.perf_counter() - t0
        reps += 1
    return {"workload": w.name, "value": w.batch * reps / t, "unit": "tokens/s", "cores": 1,
            "sample": "%d whole steps, %.1f s" % (reps, t)}


def measured_traffic(key):
    """HBM bytes per launch of the timed kernel from a committed counter
    summary under profiles/ (FETCH_SIZE + WRITE_SIZE, copy-calibrated): the
    one whose `traffic_key:` line is `key` (workload/layout/weights), when
    the kernel source it names still has the hash the counters were taken
    on; otherwise None."""
    import glob
    import hashlib
    import re

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        text = open(path).read()
        m_key = re.search(r"^traffic_key: (\S+)\s*$", text, re.M)
        if not m_key or m_key.group(1) != key:
            continue
        m_bytes = re.search(r"^traffic_bytes_per_launch: (\d+)", text, re.M)
        m_src = re.search(r"^kernel_source: (\S+) sha256 prefix ([0-9a-f]+)", text, re.M)
        if not (m_bytes and m_src):
            return None
        try:
            src = open(os.path.join(ROOT, m_src.group(1)), "rb").read()
        except OSError:
            return None
        if not hashlib.sha256(src).hexdigest().startswith(m_src.group(2)):
            return None
        return int(m_bytes.group(1))
    return None


# Key-value heads and head width of the QKV projection's synthetic width:
# four key-value heads ("Hosting Qwen on Blackwell", Prefillers, for its
# model); a head of 128 columns is a reading.
QKV_KV_HEADS = 4
QKV_HEAD_DIM = 128


def qkv_cols(k_attn, n_ranks):
    """The rank's Q, K and V columns: its k_attn / N query columns, and its
    share of the key-value heads for K and V, one head each where the ranks
    outnumber the heads (the heads are then replicated)."""
    kv = max(QKV_KV_HEADS // n_ranks, 1) * QKV_HEAD_DIM
    return k_attn // n_ranks + 2 * kv


def time_steps(step, steps, warmup, stream, check=None):
    """W untimed steps, then K timed steps between two HIP events recorded
    on the stream the library launches on. Returns ms per step. `check`
    (if given) runs after the warm-up and after the timed steps, and must
    raise if the steps were not valid (a timed-out wait)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if check:
        check()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    log("timed %d steps: %.4f ms/step (events), wall %.4f ms/step" % (steps, ms, wall * 1e3 / steps))
    if check:
        check()
    return ms


def ws_check(plan, ws, what):
    """A check for time_steps: the workspace's error word must be clear (a
    bounded wait that timed out would leave the timed steps invalid)."""
    import row_gemv_reduction_amd as tp

    def check():
        flags = tp.tp_workspace_status(plan, ws)
        if flags != 0:
            raise SystemExit("%s: the workspace reports a timed-out wait (flags %d): timing invalid"
                             % (what, flags))
    return check


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size (outside any timed region): its
    FETCH_SIZE / WRITE_SIZE counters calibrate the decode kernel's."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy calibration: %d x %d bytes read and written" % (reps, nbytes))


def dense_run(args, w, tune):
    import torch

    import row_gemv_reduction_amd as tp
    from row_gemv_reduction_amd import workloads
    fmt = args.weights
    plan = tp.Plan(w.hidden, w.inter, w.n_ranks, w.batch, k_attn=w.k_attn, tune=tune,
                   weight_format=fmt)
    info = plan.info()
    log("workload %s: K_r = %s, splits %s, path %s" % (w.name, info["k_rank"], info["splits"],
                                                      info["path"]))
    xa, wo, xf, wd, slots, h0 = build_inputs(w, args.rank)
    ws = plan.new_workspace()
    hidden = h0.clone()
    stream = torch.cuda.current_stream()
    layout = args.layout
    if layout == "auto":
        # (the packed partials exist on the vector-ALU stream only)
        packed_ok = info["packed_kind"] == 1 if args.op == "partials" else info["packed_kind"] != 0
        layout = "packed" if packed_ok else "rowmajor"
    extra = {}
    if fmt and layout != "packed":
        raise SystemExit("MX weights run on the packed step (--layout packed or auto)")
    if layout == "packed":
        # load-time layout change (and for MX weights the static conversion),
        # outside the timed region
        po = torch.empty(tp.packed_shape(plan, 0, w.layers), dtype=tp.packed_dtype(plan), device="cuda")
        pd = torch.empty(tp.packed_shape(plan, 1, w.layers), dtype=tp.packed_dtype(plan), device="cuda")
        if fmt:
            for pt, (W, P) in enumerate(((wo, po), (wd, pd))):
                codes = torch.empty(tp.mx_codes_shape(plan, pt, w.layers), dtype=torch.uint8, device="cuda")
                scales = torch.empty(tp.mx_scales_shape(plan, pt, w.layers), dtype=torch.uint8, device="cuda")
                tp.tp_quantize_mx(plan, pt, W, codes, scales)
                tp.tp_pack_weights_mx(plan, pt, codes, scales, P)
                del codes, scales
        else:
            tp.tp_pack_weights(plan, 0, wo, po)
            tp.tp_pack_weights(plan, 1, wd, pd)
        torch.cuda.synchronize()

        pa = torch.empty(tp.packed_act_shape(plan, 0, w.layers), dtype=torch.bfloat16, device="cuda")
        pf = torch.empty(tp.packed_act_shape(plan, 1, w.layers), dtype=torch.bfloat16, device="cuda")

        def step():
            # the activations' layout for the stream is part of the step
            # (none where the stream reads them row-major, as given)
            if info["packed_kind"] == 2 and info["acts_layout"] == 1:
                tp.tp_pack_activations(plan, xa, xf, pa, pf)
                tp.tp_decode_layers_packed(plan, w.layers, args.rank, pa, po, pf, pd, slots, hidden, ws)
            else:
                tp.tp_decode_layers_packed(plan, w.layers, args.rank, xa, po, xf, pd, slots, hidden, ws)
        name = "decode_stream" if info["packed_kind"] == 1 else (
            "decode_stream_mfma (%d workgroups sharing the tiles)" % info["stream_wgs"])
        if fmt:
            name += " on %s weights" % WEIGHT_NAMES[fmt]
        kernel = "%s (one launch per step, %d reconciliation points)" % (name, 2 * w.layers)
    else:
        def step():
            tp.tp_decode_layers(plan, w.layers, args.rank, xa, wo, xf, wd, slots, hidden, ws)
        if tune.get("decode_mode", 0) == 1:
            kernel = "decode step on row-major weights (one launch per point: %s + ring epilogue)" % (
                "mfma_gemm" if w.batch >= 16 else "valu_gemv")
        else:
            kernel = "decode step on row-major weights (one persistent launch: %s)" % (
                "decode_step_mfma" if w.batch >= 16 else "decode_step")
    if args.op == "partials" and layout == "packed":
        if info["packed_kind"] != 1:
            raise SystemExit("packed partials need packed_kind 1 (the vector-ALU stream)")
        pstack = torch.empty((w.layers, 2, w.batch, w.hidden), dtype=torch.float32, device="cuda")

        def step():
            tp.tp_rowparallel_partials_packed(plan, w.layers, xa, po, xf, pd, pstack, ws)
        ms = time_steps(step, args.steps, args.warmup, stream, ws_check(plan, ws, "packed partials"))
        nbytes = w.projection_bytes_per_step()
        config = {"workload": w.name, "op": "partials", "hidden": w.hidden, "inter": w.inter,
                  "k_attn": w.k_attn, "layers": w.layers, "n_ranks": w.n_ranks, "rank": args.rank,
                  "batch": w.batch, "launches_per_pass": 1, "us_per_launch": round(ms * 1e3, 3),
                  "timing": "eager, one launch", "weight_layout": "packed"}
        kernel = "tp_rowparallel_partials_packed: decode_stream, partials only, one launch per pass"
        plan.close()
        return ms, w.batch, nbytes, kernel, config, None, {"traffic": None,
                                                           "weight_bytes": w.weight_bytes_per_step()}
    if args.op != "step":
        if layout != "rowmajor" and args.op not in ("swiglu", "qkv"):
            raise SystemExit("--op %s runs on row-major weights (--layout rowmajor)" % args.op)
        return single_op_run(args, w, plan, info, tune, (xa, wo, xf, wd, slots, hidden), ws, stream)
    log("weight layout: %s" % layout)
    ms = time_steps(step, args.steps, args.warmup, stream, ws_check(plan, ws, "decode step"))
    serial_knob = (info["packed_kind"] == 1) if layout == "packed" else (w.batch < 16)
    if not args.no_serial and serial_knob:
        # the same step with the grid-wide wait per point (serial point order)
        plan.tune("serial_points", 1)
        ms_serial = time_steps(step, args.steps, args.warmup, stream,
                               ws_check(plan, ws, "serial point order"))
        plan.tune("serial_points", 0)
        b_serial = w.projection_bytes_per_step(fmt) / (ms_serial * 1e-3) / 1e9
        b_serial_all = (w.projection_bytes_per_step(fmt) + w.reduce_io_bytes_per_step()) / (ms_serial * 1e-3) / 1e9
        extra["serial_point_order"] = {
            "ms_per_step": round(ms_serial, 5), "tokens_per_s": round(w.batch / (ms_serial * 1e-3), 3),
            "achieved_gbs": round(b_serial, 2), "frac": round(b_serial / HBM_PEAK_GBS, 4),
            "frac_incl_reduce_io": round(b_serial_all / HBM_PEAK_GBS, 4),
            "note": "point j+1 reads its activation only after every column of point j is complete"}
    cpu = None
    if not args.no_cpu_baseline:
        if fmt:
            cpu = cpu_baseline_mx(w, args.rank, fmt, xa, wo, xf, wd, slots, h0, args.cpu_seconds)
        else:
            cpu = cpu_baseline(w, args.rank, xa, wo, xf, wd, slots, h0, args.cpu_seconds)
    config = {"workload": w.name, "hidden": w.hidden, "inter": w.inter, "k_attn": w.k_attn,
              "layers": w.layers, "n_ranks": w.n_ranks, "rank": args.rank, "batch": w.batch,
              "reductions_per_token": 2 * w.layers, "weight_layout": layout,
              "weights": WEIGHT_NAMES[fmt],
              "weight_bytes_per_step": w.weight_bytes_per_step(fmt)}
    extra["traffic"] = measured_traffic("%s/%s/%s" % (w.name, layout, WEIGHT_NAMES[fmt]))
    extra["reduce_io_bytes"] = w.reduce_io_bytes_per_step()
    extra["weight_bytes"] = w.weight_bytes_per_step(fmt)
    if cpu is not None and w.name == workloads.PAGE1.name and not fmt:
        cpu["tiny_single_thread"] = tiny_single_thread()
    plan.close()
    return ms, w.batch, w.projection_bytes_per_step(fmt), kernel, config, cpu, extra


def single_op_run(args, w, plan, info, tune, inputs, ws, stream):
    """One entry point on its own over the stack, weights from HBM:
    "partials" = tp_rowparallel_partials (the 2L partial projections in
    layer order, one call); "partial" = tp_rowparallel_partial and "ring" =
    tp_ring_reduce (ring-order sum of the N partials + residual), once per
    reconciliation point (2L calls per pass, each its own launch);
    "swiglu" = tp_gate_up_swiglu (the stack's column-parallel up
    projections with SwiGLU, one call); "qkv" = tp_qkv_proj (the stack's
    column-parallel mixer input projections, one call)."""
    import torch

    import row_gemv_reduction_amd as tp
    xa, wo, xf, wd, slots, hidden = inputs
    b, H, N, L = w.batch, w.hidden, w.n_ranks, w.layers
    graph_ok = True
    if args.op == "swiglu":
        # the column-parallel up projection of the same stack: gate and up
        # weights [L][H][I/N] each, the layer's full hidden state as x
        from row_gemv_reduction_amd import synth
        C = w.ki_r
        kw = dict(seed=0, workload=w.name, rank=args.rank)
        xin = synth.device_normal((L, b, H), 1.0, torch.bfloat16, tensor="x_ffn_in", **kw)
        wg = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_gate", **kw)
        wu = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_up", **kw)
        act = torch.empty((L, b, C), dtype=torch.bfloat16, device="cuda")

        def step():
            tp.tp_gate_up_swiglu(plan, L, xin, wg, wu, act, ws)
        graph_ok = False  # cooperative launches, issued from C
        # gate and up weights, x and the bf16 activation written
        nbytes = L * (2 * H * C * 2 + b * H * 2 + b * C * 2)
        kernel = ("tp_gate_up_swiglu: the persistent step's tiles (gate and up as the two "
                  "points of each layer) + swiglu_kernel, over as many layers per launch as "
                  "32 MiB of fp32 sums hold")
    elif args.op == "qkv":
        # the column-parallel mixer input projection of the same stack: Q
        # columns = the mixer output's K / N, K and V = QKV_KV_HEADS heads of
        # QKV_HEAD_DIM each, replicated where ranks outnumber them
        from row_gemv_reduction_amd import synth
        C = qkv_cols(w.k_attn, N)
        plan = tp.Plan(H, w.inter, N, b, k_attn=w.k_attn, tune=tune, qkv_cols=C)
        ws = plan.new_workspace()
        kw = dict(seed=0, workload=w.name, rank=args.rank)
        xin = synth.device_normal((L, b, H), 1.0, torch.bfloat16, tensor="x_qkv_in", **kw)
        wq = synth.device_normal((L, H, C), synth.WEIGHT_STD, torch.bfloat16, tensor="w_qkv", **kw)
        qkv = torch.empty((L, b, C), dtype=torch.bfloat16, device="cuda")

        def step():
            tp.tp_qkv_proj(plan, L, xin, wq, qkv, ws)
        graph_ok = False  # cooperative launches, issued from C
        nbytes = L * (H * C * 2 + b * H * 2 + b * C * 2)
        kernel = ("tp_qkv_proj: the persistent step's tiles (two layers as its two points, "
                  "%d columns per rank) + round_bf16_kernel" % C)
    elif args.op == "partials":
        def step():
            tp.tp_rowparallel_partials(plan, L, xa, wo, xf, wd, pstack, ws)
        pstack = torch.empty((L, 2, b, H), dtype=torch.float32, device="cuda")
        nbytes = L * ((w.ka_r + w.ki_r) * H * 2 + b * (w.ka_r + w.ki_r) * 2 + 2 * b * H * 4)
        if tune.get("decode_mode", 0) != 1:
            graph_ok = False  # one cooperative launch per pass
            kernel = ("tp_rowparallel_partials: the persistent step's tiles without ring or "
                      "residual (%s), one launch per pass"
                      % ("decode_step_mfma" if b >= 16 else "decode_step"))
        else:
            kernel = "tp_rowparallel_partials: %s, one launch per point" % (
                "mfma_gemm" if b >= 16 else "valu_gemv")
    elif args.op == "partial":
        def step():
            for l in range(L):
                tp.tp_rowparallel_partial(plan, 0, xa[l], wo[l], slots[l, 0, args.rank], ws)
                tp.tp_rowparallel_partial(plan, 1, xf[l], wd[l], slots[l, 1, args.rank], ws)
        # weights + x slices + the fp32 partials written
        nbytes = L * ((w.ka_r + w.ki_r) * H * 2 + b * (w.ka_r + w.ki_r) * 2 + 2 * b * H * 4)
        path = "MFMA skinny GEMM (mfma_gemm)" if b >= 16 else "VALU GEMV (valu_gemv)"
        kernel = "tp_rowparallel_partial, %s, splits %s, one launch per point" % (path, info["splits"])
    else:
        def step():
            for l in range(L):
                tp.tp_ring_reduce(plan, slots[l, 0], hidden, hidden)
                tp.tp_ring_reduce(plan, slots[l, 1], hidden, hidden)
        # N partials and the residual read, the sum written
        nbytes = 2 * L * (N + 2) * b * H * 4
        kernel = "tp_ring_reduce (ring_reduce_kernel), one launch per point"
    log("op %s: %d launches per pass" % (args.op, 2 * L))
    # Issued one call at a time, the pass measures the host's launch rate
    # (about 10 us per call through the binding); captured once into a HIP
    # graph and replayed, it measures the kernels.
    ms_eager = time_steps(step, args.steps, args.warmup, stream, ws_check(plan, ws, "op " + args.op))
    launches = 1 if not graph_ok else 2 * L
    config = {"workload": w.name, "op": args.op, "hidden": H, "inter": w.inter, "k_attn": w.k_attn,
              "layers": L, "n_ranks": N, "rank": args.rank, "batch": b,
              "launches_per_pass": launches, "weight_layout": "rowmajor"}
    if graph_ok:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        ms = time_steps(graph.replay, args.steps, args.warmup, stream,
                        ws_check(plan, ws, "op %s (graph)" % args.op))
        config.update({"us_per_launch": round(ms * 1e3 / launches, 3),
                       "timing": "HIP graph of the pass, replayed",
                       "us_per_launch_eager": round(ms_eager * 1e3 / launches, 3)})
    else:
        ms = ms_eager
        config.update({"us_per_launch": round(ms * 1e3 / launches, 3),
                       "timing": "eager, launches issued from the library"})
    plan.close()
    return ms, b, nbytes, kernel, config, None, {"traffic": None}


def stream_read_run(args, w):
    """The device's streaming-read ceiling: the library's read probe over as
    many bytes as one decode step of workload w streams (its weight slices),
    at a few grid sizes; the fastest is reported."""
    import torch

    import row_gemv_reduction_amd as tp
    nbytes = w.weight_bytes_per_step()
    nbytes -= nbytes % 16
    buf = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    buf.fill_(1.0)
    best = None
    for wgs in (256, 512, 768, 1024, 2048):
        sink = torch.zeros(wgs, dtype=torch.uint32, device="cuda")
        ms = time_steps(lambda: tp.tp_stream_read_probe(buf, sink), args.steps, args.warmup,
                        torch.cuda.current_stream())
        log("stream read: %d workgroups, %.4f ms, %.1f GB/s" % (wgs, ms, nbytes / ms / 1e6))
        if best is None or ms < best[0]:
            best = (ms, wgs)
    ms, wgs = best
    config = {"workload": w.name, "op": "stream_read", "bytes": nbytes, "workgroups": wgs,
              "timing": "eager, one launch per pass"}
    kernel = ("tp_stream_read_probe (stream_read_kernel: grid-stride 16-byte nontemporal loads, %d "
              "workgroups of 512 threads)" % wgs)
    return ms, 0, nbytes, kernel, config, None, {"traffic": None}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def prefill_run(args, w, tune):
    """The prefill of a w.batch-token prompt through the stack (tp_prefill_layers):
    per point the rank's T x H partial on the matrix cores, its slot, and the
    ring sum + residual fused into the product's epilogue. One launch."""
    import numpy as np
    import torch

    import row_gemv_reduction_amd as tp
    from row_gemv_reduction_amd import synth
    L, T, H, n, rank = w.layers, w.batch, w.hidden, w.n_ranks, args.rank
    plan = tp.Plan(H, w.inter, n, 1, k_attn=w.k_attn, tune=tune)
    kw = dict(seed=0, workload=w.name, rank=rank)
    xa = synth.device_normal((L, T, w.ka_r), 1.0, torch.bfloat16, tensor="x_attn", **kw)
    wo = synth.device_normal((L, w.ka_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw)
    xf = synth.device_normal((L, T, w.ki_r), 1.0, torch.bfloat16, tensor="x_ffn", **kw)
    wd = synth.device_normal((L, w.ki_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_down", **kw)
    slots = synth.device_normal((L, 2, n, T, H), synth.WEIGHT_STD * math.sqrt(w.ki_r), torch.float32,
                                tensor="slots", seed=0, workload=w.name)
    hidden = synth.device_normal((T, H), 1.0, torch.float32, tensor="residual", seed=0, workload=w.name)
    po = torch.empty(tp.prefill_packed_shape(plan, 0, L), dtype=torch.bfloat16, device="cuda")
    pd = torch.empty(tp.prefill_packed_shape(plan, 1, L), dtype=torch.bfloat16, device="cuda")
    tp.tp_prefill_pack_weights(plan, 0, wo, po)
    tp.tp_prefill_pack_weights(plan, 1, wd, pd)
    ws = plan.new_workspace()
    torch.cuda.synchronize()

    def step():
        tp.tp_prefill_layers(plan, L, rank, T, xa, po, xf, pd, slots, hidden, ws)
    ms = time_steps(step, args.steps, args.warmup, torch.cuda.current_stream(), ws_check(plan, ws, "prefill"))
    flops = 2.0 * T * (w.ka_r + w.ki_r) * H * L
    proj = w.projection_bytes_per_step()
    reduce_io = w.reduce_io_bytes_per_step()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = prefill_cpu_baseline(w, rank, xa, wo, xf, wd, slots, hidden, args.cpu_seconds)
    config = {"workload": w.name, "hidden": H, "inter": w.inter, "k_attn": w.k_attn, "layers": L,
              "n_ranks": n, "rank": rank, "tokens": T, "reductions_per_prefill": 2 * L,
              "weight_layout": "packed matrix-core tiles"}
    kernel = ("prefill_step (one cooperative launch: 128 x 256 tiles of every point on the bf16 matrix "
              "cores, ring sum + residual fused into the epilogue)")
    t = ms * 1e-3
    extra = {"mfma": {"achieved_tflops": round(flops / t / 1e12, 2), "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                      "frac": round(flops / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_launch": flops},
             "prefill_bound_note": "at peak the step needs %.2f ms of HBM (projection + ring I/O) and %.2f ms "
                                   "of matrix cores" % ((proj + reduce_io) / 8e12 * 1e3,
                                                         flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e3),
             "reduce_io_bytes": reduce_io, "weight_bytes": w.weight_bytes_per_step(),
             "traffic": measured_traffic("%s/prefill/bf16" % w.name),
             "fused_bytes": proj + reduce_io}
    plan.close()
    return ms, T, proj, kernel, config, cpu, extra


def prefill_cpu_baseline(w, rank, xa, wo, xf, wd, slots, hidden, budget_s):
    """The oracle on a bounded sample of the prefill: the first m tokens of
    the first layer (both points' projections and the ring sums of those
    tokens' payloads), scaled to T tokens and L layers."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    a, o, f, d = bits(xa[0]), bits(wo[0]), bits(xf[0]), bits(wd[0])
    s = slots[0].cpu().numpy()
    h = hidden.cpu().numpy()
    m, spent = 8, 0.0
    while True:
        t0 = time.perf_counter()
        for pt, (x, W) in enumerate(((a, o), (f, d))):
            _, p32 = oracle.partial(x[:m], W, nthreads=cores)
            part = s[pt, :, :m].copy()
            part[rank] = p32
            oracle.ring_reduce(part, h[:m])
        spent = time.perf_counter() - t0
        if spent * 2 > budget_s or m >= w.batch:
            break
        m = min(w.batch, m * 2)
    per_token_layer = spent / m
    return {"value": 1.0 / (per_token_layer * w.layers), "unit": "tokens/s", "cores": cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "the first %d of %d tokens of layer 0 (both points' projections and ring sums), "
                      "%.1f s, scaled to %d layers" % (m, w.batch, spent, w.layers)}


def moe_build(w, rank, copies, seed=0):
    """Inputs of the MoE decode share, `copies` independent layer copies."""
    import torch

    from row_gemv_reduction_amd import synth
    T, H, E, k, I, ep = w.batch, w.hidden, w.n_experts, w.top_k, w.moe_inter, w.ep
    el = E // ep
    layers = []
    for c in range(copies):
        kw = dict(seed=seed, workload=w.name, rank=rank, layer=c)
        layers.append(dict(
            xa=synth.device_normal((T, w.ka_r), 1.0, torch.bfloat16, tensor="x_attn", **kw),
            wo=synth.device_normal((w.ka_r, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_o", **kw),
            logits=synth.device_normal((T, E), 1.0, torch.float32, tensor="logits", seed=seed,
                                       workload=w.name, layer=c),
            u=synth.device_normal((T, k, I), 1.0, torch.bfloat16, tensor="u", **kw),
            we=synth.device_normal((el, I, H), synth.WEIGHT_STD, torch.bfloat16, tensor="w_expert",
                                   **kw)))
    slots = synth.device_normal((copies, 2, w.n_ranks, T, H), synth.WEIGHT_STD * 40, torch.float32,
                                tensor="slots", seed=seed, workload=w.name)
    h0 = synth.device_normal((T, H), 1.0, torch.float32, tensor="residual", seed=seed, workload=w.name)
    torch.cuda.synchronize()
    return layers, slots, h0


def moe_run(args, w, tune):
    import torch

    import row_gemv_reduction_amd as tp
    T, H, E, k, I, ep = w.batch, w.hidden, w.n_experts, w.top_k, w.moe_inter, w.ep
    rank = args.rank
    plan = tp.Plan(H, w.k_attn, w.n_ranks, T, k_attn=w.k_attn, tune=tune,
                   moe=dict(n_experts=E, top_k=k, ep=ep, moe_inter=I, max_tokens=T))
    copies = 3  # 3 x ~400 MB of distinct weights per rotation: more than the 256 MB cache
    layers, slots, h0 = moe_build(w, rank, copies)
    for L in layers:  # load-time packing of the experts and the attention slice (untimed)
        L["wp"] = torch.empty(tp.moe_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
        tp.tp_moe_pack_experts(plan, L["we"], L["wp"])
        del L["we"]
        L["wap"] = torch.empty(tp.moe_attn_packed_shape(plan), dtype=torch.bfloat16, device="cuda")
        tp.tp_moe_pack_attn(plan, L["wo"], L["wap"])
    torch.cuda.synchronize()
    ws = plan.new_workspace()
    hidden = h0.clone()
    se = torch.empty((T, k), dtype=torch.int32, device="cuda")
    sw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    it = [0]
    stream = torch.cuda.current_stream()

    def step():
        # the whole layer share: routing, the attention slice and the
        # rank's experts in one launch, both ring sums in a second
        c = it[0] % copies
        it[0] += 1
        L = layers[c]
        tp.tp_moe_layer_decode(plan, rank, L["logits"], L["xa"], L["wap"], L["u"], L["wp"], se, sw,
                               slots[c, 0], slots[c, 1], hidden, ws)

    ms = time_steps(step, args.steps, args.warmup, stream, ws_check(plan, ws, "MoE layer share"))
    # algorithmic bytes of one layer share (averaged over the rotated copies)
    el = E // ep
    step_bytes = 0
    active_total = 0
    for c in range(copies):
        tp.tp_moe_route(plan, layers[c]["logits"], se, sw)
        sel = se.cpu().numpy()
        local = sel[(sel >= rank * el) & (sel < (rank + 1) * el)]
        active = len(set(local.tolist()))
        active_total += active
        pairs = local.size
        b = (w.ka_r * H * 2 + T * w.ka_r * 2 + T * H * 4                  # attention slice
             + T * E * 4 + T * k * 8                                         # routing
             + active * I * H * 2 + pairs * I * 2 + pairs * H * 8 + T * H * 4  # experts, combine
             + 2 * (w.n_ranks + 2) * T * H * 4)                              # two ring sums
        step_bytes += b
    step_bytes //= copies
    cpu = None
    if not args.no_cpu_baseline:
        cpu = moe_cpu_baseline(w, rank, layers[0], slots, h0, plan, args.cpu_seconds)
    config = {"workload": w.name, "hidden": H, "k_attn": w.k_attn, "n_ranks": w.n_ranks,
              "rank": rank, "tokens": T, "n_experts": E, "top_k": k, "ep": ep, "moe_inter": I,
              "layers": 1, "active_local_experts_mean": active_total / copies,
              "weight_layout": "attention slice and experts packed as MFMA tiles",
              "timing": "eager, tp_moe_layer_decode: two launches per step",
              "weight_copies_rotated": copies}
    kernel = ("tp_moe_layer_decode: moe_layer_kernel (routing, attention slice and expert MFMA "
              "GEMV in one launch) + moe_layer_combine_kernel (local combine, both ring sums)")
    reduce_io = 2 * (w.n_ranks + 2) * T * H * 4
    # both launches' HBM bytes (the ring sums' included), from the counters
    extra = {"reduce_io_bytes": reduce_io, "traffic": measured_traffic("%s/layer/bf16" % w.name)}
    plan.close()
    return ms, T, step_bytes - reduce_io, kernel, config, cpu, extra


def moe_cpu_baseline(w, rank, L, slots, h0, plan, budget_s):
    """The oracle on the same MoE layer share: attention partial, ring sum
    and routing in full; the expert projections + combine on a sample of
    columns sized to the time budget, scaled to all columns (every column
    costs the same)."""
    import numpy as np
    import torch

    import oracle
    cores = len(os.sched_getaffinity(0))

    def bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    H, E, k, ep = w.hidden, w.n_experts, w.top_k, w.ep
    el = E // ep
    xa, wo, u = bits(L["xa"]), bits(L["wo"]), bits(L["u"])
    logits = L["logits"].cpu().numpy()
    s = slots[0].cpu().numpy()
    h = h0.cpu().numpy()
    t0 = time.perf_counter()
    _, p32 = oracle.partial(xa, wo, nthreads=cores)
    s[0, rank] = p32
    oracle.ring_reduce(s[0], h)
    se, sw = oracle.moe_route(logits, k, True)
    t_fixed = time.perf_counter() - t0

    def expert_cols(ncols):
        we = bits(synth_cols(w, rank, ncols))
        t1 = time.perf_counter()
        oracle.moe_partial(se, sw, rank * el, u, we, nthreads=cores)
        return time.perf_counter() - t1

    ncols = 64
    t_cols = expert_cols(ncols)
    want = int(min(H, max(ncols, ncols * max(budget_s - t_fixed, 0.0) / max(t_cols, 1e-6))))
    if want > ncols:
        ncols = want
        t_cols = expert_cols(ncols)
    per_share = t_fixed + t_cols * H / ncols
    # repeat whole shares until the budget is spent, for a stable figure
    reps, spent = 1, t_fixed + t_cols
    while spent < budget_s and ncols == H:
        t0 = time.perf_counter()
        _, p32 = oracle.partial(xa, wo, nthreads=cores)
        oracle.ring_reduce(s[0], h)
        oracle.moe_route(logits, k, True)
        dt = time.perf_counter() - t0 + expert_cols(ncols)
        spent += dt
        reps += 1
        per_share = spent / reps
    return {"value": w.batch / per_share, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "%d run(s) of one layer share: attention partial, ring sum and routing in "
                      "full; expert projections + combine on %d of %d columns, scaled to all "
                      "columns; %.1f s in all" % (reps, ncols, H, spent)}


def synth_cols(w, rank, ncols):
    """The first ncols columns of copy 0's local experts (same seeded draw)."""
    import torch

    from row_gemv_reduction_amd import synth
    el = w.n_experts // w.ep
    full = synth.device_normal((el, w.moe_inter, w.hidden), synth.WEIGHT_STD, torch.bfloat16,
                               tensor="w_expert", seed=0, workload=w.name, rank=rank, layer=0)
    return full[:, :, :ncols].contiguous()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 100 timed steps: the timed region starts on an idle GPU (synchronised),
    # so its fixed start-up cost (the first step's host-side issue, about
    # 14 us) is spread over enough steps to stay below 0.3 % at the smallest
    # stacks
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="workload name (default: page-1 stack, N=4, b=1)")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-serial", action="store_true", help="skip the serial-point-order timing")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--tune", action="append", default=[], help="key=value plan knob")
    ap.add_argument("--weights", default="bf16", choices=["bf16", "mxfp8", "mxfp4", "0", "1", "2"],
                    help="element format of the packed step's weights: bf16, or microscaled "
                         "MXFP8 / MXFP4 (converted once at load, untimed)")
    ap.add_argument("--layout", choices=["auto", "packed", "rowmajor"], default="auto",
                    help="weight layout: pair-strip packed (packed once at load, untimed) or row-major")
    ap.add_argument("--op", choices=["step", "partials", "partial", "ring", "swiglu", "qkv", "stream_read"],
                    default="step",
                    help="what a timed pass runs: the whole decode step (default); the stack's "
                         "2L partial projections in one call (tp_rowparallel_partials); one "
                         "entry point per reconciliation point (tp_rowparallel_partial, "
                         "tp_ring_reduce); the stack's column-parallel up projections with "
                         "SwiGLU (tp_gate_up_swiglu) or QKV projections (tp_qkv_proj); or the "
                         "device's streaming-read ceiling over the step's weight bytes")
    args = ap.parse_args()
    args.weights = {"bf16": 0, "mxfp8": 1, "mxfp4": 2}.get(args.weights, None) \
        if not args.weights.isdigit() else int(args.weights)

    if args.gpus != 1:
        print("bench.py measures one GPU: the N virtual ranks are emulated on a single "
              "MI355X, so --gpus %d is not supported (use --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from row_gemv_reduction_amd import workloads

    w = workloads.ALL[args.workload] if args.workload else workloads.PAGE1
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    tune = {}
    for kv in args.tune:
        k, v = kv.split("=")
        tune[k] = int(v)
    if w.n_experts and args.op not in ("step", "stream_read"):
        raise SystemExit("--op applies to the dense workloads")
    if args.op == "stream_read":
        ms, tokens, step_bytes, kernel, config, cpu, extra = stream_read_run(args, w)
    else:
        run = moe_run if w.n_experts else (prefill_run if w.name == workloads.PREFILL.name else dense_run)
        ms, tokens, step_bytes, kernel, config, cpu, extra = run(args, w, tune)
    if args.copy_calibration:
        copy_calibration()

    tok_s = tokens / (ms * 1e-3)
    achieved = step_bytes / (ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": extra.pop("traffic", None),
        "kernel": kernel, "algorithmic_bytes_per_launch": step_bytes,
    }
    # the emulated ring reductions' I/O, reported beside the projection bytes
    reduce_io = extra.pop("reduce_io_bytes", 0)
    if reduce_io:
        roofline["reduce_io_bytes_per_launch"] = reduce_io
        roofline["frac_incl_reduce_io"] = round((step_bytes + reduce_io) / (ms * 1e-3) / 1e9
                                                / HBM_PEAK_GBS, 4)
    wbytes = extra.pop("weight_bytes", 0)
    if wbytes:
        roofline["weights_only_frac"] = round(wbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    fused = extra.pop("fused_bytes", 0)
    if fused:
        # prefill: the ring I/O is the kernel's own work and dominates its bytes;
        # the HBM roofline takes all of them (the projection-only rate is kept)
        roofline["projection_only_achieved"] = roofline["achieved"]
        roofline["projection_only_frac"] = roofline["frac"]
        roofline["achieved"] = round(fused / (ms * 1e-3) / 1e9, 2)
        roofline["frac"] = round(fused / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        roofline["algorithmic_bytes_per_launch"] = fused
    out = {
        "metric": METRIC, "value": round(tok_s, 3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if not getattr(args, "weights", 0) else "bf16 x " + WEIGHT_NAMES[args.weights],
        "data": "synthetic (seeded N(0,0.02) bf16 weights, N(0,1) activations)",
        "config": config,
        "roofline": roofline,
        "context": {"pages_collective_latency_us": {"fast": 10, "slow": 50},
                    "pages_comm_ms_per_token": {"fast": 1.28, "slow": 6.4},
                    "pages_peer_bandwidth_gbs_gb200": 1800},
    }
    out.update(extra)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
