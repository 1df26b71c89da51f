#!/usr/bin/env python3
"""Throughput of the packed ternary decode product (W1.58A16) on one MI355X.

Headline workload: the Qwen3-4B-class decoder layer at M=1 (q 2560->4096,
k/v 2560->1024, o 4096->2560, gate/up 2560->9728, down 9728->2560; group
128; a residual plane on 10 % of groups; 2-bit planes).  One step is one
decode token through one layer: the seven products in one grouped launch.
The model has 36 layers (arXiv 2609.01962 §3.1), so the timed steps walk 36
distinct, HBM-resident layer copies (1.07 GB; more than the 256 MB Infinity
Cache) the way a decode does; steps are replayed from a HIP graph.

value = packed-weight bytes of the step (every byte of the representation:
planes, scales, residual blocks and metadata; activations excluded) divided
by the step time.  Extra measurements on the same line: the Qwen3-8B-class
36 x 7 base-3 stack at M=1 (tokens/s-equivalent) and the 8B-class layer at
M=512 through the MFMA path (TFLOP/s).  The CPU baseline is the oracle's
plain unpack-and-dot on one thread over a bounded sample of the workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
F16_MFMA_PEAK_TFS = 2500.0   # MI355X dense FP16 MFMA, TFLOP/s
LAYERS = 36


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROFILE = os.path.join(ROOT, "profiles", "gemv_mfma_2bit_qwen3_4b_layer_m1.txt")


def profiled_traffic(path=PROFILE):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when the
    summary is missing or was taken on a different kernel source."""
    import hashlib
    try:
        fields = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith(" "))
        sha, src = fields["kernel_source_sha256"].split()[0], fields["kernel_source_sha256"].split("(")[1].rstrip(")\n ")
        if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, IndexError, ValueError):
        return None


def clone_packed(pm):
    from ternary_weight_only_tern_amd import lib as L
    c = L.PackedMatrix.__new__(L.PackedMatrix)
    c.__dict__.update(pm.__dict__)
    c.plane0 = pm.plane0.clone()
    c.scale0 = pm.scale0.clone()
    c.mask = [t.clone() for t in pm.mask]
    c.rowptr = [t.clone() for t in pm.rowptr]
    c.blocks = [t.clone() for t in pm.blocks]
    c.rscale = [t.clone() for t in pm.rscale]
    c.offset = None if pm.offset is None else pm.offset.clone()
    return c


def pack_workload(wl: str, fmt: int, proj: int, layer: int = 0):
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    mat = synth.workload_matrix(wl, proj, layer)
    nnz = [int(m.sum()) for m in mat["masks"]]
    pm = L.PackedMatrix(mat["n"], mat["k"], mat["group"], mat["planes"], fmt, mat["offset_mode"], nnz)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    masks = dev(np.stack(mat["mask_bits"]).view(np.int32)) if mat["planes"] > 1 else None
    off = dev(mat["offset"]) if mat["offset"] is not None else None
    L.tern_pack(pm, dev(mat["trits"]), dev(mat["scales"]), masks, off)
    return pm, mat


def x_for(wl, proj, m, layer=0):
    import torch
    from ternary_weight_only_tern_amd import synth
    x = synth.workload_x(wl, m, proj, layer)
    return torch.from_numpy(x.view(np.uint16)).cuda().view(torch.float16), x


EAGER = False  # --eager: launch the steps directly instead of replaying a graph
LAST_REPLAYS_MS = []  # event times of the last time_graph call's replays (one per rotation)


def time_eager(step_fns, steps, warmup, stream):
    import torch
    per = len(step_fns)
    with torch.cuda.stream(stream):
        for i in range(max(warmup, per)):
            step_fns[i % per]()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record(stream)
        for i in range(steps):
            step_fns[i % per]()
        e.record(stream)
        torch.cuda.synchronize()
    return time.perf_counter() - t0, s.elapsed_time(e) / 1e3, None


def time_graph(step_fns, steps, warmup, stream):
    """Capture one call of every step function into a HIP graph, replay it so
    that exactly `steps` steps run; returns (total seconds, per-step seconds
    from events around each replayed step group)."""
    import torch
    if EAGER:
        return time_eager(step_fns, steps, warmup, stream)
    per = len(step_fns)
    assert steps % per == 0, "steps must be a multiple of the rotation length"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for f in step_fns:  # eager warm-up before capture
            f()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for f in step_fns:
                f()
    torch.cuda.synchronize()
    reps_w = max(1, warmup // per)
    reps = steps // per
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    with torch.cuda.stream(stream):  # replay on the stream the events are recorded on
        for _ in range(reps_w):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s, e in evs:
            s.record(stream)
            g.replay()
            e.record(stream)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    LAST_REPLAYS_MS[:] = [s.elapsed_time(e) for s, e in evs]
    gpu = sum(LAST_REPLAYS_MS) / 1e3
    return wall, gpu, g


def bench_layer4b(args, stream):
    """Qwen3-4B-class layer, M=1, 36 distinct layer copies."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    fmt = 0 if args.fmt == "2bit" else 1
    base, xs, ys, mats = [], [], [], []
    for proj in range(len(synth.QWEN3_4B_LAYER)):
        pm, mat = pack_workload("qwen3_4b_layer", fmt, proj)
        base.append(pm)
        mats.append(mat)
        xd, _ = x_for("qwen3_4b_layer", proj, 1)
        xs.append(xd)
        ys.append(torch.empty((1, pm.n), dtype=torch.float16, device="cuda"))
    layer_bytes = sum(pm.nbytes() for pm in base)
    layers = [base] + [[clone_packed(pm) for pm in base] for _ in range(LAYERS - 1)]
    plans = [L.Plan(layer, xs, ys) for layer in layers]
    torch.cuda.synchronize()
    steps = max(LAYERS, (args.steps + LAYERS - 1) // LAYERS * LAYERS)
    fns = [(lambda p=p: p.run(stream.cuda_stream)) for p in plans]
    wall, gpu, _ = time_graph(fns, steps, args.warmup, stream)
    step_s = gpu / steps
    median_step_s = float(np.median(LAST_REPLAYS_MS)) / 1e3 / len(fns) if LAST_REPLAYS_MS else step_s
    # one kernel launch per step: the average launch duration over the timed
    # region is the step time
    launch_s = step_s
    return dict(layer_bytes=layer_bytes, steps=steps, wall_s=wall, gpu_s=gpu, step_s=step_s, median_step_s=median_step_s,
                replays=len(LAST_REPLAYS_MS),
                gbs=layer_bytes / step_s / 1e9, launch_s=launch_s, launch_gbs=layer_bytes / launch_s / 1e9,
                mats=mats, base=base, xs=xs, weights=sum(pm.n * pm.k for pm in base))


def bench_stack8b(args, stream):
    """Qwen3-8B-class 36 x 7 stack, base-3, M=1: one grouped launch per token."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    base, xs = [], []
    for proj in range(len(synth.QWEN3_8B_LAYER)):
        pm, _ = pack_workload("qwen3_8b_stack", 1, proj)
        base.append(pm)
        xd, _ = x_for("qwen3_8b_stack", proj, 1)
        xs.append(xd)
    mats, xl, yl = [], [], []
    for layer in range(LAYERS):
        for proj, pm in enumerate(base):
            mats.append(pm if layer == 0 else clone_packed(pm))
            xl.append(xs[proj])
            yl.append(torch.empty((1, pm.n), dtype=torch.float16, device="cuda"))
    stack_bytes = sum(pm.nbytes() for pm in mats)
    bits = [L.tern_bits(pm) for pm in base]
    wts = [pm.n * pm.k for pm in base]
    bpw = {key: round(sum(b[key] * w for b, w in zip(bits, wts)) / sum(wts), 4) for key in ("info", "plane", "storage")}
    plan = L.Plan(mats, xl, yl)
    torch.cuda.synchronize()
    per = 3  # steps captured per graph replay
    steps = max(per, args.steps // 20 // per * per)
    wall, gpu, _ = time_graph([lambda: plan.run(stream.cuda_stream)] * per, steps, per, stream)
    step_s = gpu / steps
    return dict(stack_bytes=stack_bytes, steps=steps, step_s=step_s, gbs=stack_bytes / step_s / 1e9,
                tok_s=1.0 / step_s, bpw=bpw)


def bench_gemm512(args, stream):
    """Qwen3-8B-class layer at M=512 through the matrix-core product (base-3):
    the seven projections in one grouped launch (a plan)."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    m = 512
    items = []
    for proj in range(len(synth.QWEN3_8B_LAYER)):
        pm, _ = pack_workload("qwen3_8b_layer", 1, proj)
        xd, _ = x_for("qwen3_8b_layer", proj, m)
        y = torch.empty((m, pm.n), dtype=torch.float16, device="cuda")
        items.append((pm, xd, y))
    flops = sum(2.0 * m * pm.n * pm.k for pm, _, _ in items)
    plan = L.Plan([pm for pm, _, _ in items], [xd for _, xd, _ in items], [y for _, _, y in items])
    step = lambda: plan.run(stream.cuda_stream)
    per = 6  # steps captured per graph replay
    steps = max(per, args.steps // 20 // per * per)
    wall, gpu, _ = time_graph([step] * per, steps, per, stream)
    step_s = gpu / steps
    return dict(flops=flops, steps=steps, step_s=step_s, tflops=flops / step_s / 1e12)


def bench_layer8b(args, stream, m, fmt=1):
    """One Qwen3-8B-class layer (seven projections, one plan) at m activation
    rows: the batched variant's sweep points below M=512."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    pms, xs, ys = [], [], []
    for proj in range(len(synth.QWEN3_8B_LAYER)):
        pm, _ = pack_workload("qwen3_8b_layer", fmt, proj)
        xd, _ = x_for("qwen3_8b_layer", proj, m)
        pms.append(pm)
        xs.append(xd)
        ys.append(torch.empty((m, pm.n), dtype=torch.float16, device="cuda"))
    plan = L.Plan(pms, xs, ys)
    per = 6  # steps captured per graph replay (a replay's own launch cost is then shared)
    steps = max(per, args.steps // 20 // per * per)
    wall, gpu, _ = time_graph([lambda: plan.run(stream.cuda_stream)] * per, steps, per, stream)
    step_s = gpu / steps
    nbytes = sum(pm.nbytes() for pm in pms)
    flops = sum(2.0 * m * pm.n * pm.k for pm in pms)
    return dict(us_per_layer=step_s * 1e6, gbs=nbytes / step_s / 1e9, tflops=flops / step_s / 1e12, steps=steps)


def bench_stack8b_launches(args, stream):
    """The same 8B-class stack as 252 single-product launches (one plan per
    matrix) replayed from one HIP graph per token, beside the one-launch
    plan."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    base, xs = [], []
    for proj in range(len(synth.QWEN3_8B_LAYER)):
        pm, _ = pack_workload("qwen3_8b_stack", 1, proj)
        base.append(pm)
        xd, _ = x_for("qwen3_8b_stack", proj, 1)
        xs.append(xd)
    plans, nbytes = [], 0
    for layer in range(LAYERS):
        for proj, pm in enumerate(base):
            c = pm if layer == 0 else clone_packed(pm)
            y = torch.empty((1, c.n), dtype=torch.float16, device="cuda")
            plans.append(L.Plan([c], [xs[proj]], [y]))
            nbytes += c.nbytes()
    torch.cuda.synchronize()
    steps = max(2, args.steps // 40)

    def token():
        for p in plans:
            p.run(stream.cuda_stream)
    wall, gpu, _ = time_graph([token], steps, 2, stream)
    step_s = gpu / steps
    return dict(stack_bytes=nbytes, steps=steps, step_s=step_s, gbs=nbytes / step_s / 1e9, tok_s=1.0 / step_s)


STRESS_COPIES = 57  # 57 x 18.9 MB (2-bit) > 1 GiB: beyond the Infinity Cache


def bench_stress(args, stream, fmt, m):
    """Down-projection stress matrix (K=12288, N=4096; three planes on the
    same 20 % of groups; per-row offsets; log-normal scales; Student-t x) at
    m rows: one single-product plan per distinct copy, rotated."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    pm, _ = pack_workload("down_proj_stress", fmt, 0)
    xd, _ = x_for("down_proj_stress", 0, m)
    copies = [pm] + [clone_packed(pm) for _ in range(STRESS_COPIES - 1)]
    y = torch.empty((m, pm.n), dtype=torch.float16, device="cuda")
    plans = [L.Plan([c], [xd], [y]) for c in copies]
    fns = [(lambda p=p: p.run(stream.cuda_stream)) for p in plans]
    steps = STRESS_COPIES * max(1, args.steps // (4 * STRESS_COPIES))
    wall, gpu, _ = time_graph(fns, steps, STRESS_COPIES, stream)
    step_s = gpu / steps
    nbytes = pm.nbytes()
    del plans, copies
    return dict(us=round(step_s * 1e6, 2), gbs=round(nbytes / step_s / 1e9, 1),
                hbm_frac=round(nbytes / step_s / 1e9 / HBM_PEAK_GBS, 4), bytes=nbytes, steps=steps)


def bench_quantize(args, stream):
    """The quantizer front-end on a 4B-class layer: FP16 weights of the seven
    projections (unit normal; the method is scale-equivariant) with a 10 %
    salience mask -> trit planes, scales and offsets, one launch per
    projection, 15 refinement iterations."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    rng = np.random.default_rng(2024)
    items, nw = [], 0
    for _, k, n in synth.QWEN3_4B_LAYER:
        w = synth.draw_x(rng, n, k, "normal")
        _, mb = synth.draw_mask(rng, n, k // 128, 0.10)
        wd = torch.from_numpy(w.view(np.uint16)).cuda()
        md = torch.from_numpy(mb.view(np.int32)).cuda()
        t = torch.empty((2, n, k), dtype=torch.int8, device="cuda")
        sc = torch.empty((2, n, k // 128), dtype=torch.float16, device="cuda")
        of = torch.empty((n, k // 128), dtype=torch.float16, device="cuda")
        items.append((wd, md, t, sc, of, n, k))
        nw += n * k
    lib = L.load()

    def step():
        for wd, md, t, sc, of, n, k in items:
            L.check(lib.tern_quantize(wd.data_ptr(), n, k, 128, md.data_ptr(), 15, t.data_ptr(), sc.data_ptr(),
                                      of.data_ptr(), stream.cuda_stream))
    per = 2  # steps captured per graph replay
    steps = max(per, args.steps // 100 // per * per)
    wall, gpu, _ = time_graph([step] * per, steps, per, stream)
    step_s = gpu / steps
    io_bytes = nw * 2 + nw * 2 + sum(n * (k // 128) * 2 * 3 + n * ((k // 128 + 31) // 32) * 4 for _, _, _, _, _, n, k in items)
    return dict(ms_per_layer=step_s * 1e3, weights_per_s=nw / step_s, gbs=io_bytes / step_s / 1e9, steps=steps,
                weights=nw, io_bytes=io_bytes)


def bench_rotate(args, stream):
    """The activation rotation at M=1 for the three inputs of a 4B-class
    layer (hidden 2560 for q/k/v and gate/up, attention output 4096 for o,
    MLP intermediate 9728 for down), 128 x 128 blocks, one batched launch
    per step."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    rng = np.random.default_rng(7)
    items, nbytes = [], 0
    for k in (2560, 4096, 9728):
        R = torch.from_numpy(synth.draw_rotation(rng, k // 128, 128).view(np.uint16)).cuda()
        x = torch.from_numpy(synth.draw_x(rng, 1, k, "normal").view(np.uint16)).cuda()
        o = torch.empty_like(x)
        items.append((R, x, o, k))
        nbytes += k * 128 * 2 + 2 * k * 2
    Rs, xs, outs = [it[0] for it in items], [it[1] for it in items], [it[2] for it in items]

    def step():
        L.tern_rotate_batched(Rs, xs, outs, stream.cuda_stream)
    per = 12  # steps captured per graph replay (a replay's own launch cost is then shared)
    steps = max(per, args.steps // 10 // per * per)
    wall, gpu, _ = time_graph([step] * per, steps, per, stream)
    step_s = gpu / steps
    return dict(us_per_layer=step_s * 1e6, gbs=nbytes / step_s / 1e9, bytes=nbytes, steps=steps)


def cpu_quantize_baseline(budget_s=6.0):
    """The quantizer oracle (vectorized numpy FP32, one thread) on the 4B-class
    k projection's shape (1024 x 2560), repeated for about budget_s seconds."""
    from threadpoolctl import threadpool_limits
    import oracle.quant_oracle as Q
    from ternary_weight_only_tern_amd import synth
    rng = np.random.default_rng(2024)
    _, k, n = synth.QWEN3_4B_LAYER[1]
    w = synth.draw_x(rng, n, k, "normal")
    _, mb = synth.draw_mask(rng, n, k // 128, 0.10)
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            Q.quantize(w, mb, 128)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return dict(weights_per_s=done * n * k / dt, cores=1, kind="oracle",
                sample=f"{done} quantization(s) of a {n} x {k} projection, 1 thread, {dt:.1f} s")


def bench_read_probe(stream, nbytes, copies):
    """Attainable read bandwidth: the library's plain streaming-read probe
    over `copies` distinct buffers of nbytes each, one launch per buffer."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    bufs = [torch.ones(nbytes // 4, dtype=torch.float32, device="cuda") for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    fns = [(lambda b=b: L.tern_read_probe(b, sink, stream.cuda_stream)) for b in bufs]
    steps = copies * max(1, 360 // copies)
    wall, gpu, _ = time_graph(fns, steps, copies, stream)
    step_s = gpu / steps
    del bufs
    return dict(bytes=nbytes, us=step_s * 1e6, gbs=nbytes / step_s / 1e9)


def cpu_baseline(mats, fmt, budget_s=12.0):
    """The oracle's unpack-and-dot on one thread, over whole layers of the
    same workload until about budget_s seconds of CPU work."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    from ternary_weight_only_tern_amd import synth
    packed = [O.pack(m["trits"], m["scales"], m["mask_bits"], m["offset"], m["group"], fmt) for m in mats]
    xs = [synth.workload_x("qwen3_4b_layer", 1, p) for p in range(len(mats))]
    nbytes = 0
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            for pk, x in zip(packed, xs):
                O.gemv_packed(pk, x)
                nbytes += O.bits(pk)["total_bytes"]
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{done} pass(es) over the 7 projections of one Qwen3-4B-class layer "
                       f"({'2-bit' if fmt == 0 else 'base-3'}, M=1), fp64 unpack-and-dot, 1 thread, {dt:.1f} s")


def cpu_host_dense(mats, budget_s=6.0):
    """Host baseline beside the strict oracle: the oracle's fp64 dense
    dequantization and a numpy (BLAS) product on every thread the BLAS pool
    has, over whole layers of the same workload."""
    from threadpoolctl import threadpool_info
    import oracle as O
    from ternary_weight_only_tern_amd import synth
    xs = [synth.workload_x("qwen3_4b_layer", 1, p) for p in range(len(mats))]
    layer_bytes = sum(O.bits(O.pack(mt["trits"], mt["scales"], mt["mask_bits"], mt["offset"], mt["group"], 0))["total_bytes"]
                      for mt in mats)
    nbytes, done = 0, 0
    t0 = time.perf_counter()
    while True:
        for mt, x in zip(mats, xs):
            masks = [O.mask_bool(mb, mt["k"] // mt["group"]) for mb in mt["mask_bits"]]
            w = O.dequant(mt["trits"], mt["scales"], masks, mt["offset"], mt["offset_mode"], mt["group"])
            _ = np.asarray(x, dtype=np.float64) @ w.T
        nbytes += layer_bytes
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=nbytes / dt / 1e9, unit="GB/s", cores=threads, kind="host dense fp64 dequantize + BLAS",
                cpu_model=model, cpu_count=os.cpu_count(),
                sample=f"{done} pass(es) over the 7 projections of one Qwen3-4B-class layer (2-bit bytes), {dt:.1f} s")


def cpu_stack_extrapolated(runs=3):
    """The strict oracle (unpack-and-dot, one thread) on one layer of the
    8B-class base-3 stack, median of `runs` timings, times 36 layers (the
    whole stack would take minutes, so this figure is extrapolated)."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    from ternary_weight_only_tern_amd import synth
    mats = [synth.workload_matrix("qwen3_8b_stack", p) for p in range(len(synth.QWEN3_8B_LAYER))]
    packed = [O.pack(m["trits"], m["scales"], m["mask_bits"], m["offset"], m["group"], 1) for m in mats]
    xs = [synth.workload_x("qwen3_8b_stack", 1, p) for p in range(len(mats))]
    layer_bytes = sum(O.bits(pk)["total_bytes"] for pk in packed)
    times = []
    with threadpool_limits(limits=1):
        for _ in range(runs):
            t0 = time.perf_counter()
            for pk, x in zip(packed, xs):
                O.gemv_packed(pk, x)
            times.append(time.perf_counter() - t0)
    layer_s = float(np.median(times))
    tok_s = LAYERS * layer_s
    return dict(us_per_token=tok_s * 1e6, tokens_per_s_equiv=1.0 / tok_s, gbs=LAYERS * layer_bytes / tok_s / 1e9,
                cores=1, kind="oracle", layer_runs_s=[round(t, 3) for t in times],
                note="one layer timed (median of runs), times 36 layers: extrapolated")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1080, help="timed steps (rounded up to a multiple of 36)")
    ap.add_argument("--warmup", type=int, default=72)
    ap.add_argument("--fmt", choices=["2bit", "b3"], default="2bit")
    ap.add_argument("--skip-extra", action="store_true", help="only the headline measurement")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="direct launches instead of graph replay (profiling)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 8 times (HBM counter calibration)")
    ap.add_argument("--gemm512-only", action="store_true",
                    help="only the M=512 matrix-core layer (profiling); prints its result, no JSON line")
    ap.add_argument("--stack8b-only", action="store_true",
                    help="only the 8B-class base-3 stack at M=1 (profiling); prints its result, no JSON line")
    ap.add_argument("--quantize-only", action="store_true",
                    help="only the quantizer on a 4B-class layer (profiling); prints its result, no JSON line")
    ap.add_argument("--rotate-only", action="store_true",
                    help="only the activation rotation of a 4B-class layer's M=1 inputs (profiling); no JSON line")
    ap.add_argument("--layer8b-only", type=int, metavar="M", default=0,
                    help="only the base-3 8B-class layer at M activation rows (profiling); no JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the product shards by output rows with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(8):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("bench: copied 8 x 256 MiB")
        return
    global EAGER
    EAGER = args.eager
    from ternary_weight_only_tern_amd import lib as L
    L.load()
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()

    if args.gemm512_only:
        g = bench_gemm512(args, stream)
        log(f"bench: M=512 layer {g['step_s']*1e6:.1f} us, {g['tflops']:.1f} TFLOP/s")
        return
    if args.quantize_only:
        qz = bench_quantize(args, stream)
        log(f"bench: quantize 4B-class layer {qz['ms_per_layer']:.3f} ms, {qz['weights_per_s']/1e9:.2f} G weights/s")
        return
    if args.rotate_only:
        ro = bench_rotate(args, stream)
        log(f"bench: rotation of a 4B-class layer's M=1 inputs {ro['us_per_layer']:.2f} us, {ro['gbs']:.1f} GB/s")
        return
    if args.layer8b_only > 0:
        q = bench_layer8b(args, stream, args.layer8b_only)
        log(f"bench: 8B-class layer base-3 M={args.layer8b_only}: {q['us_per_layer']:.1f} us, {q['gbs']:.1f} GB/s, "
            f"{q['tflops']:.1f} TFLOP/s")
        return
    if args.stack8b_only:
        s8 = bench_stack8b(args, stream)
        log(f"bench: 8B-class stack {s8['step_s']*1e6:.1f} us per token, {s8['gbs']:.1f} GB/s")
        return

    log("bench: packing the 4B-class layer")
    r = bench_layer4b(args, stream)
    log(f"bench: layer {r['layer_bytes']} B, {r['step_s']*1e6:.2f} us/step, {r['gbs']:.1f} GB/s; "
        f"single launch {r['launch_s']*1e6:.2f} us = {r['launch_gbs']:.1f} GB/s")
    bits = [L.tern_bits(pm) for pm in r["base"]]
    wts = [pm.n * pm.k for pm in r["base"]]
    extra = {"headline_bpw": {key: round(sum(b[key] * w for b, w in zip(bits, wts)) / sum(wts), 4)
                              for key in ("info", "plane", "storage")},
             "headline_tokens_per_s_equiv": 1.0 / (LAYERS * r["step_s"]),
             "headline_median_step_us": round(r["median_step_s"] * 1e6, 3),
             "headline_timed_replays": r["replays"]}
    if not args.skip_extra:
        log("bench: 8B-class stack")
        s8 = bench_stack8b(args, stream)
        extra["qwen3_8b_stack_m1_b3"] = dict(bytes=s8["stack_bytes"], us_per_token=s8["step_s"] * 1e6,
                                             gbs=s8["gbs"], hbm_frac=s8["gbs"] / HBM_PEAK_GBS,
                                             tokens_per_s_equiv=s8["tok_s"], steps=s8["steps"], bpw=s8["bpw"])
        log(f"bench: stack {s8['gbs']:.1f} GB/s, {s8['tok_s']:.0f} tok/s-eq")
        s8l = bench_stack8b_launches(args, stream)
        extra["qwen3_8b_stack_m1_b3_252_launches"] = dict(us_per_token=s8l["step_s"] * 1e6, gbs=s8l["gbs"],
                                                          hbm_frac=s8l["gbs"] / HBM_PEAK_GBS,
                                                          tokens_per_s_equiv=s8l["tok_s"], steps=s8l["steps"])
        log(f"bench: stack as 252 launches {s8l['gbs']:.1f} GB/s, {s8l['tok_s']:.0f} tok/s-eq")
        log("bench: M=512 MFMA layer")
        g = bench_gemm512(args, stream)
        extra["qwen3_8b_layer_m512_b3"] = dict(tflops=g["tflops"], mfma_frac=g["tflops"] / F16_MFMA_PEAK_TFS,
                                               us_per_layer=g["step_s"] * 1e6, steps=g["steps"])
        log(f"bench: M=512 {g['tflops']:.1f} TFLOP/s")
        sweep = {}
        for m in (1, 4, 16, 64):
            q = bench_layer8b(args, stream, m)
            sweep[f"m{m}"] = dict(us_per_layer=round(q["us_per_layer"], 2), gbs=round(q["gbs"], 1),
                                  tflops=round(q["tflops"], 2))
            log(f"bench: 8B-class layer base-3 M={m}: {q['us_per_layer']:.1f} us, {q['gbs']:.1f} GB/s")
        extra["qwen3_8b_layer_b3_sweep"] = sweep
        stress = {}
        for fmt, fname in ((0, "2bit"), (1, "b3")):
            for m in (1, 8):
                q = bench_stress(args, stream, fmt, m)
                stress[f"{fname}_m{m}"] = q
                log(f"bench: stress down-projection {fname} M={m}: {q['us']:.2f} us, {q['gbs']:.1f} GB/s")
        extra["stress_down_proj_k12288"] = stress
        qz = bench_quantize(args, stream)
        extra["quantize_qwen3_4b_layer"] = dict(ms_per_layer=round(qz["ms_per_layer"], 4),
                                                weights_per_s=qz["weights_per_s"], gbs=round(qz["gbs"], 1),
                                                hbm_frac=round(qz["gbs"] / HBM_PEAK_GBS, 4), steps=qz["steps"],
                                                kernel="quantize_kernel<128>: sixteen lanes per (row, group)")
        log(f"bench: quantize 4B-class layer {qz['ms_per_layer']:.3f} ms, {qz['weights_per_s']/1e9:.2f} G weights/s")
        rt = bench_rotate(args, stream)
        extra["rotate_m1_qwen3_4b_inputs"] = dict(us_per_layer=round(rt["us_per_layer"], 3), gbs=round(rt["gbs"], 1),
                                                  bytes=rt["bytes"], steps=rt["steps"],
                                                  note="one launch for K = 2560, 4096, 9728; 128 x 128 blocks")
        log(f"bench: rotate M=1 inputs of a 4B-class layer {rt['us_per_layer']:.2f} us")
        # attainable read bandwidth on this machine: a plain reduction over 1 GiB
        # buffers, and over 36 buffers of the headline layer's size
        big = bench_read_probe(stream, 1 << 30, 2)
        lay = bench_read_probe(stream, r["layer_bytes"] // 256 * 256, LAYERS)
        extra["read_probe"] = dict(gbs_1gib=round(big["gbs"], 1), gbs_layer_size=round(lay["gbs"], 1),
                                   us_layer_size=round(lay["us"], 2), kernel="tern_read_probe (plain streaming read)",
                                   headline_frac_of_layer_size_read=round(r["gbs"] / lay["gbs"], 4))
        log(f"bench: read probe {big['gbs']:.1f} GB/s (1 GiB), {lay['gbs']:.1f} GB/s ({lay['bytes']} B per launch)")
    cpu = None
    if not args.skip_cpu:
        log("bench: cpu baseline (oracle)")
        cpu = cpu_baseline(r["mats"], 0 if args.fmt == "2bit" else 1)
        log(f"bench: cpu {cpu['value']:.4f} GB/s")
        host = cpu_host_dense(r["mats"])
        extra["cpu_host_dense"] = host
        log(f"bench: cpu host dense {host['value']:.4f} GB/s on {host['cores']} threads")
        if not args.skip_extra:
            cq = cpu_quantize_baseline()
            extra["cpu_oracle_quantize"] = cq
            log(f"bench: cpu quantize {cq['weights_per_s']/1e6:.2f} M weights/s")
            cs = cpu_stack_extrapolated()
            extra["cpu_oracle_qwen3_8b_stack_extrapolated"] = cs
            log(f"bench: cpu oracle 8B-class stack {cs['tokens_per_s_equiv']:.4f} tok/s-eq (extrapolated)")

    out = {
        "metric": "ternary GEMV packed-weight GB/s (% HBM peak) at M=1; TFLOP/s at M=512",
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": r["step_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 x, 2-bit trits" if args.fmt == "2bit" else "fp16 x, base-3 trits",
        "data": "synthetic (seeded; Qwen3-4B-class shapes, random trits/scales/masks)",
        "config": {"workload": "qwen3-4b-class decoder layer, M=1, 7 projections in one grouped launch, "
                               "36 distinct layer copies rotated",
                   "format": args.fmt, "group": 128, "residual_frac": 0.10, "layer_bytes": r["layer_bytes"],
                   "weights_per_step": r["weights"]},
        "roofline": {"bound": "hbm", "achieved": round(r["launch_gbs"], 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["launch_gbs"] / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(),
                     "kernel": "gemv_mfma_kernel<128,1> (2-bit, G=128, M=1): one grouped launch per layer",
                     "launch_us": round(r["launch_s"] * 1e6, 3),
                     "bytes_per_launch": r["layer_bytes"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
