#!/usr/bin/env python3
"""Throughput of the packed ternary decode product (W1.58A16) on one MI355X.

Headline workload: the Qwen3-8B-class linear stack at M=1 -- 36 distinct
seeded layers x 7 projections (q/o 4096 -> 4096, k/v 4096 -> 1024, gate/up
4096 -> 12288, down 12288 -> 4096; 252 matrices), base-3 five-trits-per-byte
plane 0, group 128, a residual plane on 8 % of groups (1.67 GB of packed
weights, far beyond the 256 MB Infinity Cache).  One step is one decode
token through the whole stack: one plan run (activation layout, residual
pass, then the matrix-core stream kernel over all 252 products).  q/k/v and
gate/up of a layer read the same activations.

value = packed-weight bytes of the stack (every byte of the representation:
plane 0, scales, residual blocks and scales, masks and row pointers;
activations excluded) times the timed steps, divided by the time between
events recorded before the first and after the last timed step.  roofline:
the stream kernel's algorithmic bytes over its average duration, from events
recorded around its launch in every timed step.  cpu_baseline: the oracle's
plain unpack-and-dot (fp64, one thread) over a bounded sample of the same
stack.  extra: the Qwen3-4B-class layer at M=1 (2-bit), the 8B-class layer
at M = 1, 4, 16, 64, 512 (rotating >= 1 GiB of copies), the down-projection
stress layer, the quantizer, the rotation and a plain read probe.
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
STACK = "qwen3_8b_stack"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


PROFILE = os.path.join(ROOT, "profiles", "gemv_b3_kernel_qwen3_8b_stack_m1.txt")


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


def pack_matrix(mat: dict, fmt: int):
    """Upload one synth matrix and pack it on the GPU (tern_pack)."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    nnz = [int(m.sum()) for m in mat["masks"]]
    pm = L.PackedMatrix(mat["n"], mat["k"], mat["group"], mat["planes"], fmt, mat["offset_mode"], nnz)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    masks = dev(np.stack(mat["mask_bits"]).view(np.int32)) if mat["planes"] > 1 else None
    off = dev(mat["offset"]) if mat["offset"] is not None else None
    L.tern_pack(pm, dev(mat["trits"]), dev(mat["scales"]), masks, off)
    return pm


def pack_workload(wl: str, fmt: int, proj: int, layer: int = 0):
    from ternary_weight_only_tern_amd import synth
    mat = synth.workload_matrix(wl, proj, layer)
    return pack_matrix(mat, fmt), mat


def x_for(wl, proj, m, layer=0):
    import torch
    from ternary_weight_only_tern_amd import synth
    x = synth.workload_x(wl, m, proj, layer)
    return torch.from_numpy(x.view(np.uint16)).cuda().view(torch.float16), x


def build_stack8b(layers=LAYERS, threads=8):
    """The 8B-class stack on the GPU: `layers` distinct seeded layers
    (synth.workload_matrix(STACK, proj, layer)) of seven base-3 projections,
    drawn on `threads` host threads (a bounded window in flight) and packed
    in order.  Activations: one draw per layer and distinct input
    (synth.LAYER_INPUT), shared by q/k/v and by gate/up.  Returns (packed
    matrices, x per matrix, y per matrix), layer-major."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from ternary_weight_only_tern_amd import synth
    nproj = len(synth.QWEN3_8B_LAYER)
    jobs = [(layer, proj) for layer in range(layers) for proj in range(nproj)]
    mats = []
    with ThreadPoolExecutor(threads) as ex:
        window = 2 * threads
        futs = [ex.submit(synth.workload_matrix, STACK, proj, layer) for layer, proj in jobs[:window]]
        for i in range(len(jobs)):
            mat = futs[i].result()
            futs[i] = None
            if i + window < len(jobs):
                layer, proj = jobs[i + window]
                futs.append(ex.submit(synth.workload_matrix, STACK, proj, layer))
            mats.append(pack_matrix(mat, synth.FMT_B3))
            del mat
    xs, yl = [], []
    for layer in range(layers):
        xin = {inp: x_for(STACK, inp, 1, layer)[0] for inp in sorted(set(synth.LAYER_INPUT))}
        for proj in range(nproj):
            xs.append(xin[synth.LAYER_INPUT[proj]])
            yl.append(torch.empty((1, mats[layer * nproj + proj].n), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    return mats, xs, yl


def stream_kernel_bytes(mats, xs):
    """Algorithmic bytes of one launch of the base-3 stream kernel at M=1:
    plane 0 and its scales of every product, the residual sums it adds (FP32
    per row of products with residual planes), y (FP16), and the slot-ordered
    activations once per distinct input (33 four-slot chunks of 8 bytes per
    128-wide group)."""
    from ternary_weight_only_tern_amd import lib as L
    total = 0
    for pm in mats:
        total += pm.n * L.tern_row_stride(pm.k, pm.group, pm.fmt) + pm.n * (pm.k // pm.group) * 2
        total += (4 * pm.n if pm.planes > 1 else 0) + 2 * pm.n
    seen = {}
    for pm, x in zip(mats, xs):
        seen[x.data_ptr()] = (pm.k // pm.group) * 33 * 8
    return total + sum(seen.values())


EAGER = False  # --eager: launch the steps directly instead of replaying a graph
LAST_REPLAYS_MS = []  # event times of the last time_graph call's replays (one per rotation)


def time_eager(step_fns, steps, warmup, stream):
    import torch
    per = len(step_fns)
    LAST_REPLAYS_MS[:] = []  # no replays: callers fall back to the mean
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


MIN_REPLAYS = 30  # every graph-timed figure is the median of at least this many replays
SETTLE_S = 0.5    # untimed headline runs after the warm-up, in seconds (clocks reach their steady state)


def replay_stats(per):
    """Per-step seconds from the last time_graph call's replays (each of `per`
    steps): median, min and max over the replays, and their count."""
    ms = sorted(LAST_REPLAYS_MS)
    if not ms:
        return dict(median_s=None, min_s=None, max_s=None, replays=0)
    return dict(median_s=float(np.median(ms)) / 1e3 / per, min_s=ms[0] / 1e3 / per, max_s=ms[-1] / 1e3 / per,
                replays=len(ms))


def bench_layer4b(args, stream, fmt=0):
    """Qwen3-4B-class layer, M=1, 2-bit: 36 byte copies of the layer rotated
    (1.07 GB), one grouped launch per step, replayed from a HIP graph."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
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
    steps = LAYERS * max(MIN_REPLAYS, (args.steps + LAYERS - 1) // LAYERS)
    fns = [(lambda p=p: p.run(stream.cuda_stream)) for p in plans]
    wall, gpu, _ = time_graph(fns, steps, LAYERS, stream)
    step_s = gpu / steps
    median_step_s = float(np.median(LAST_REPLAYS_MS)) / 1e3 / len(fns) if LAST_REPLAYS_MS else step_s
    del plans, layers
    return dict(layer_bytes=layer_bytes, steps=steps, wall_s=wall, gpu_s=gpu, step_s=step_s, median_step_s=median_step_s,
                replays=len(LAST_REPLAYS_MS), gbs=layer_bytes / step_s / 1e9,
                mats=mats, base=base, xs=xs, weights=sum(pm.n * pm.k for pm in base))


def bench_stack8b(args, stream, mats, xs, ys):
    """The headline: exactly args.steps tokens through the stack, one plan
    run each, launched directly on `stream`; events around every run's
    stream-kernel launch give per-step and per-kernel times."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    stack_bytes = sum(pm.nbytes() for pm in mats)
    plan = L.Plan(mats, xs, ys)
    cs = stream.cuda_stream
    steps = args.steps
    with torch.cuda.stream(stream):
        for _ in range(max(args.warmup, 1)):
            plan.run(cs)
        torch.cuda.synchronize()
        # settle: after the stack's CPU-side build the GPU has idled for
        # seconds and its clocks are down; untimed runs continue until
        # SETTLE_S of work has passed since the warm-up began, so that the
        # timed steps see the steady state whatever --warmup is (measured:
        # 485 us/token over 20 steps after 5 warm-up runs, 417 once settled)
        settle_runs, t_w = 0, time.perf_counter()
        while time.perf_counter() - t_w < SETTLE_S:
            for _ in range(20):
                plan.run(cs)
            settle_runs += 20
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        before = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        after = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
        for e in before + after + [start]:  # create the events before timing
            e.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(steps):
            plan.run_events(before[i], after[i], cs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    total_s = start.elapsed_time(after[-1]) / 1e3
    step_ms = [start.elapsed_time(after[0])] + [after[i - 1].elapsed_time(after[i]) for i in range(1, steps)]
    kern_ms = [before[i].elapsed_time(after[i]) for i in range(steps)]
    bits = [L.tern_bits(pm) for pm in mats]
    wts = [pm.n * pm.k for pm in mats]
    bpw = {key: round(sum(b[key] * w for b, w in zip(bits, wts)) / sum(wts), 4) for key in ("info", "plane", "storage")}
    return dict(stack_bytes=stack_bytes, steps=steps, wall_s=wall, total_s=total_s, step_s=total_s / steps,
                settle_runs=settle_runs,
                step_ms=step_ms, kern_ms=kern_ms, kern_bytes=stream_kernel_bytes(mats, xs), bpw=bpw,
                weights=sum(wts), plan=plan)


def time_plan(plan, steps, warmup, stream):
    """Mean step time of a plan launched directly on `stream`, events around
    the timed steps."""
    import torch
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            plan.run(stream.cuda_stream)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            plan.run(stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / steps


def bench_stack8b_rotated(stream, mats, xs, ys, steps=200):
    """The headline stack with a rotation on every distinct input of every
    layer (one seeded 128 x 128 block-diagonal R per layer and input: 216 MB
    of rotation blocks per token), folded into the activation preparation of
    one rotated plan; beside the same plan without rotations."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    rng = np.random.default_rng(4242)
    rot_of, rots = {}, []
    for x, pm in zip(xs, mats):
        if x.data_ptr() not in rot_of:
            R = synth.draw_rotation(rng, pm.k // 128, 128)
            rot_of[x.data_ptr()] = torch.from_numpy(R.view(np.uint16)).cuda().view(torch.float16)
        rots.append(rot_of[x.data_ptr()])
    rbytes = sum(r.numel() * 2 for r in rot_of.values())
    plan_r = L.Plan(mats, xs, ys, rots=rots, rot_block=128)
    plan_p = L.Plan(mats, xs, ys)
    torch.cuda.synchronize()
    t_r = time_plan(plan_r, steps, 10, stream)
    t_p = time_plan(plan_p, steps, 10, stream)
    del plan_r, plan_p, rot_of, rots
    return dict(us_per_token=round(t_r * 1e6, 2), us_per_token_unrotated=round(t_p * 1e6, 2),
                rotation_bytes=rbytes, steps=steps)


def bench_layer4b_rotated(stream, steps=720):
    """The 4B-class layer (2-bit, M=1) with its four distinct inputs (q/k/v
    and gate/up share one each) rotated by 128 x 128 blocks inside the
    decode launch (its first workgroups rotate; tern_plan_launches is 1),
    beside the same layer unrotated; 36 byte copies rotated."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    base, xs, ys, xin = [], [], [], {}
    for proj in range(len(synth.QWEN3_4B_LAYER)):
        pm, _ = pack_workload("qwen3_4b_layer", 0, proj)
        base.append(pm)
        src = synth.LAYER_INPUT[proj]
        if src not in xin:
            xin[src] = x_for("qwen3_4b_layer", src, 1)[0]
        xs.append(xin[src])
        ys.append(torch.empty((1, pm.n), dtype=torch.float16, device="cuda"))
    rng = np.random.default_rng(4243)
    rot_of = {}
    for x, pm in zip(xs, base):
        if x.data_ptr() not in rot_of:
            R = synth.draw_rotation(rng, pm.k // 128, 128)
            rot_of[x.data_ptr()] = torch.from_numpy(R.view(np.uint16)).cuda().view(torch.float16)
    rots = [rot_of[x.data_ptr()] for x in xs]
    layers = [base] + [[clone_packed(pm) for pm in base] for _ in range(LAYERS - 1)]
    out = {}
    launches = {}
    for name, kw in (("rotated", dict(rots=rots, rot_block=128)), ("unrotated", {})):
        plans = [L.Plan(layer, xs, ys, **kw) for layer in layers]
        launches[name] = plans[0].launches()
        fns = [(lambda p=p: p.run(stream.cuda_stream)) for p in plans]
        wall, gpu, _ = time_graph(fns, steps, LAYERS, stream)
        out[name] = round(gpu / steps * 1e6, 3)
        del plans, fns
    del layers
    return dict(us_per_layer=out["rotated"], us_per_layer_unrotated=out["unrotated"],
                launches=launches["rotated"], launches_unrotated=launches["unrotated"],
                rotation_bytes=sum(r.numel() * 2 for r in rot_of.values()), steps=steps)


def bench_stack8b_graph(stream, plan):
    """The same plan replayed from a HIP graph (three tokens per replay)."""
    per = 3
    wall, gpu, _ = time_graph([lambda: plan.run(stream.cuda_stream)] * per, 30 * per, per, stream)
    return dict(step_s=gpu / (30 * per), replays=30)


SWEEP_BYTES = 1 << 30  # rotate at least this many bytes of distinct layer copies


def bench_layer8b(args, stream, m, fmt=1):
    """One Qwen3-8B-class layer (seven projections, one plan) at m activation
    rows, over as many byte copies of the layer as make SWEEP_BYTES (each
    copy its own plan, rotated, so that the weights come from HBM, not the
    Infinity Cache); replayed from one HIP graph per rotation."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    from ternary_weight_only_tern_amd import synth
    base, xs, ys = [], [], []
    for proj in range(len(synth.QWEN3_8B_LAYER)):
        pm, _ = pack_workload("qwen3_8b_layer", fmt, proj)
        xd, _ = x_for("qwen3_8b_layer", synth.LAYER_INPUT[proj], m)
        base.append(pm)
        xs.append(xd)
        ys.append(torch.empty((m, pm.n), dtype=torch.float16, device="cuda"))
    nbytes = sum(pm.nbytes() for pm in base)
    copies = max(1, -(-SWEEP_BYTES // nbytes))
    layers = [base] + [[clone_packed(pm) for pm in base] for _ in range(copies - 1)]
    plans = [L.Plan(layer, xs, ys) for layer in layers]
    torch.cuda.synchronize()
    fns = [(lambda p=p: p.run(stream.cuda_stream)) for p in plans]
    steps = copies * max(MIN_REPLAYS, args.steps // (20 * copies))
    wall, gpu, _ = time_graph(fns, steps, copies, stream)
    rs = replay_stats(copies)
    step_s = rs["median_s"] or gpu / steps
    flops = sum(2.0 * m * pm.n * pm.k for pm in base)
    del plans, layers
    return dict(us_per_layer=step_s * 1e6, gbs=nbytes / step_s / 1e9, tflops=flops / step_s / 1e12, steps=steps,
                copies=copies, rotated_bytes=copies * nbytes, replays=rs["replays"],
                us_min=(rs["min_s"] or step_s) * 1e6, us_max=(rs["max_s"] or step_s) * 1e6)


def bench_stack8b_launches(stream, mats, xs, ys):
    """The headline stack as 252 single-product launches (one plan per
    matrix) replayed from one HIP graph per token, beside the one-launch
    plan."""
    import torch
    from ternary_weight_only_tern_amd import lib as L
    plans = [L.Plan([pm], [x], [y]) for pm, x, y in zip(mats, xs, ys)]
    nbytes = sum(pm.nbytes() for pm in mats)
    torch.cuda.synchronize()

    def token():
        for p in plans:
            p.run(stream.cuda_stream)
    steps = 4
    wall, gpu, _ = time_graph([token], steps, 2, stream)
    step_s = gpu / steps
    del plans
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
    steps = STRESS_COPIES * max(MIN_REPLAYS, args.steps // (4 * STRESS_COPIES))
    wall, gpu, _ = time_graph(fns, steps, STRESS_COPIES, stream)
    rs = replay_stats(STRESS_COPIES)
    step_s = rs["median_s"] or gpu / steps
    nbytes = pm.nbytes()
    del plans, copies
    return dict(us=round(step_s * 1e6, 2), gbs=round(nbytes / step_s / 1e9, 1),
                hbm_frac=round(nbytes / step_s / 1e9 / HBM_PEAK_GBS, 4), bytes=nbytes, steps=steps,
                replays=rs["replays"], us_min=round((rs["min_s"] or step_s) * 1e6, 2),
                us_max=round((rs["max_s"] or step_s) * 1e6, 2))


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
    steps = per * max(MIN_REPLAYS, args.steps // 100 // per)
    wall, gpu, _ = time_graph([step] * per, steps, per, stream)
    rs = replay_stats(per)
    step_s = rs["median_s"] or gpu / steps
    io_bytes = nw * 2 + nw * 2 + sum(n * (k // 128) * 2 * 3 + n * ((k // 128 + 31) // 32) * 4 for _, _, _, _, _, n, k in items)
    return dict(ms_per_layer=step_s * 1e3, weights_per_s=nw / step_s, gbs=io_bytes / step_s / 1e9, steps=steps,
                weights=nw, io_bytes=io_bytes, replays=rs["replays"])


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
    per = 48  # steps captured per graph replay (a replay's own submission cost is then shared by 48 short launches)
    steps = per * max(MIN_REPLAYS, args.steps // 10 // per)
    wall, gpu, _ = time_graph([step] * per, steps, per, stream)
    rs = replay_stats(per)
    step_s = rs["median_s"] or gpu / steps
    return dict(us_per_layer=step_s * 1e6, gbs=nbytes / step_s / 1e9, bytes=nbytes, steps=steps,
                replays=rs["replays"])


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


def cpu_baseline(budget_s=12.0):
    """The oracle's unpack-and-dot (fp64, one thread) over the seven
    projections of the stack's layer 0, repeated until about budget_s seconds
    of CPU work: GB/s over the same byte count as the GPU figure."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    from ternary_weight_only_tern_amd import synth
    mats = [synth.workload_matrix(STACK, p, 0) for p in range(len(synth.QWEN3_8B_LAYER))]
    packed = [O.pack(m["trits"], m["scales"], m["mask_bits"], m["offset"], m["group"], synth.FMT_B3) for m in mats]
    del mats
    xs = [synth.workload_x(STACK, 1, synth.LAYER_INPUT[p], 0) for p in range(len(packed))]
    nbytes, done, nmat = 0, 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            for pk, x in zip(packed, xs):
                O.gemv_packed(pk, x)
                nbytes += O.bits(pk)["total_bytes"]
                nmat += 1
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
    dt = time.perf_counter() - t0
    return dict(value=round(nbytes / dt / 1e9, 6), unit="GB/s", cores=1, kind="oracle",
                sample=f"{done} pass(es) over the {len(packed)} projections of layer 0 of the Qwen3-8B-class stack "
                       f"(base-3, M=1; {nmat} products and {nbytes} packed bytes in all), fp64 unpack-and-dot, "
                       f"1 thread, {dt:.1f} s",
                tokens_per_s_equiv=round(nbytes / dt / (LAYERS * sum(O.bits(pk)["total_bytes"] for pk in packed)), 8))


def cpu_baseline_4b(mats, budget_s=6.0):
    """The oracle's unpack-and-dot on one thread over whole Qwen3-4B-class
    layers (2-bit), for the 4B-class figure."""
    from threadpoolctl import threadpool_limits
    import oracle as O
    from ternary_weight_only_tern_amd import synth
    packed = [O.pack(m["trits"], m["scales"], m["mask_bits"], m["offset"], m["group"], 0) for m in mats]
    xs = [synth.workload_x("qwen3_4b_layer", 1, p) for p in range(len(mats))]
    nbytes, done = 0, 0
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
                sample=f"{done} pass(es) over the 7 projections of one Qwen3-4B-class layer (2-bit, M=1), "
                       f"fp64 unpack-and-dot, 1 thread, {dt:.1f} s")


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1080, help="timed steps (tokens through the stack)")
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--skip-extra", action="store_true", help="only the headline measurement")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true", help="direct launches instead of graph replay (extras)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 256 MiB device copy 8 times (HBM counter calibration)")
    ap.add_argument("--stack8b-only", action="store_true",
                    help="only the headline stack (profiling); prints its result, no JSON line")
    ap.add_argument("--gemm512-only", action="store_true",
                    help="only the M=512 matrix-core layer (profiling); no JSON line")
    ap.add_argument("--layer4b-only", action="store_true",
                    help="only the 4B-class 2-bit layer at M=1 (profiling); no JSON line")
    ap.add_argument("--layer4b-rotated-only", action="store_true",
                    help="only the 4B-class 2-bit layer at M=1 with and without its inputs rotated inside the "
                         "decode launch (profiling); no JSON line")
    ap.add_argument("--quantize-only", action="store_true",
                    help="only the quantizer on a 4B-class layer (profiling); no JSON line")
    ap.add_argument("--rotate-only", action="store_true",
                    help="only the activation rotation of a 4B-class layer's M=1 inputs (profiling); no JSON line")
    ap.add_argument("--layer8b-only", type=int, metavar="M", default=0,
                    help="only the base-3 8B-class layer at M activation rows (profiling); no JSON line")
    ap.add_argument("--stress-only", metavar="FMT:M", default="",
                    help="only the stress down-projection, FMT 2bit or b3, at M rows (profiling); no JSON line")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the product shards by output rows with no communication; see the design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
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

    if args.gemm512_only or args.layer8b_only > 0:
        m = 512 if args.gemm512_only else args.layer8b_only
        q = bench_layer8b(args, stream, m)
        log(f"bench: 8B-class layer base-3 M={m}: {q['us_per_layer']:.1f} us, {q['gbs']:.1f} GB/s, "
            f"{q['tflops']:.1f} TFLOP/s ({q['copies']} copies rotated)")
        return
    if args.stress_only:
        fname, m = args.stress_only.split(":")
        q = bench_stress(args, stream, {"2bit": 0, "b3": 1}[fname], int(m))
        log(f"bench: stress down-projection {fname} M={m}: {q['us']:.2f} us, {q['gbs']:.1f} GB/s")
        return
    if args.layer4b_only:
        r = bench_layer4b(args, stream)
        log(f"bench: 4B-class layer {r['step_s']*1e6:.2f} us/step, {r['gbs']:.1f} GB/s")
        return
    if args.layer4b_rotated_only:
        r4 = bench_layer4b_rotated(stream, steps=max(LAYERS, args.steps // LAYERS * LAYERS))
        log(f"bench: 4B-class layer with rotations {r4['us_per_layer']:.2f} us (without "
            f"{r4['us_per_layer_unrotated']:.2f}), {r4['launches']} launch(es) per layer")
        return
    if args.quantize_only:
        qz = bench_quantize(args, stream)
        log(f"bench: quantize 4B-class layer {qz['ms_per_layer']:.3f} ms, {qz['weights_per_s']/1e9:.2f} G weights/s")
        return
    if args.rotate_only:
        ro = bench_rotate(args, stream)
        log(f"bench: rotation of a 4B-class layer's M=1 inputs {ro['us_per_layer']:.2f} us, {ro['gbs']:.1f} GB/s")
        return

    log("bench: drawing and packing the 8B-class stack (36 distinct layers)")
    t0 = time.perf_counter()
    mats, xs, ys = build_stack8b()
    log(f"bench: stack ready in {time.perf_counter() - t0:.1f} s")
    r = bench_stack8b(args, stream, mats, xs, ys)
    med = float(np.median(r["step_ms"]))
    kern_s = float(np.mean(r["kern_ms"])) / 1e3
    log(f"bench: stack {r['stack_bytes']} B, {r['step_s']*1e6:.1f} us/token (median {med*1e3:.1f}), "
        f"{r['stack_bytes'] / r['step_s'] / 1e9:.1f} GB/s; stream kernel {kern_s*1e6:.1f} us "
        f"(event mean over {r['steps']} launches) for {r['kern_bytes']} algorithmic bytes = "
        f"{r['kern_bytes'] / kern_s / 1e9:.1f} GB/s")
    if args.stack8b_only:
        return
    extra = {"headline_bpw": r["bpw"],
             "headline_tokens_per_s_equiv": round(1.0 / r["step_s"], 2),
             "headline_step_us": {"median": round(med * 1e3, 2), "min": round(min(r["step_ms"]) * 1e3, 2),
                                  "max": round(max(r["step_ms"]) * 1e3, 2), "timed_steps": r["steps"]},
             "headline_wall_s": round(r["wall_s"], 4),
             "headline_settle": {"untimed_runs_after_warmup": r["settle_runs"], "seconds": SETTLE_S,
                                 "why": "steady clocks before the timed steps (the stack is built on the CPU first)"},
             "headline_stream_kernel_us": {"mean": round(kern_s * 1e6, 2),
                                           "median": round(float(np.median(r["kern_ms"])) * 1e3, 2),
                                           "min": round(min(r["kern_ms"]) * 1e3, 2),
                                           "max": round(max(r["kern_ms"]) * 1e3, 2)}}
    if not args.skip_extra:
        gr = bench_stack8b_graph(stream, r["plan"])
        extra["qwen3_8b_stack_m1_b3_graph"] = dict(us_per_token=round(gr["step_s"] * 1e6, 2),
                                                   gbs=round(r["stack_bytes"] / gr["step_s"] / 1e9, 1),
                                                   replays=gr["replays"], tokens_per_replay=3)
        log(f"bench: stack from a graph {gr['step_s']*1e6:.1f} us/token")
        rot = bench_stack8b_rotated(stream, mats, xs, ys)
        extra["qwen3_8b_stack_m1_b3_rotated"] = dict(rot, note="rotation folded into the activation preparation "
                                                     "(tern_plan_create_rotated), one 128x128 block-diagonal R per "
                                                     "layer and distinct input")
        log(f"bench: stack with rotations {rot['us_per_token']:.1f} us/token (without {rot['us_per_token_unrotated']:.1f})")
        s8l = bench_stack8b_launches(stream, mats, xs, ys)
        extra["qwen3_8b_stack_m1_b3_252_launches"] = dict(us_per_token=round(s8l["step_s"] * 1e6, 2),
                                                          gbs=round(s8l["gbs"], 1),
                                                          hbm_frac=round(s8l["gbs"] / HBM_PEAK_GBS, 4),
                                                          tokens_per_s_equiv=round(s8l["tok_s"], 2),
                                                          steps=s8l["steps"])
        log(f"bench: stack as 252 launches {s8l['gbs']:.1f} GB/s")
    del r["plan"]
    del mats, xs, ys
    torch.cuda.empty_cache()
    cpu4 = None
    if not args.skip_extra:
        log("bench: 4B-class layer (2-bit, M=1)")
        l4 = bench_layer4b(args, stream)
        bits = [L.tern_bits(pm) for pm in l4["base"]]
        wts = [pm.n * pm.k for pm in l4["base"]]
        extra["qwen3_4b_layer_m1_2bit"] = dict(
            bytes=l4["layer_bytes"], us_per_step=round(l4["step_s"] * 1e6, 3),
            median_us_per_step=round(l4["median_step_s"] * 1e6, 3), gbs=round(l4["gbs"], 1), replays=l4["replays"],
            hbm_frac=round(l4["gbs"] / HBM_PEAK_GBS, 4), steps=l4["steps"],
            tokens_per_s_equiv=round(1.0 / (LAYERS * l4["step_s"]), 1),
            bpw={key: round(sum(b[key] * w for b, w in zip(bits, wts)) / sum(wts), 4)
                 for key in ("info", "plane", "storage")},
            note="one grouped launch per layer; 36 byte copies of the layer rotated")
        log(f"bench: 4B-class layer {l4['step_s']*1e6:.2f} us/step, {l4['gbs']:.1f} GB/s")
        r4 = bench_layer4b_rotated(stream)
        extra["qwen3_4b_layer_m1_2bit_rotated"] = dict(r4, note="the layer's four distinct inputs rotated inside "
                                                       "the decode launch (one plan, one launch)")
        log(f"bench: 4B-class layer with rotations {r4['us_per_layer']:.2f} us (without {r4['us_per_layer_unrotated']:.2f})")
        sweep = {}
        for m in (1, 4, 16, 64, 512):
            q = bench_layer8b(args, stream, m)
            sweep[f"m{m}"] = dict(us_per_layer=round(q["us_per_layer"], 2), gbs=round(q["gbs"], 1),
                                  tflops=round(q["tflops"], 2), copies_rotated=q["copies"], replays=q["replays"],
                                  us_min=round(q["us_min"], 2), us_max=round(q["us_max"], 2))
            if m == 512:
                sweep[f"m{m}"]["mfma_frac"] = round(q["tflops"] / F16_MFMA_PEAK_TFS, 4)
            log(f"bench: 8B-class layer base-3 M={m}: {q['us_per_layer']:.1f} us, {q['gbs']:.1f} GB/s, "
                f"{q['tflops']:.1f} TFLOP/s")
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
                                                replays=qz["replays"],
                                                kernel="quantize_kernel<128>: sixteen lanes per (row, group)")
        log(f"bench: quantize 4B-class layer {qz['ms_per_layer']:.3f} ms")
        rt = bench_rotate(args, stream)
        extra["rotate_m1_qwen3_4b_inputs"] = dict(us_per_layer=round(rt["us_per_layer"], 3), gbs=round(rt["gbs"], 1),
                                                  bytes=rt["bytes"], steps=rt["steps"], replays=rt["replays"],
                                                  note="one launch for K = 2560, 4096, 9728; 128 x 128 blocks")
        log(f"bench: rotate M=1 inputs of a 4B-class layer {rt['us_per_layer']:.2f} us")
        big = bench_read_probe(stream, 1 << 30, 2)
        extra["read_probe"] = dict(gbs_1gib=round(big["gbs"], 1), kernel="tern_read_probe (plain streaming read)")
        log(f"bench: read probe {big['gbs']:.1f} GB/s (1 GiB)")
        if not args.skip_cpu:
            cpu4 = cpu_baseline_4b(l4["mats"])
            extra["cpu_oracle_qwen3_4b_layer"] = cpu4
            host = cpu_host_dense(l4["mats"])
            extra["cpu_host_dense_qwen3_4b_layer"] = host
            cq = cpu_quantize_baseline()
            extra["cpu_oracle_quantize"] = cq
            log(f"bench: cpu 4B-class {cpu4['value']:.4f} GB/s, host dense {host['value']:.4f} GB/s")
    cpu = None
    if not args.skip_cpu:
        log("bench: cpu baseline (oracle) on the stack")
        cpu = cpu_baseline()
        log(f"bench: cpu {cpu['value']:.5f} GB/s")

    value = r["stack_bytes"] / r["step_s"] / 1e9
    achieved = r["kern_bytes"] / kern_s / 1e9
    out = {
        "metric": "ternary GEMV packed-weight GB/s (% HBM peak) at M=1; TFLOP/s at M=512",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": r["steps"],
        "warmup": args.warmup,
        "ms_per_step": r["step_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 x, base-3 trits (fp32 accumulation)",
        "data": "synthetic (seeded; Qwen3-8B-class shapes, random trits, scales and masks)",
        "config": {"workload": "qwen3-8b-class linear stack, M=1: 36 distinct layers x 7 projections (252 matrices), "
                               "base-3 five trits per byte, group 128, residual plane on 8% of groups; "
                               "one plan run per token",
                   "stack_bytes": r["stack_bytes"], "weights": r["weights"], "hbm_frac": round(value / HBM_PEAK_GBS, 4),
                   "tokens_per_s_equiv": round(1.0 / r["step_s"], 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": profiled_traffic(),
                     "kernel": "gemv_b3_kernel<128,1,true> (base-3 stream decode on the matrix cores, "
                               "all 252 products in one launch)",
                     "launch_us": round(kern_s * 1e6, 3), "bytes_per_launch": r["kern_bytes"]},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
