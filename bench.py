"""Benchmark of the MoE normal-mode hot path on one MI355X.

One step = layout + dispatch + combine over one batch of seeded
synthetic input already resident in HBM (default: the DeepSeek-V3-shaped
prefill, S=4096 H=7168 E=256 P=8 K=8, bf16). Prints ONE JSON line with the
whole-step throughput in GB/s of algorithmic bytes, tokens/s, per-kernel event
timings, the roofline of the dominant kernel and the CPU oracle timed on the
host cores as a reported baseline.

The layout is moe_layout_ws (two kernels; in bf16 the second also writes the
pack's plan into the workspace), the dispatch moe_dispatch_planned (the
planned pack kernel alone, reading that plan) and the combine moe_combine, each
checked once per input set into a pre-validated call (moe_plan_layout_ws,
moe_plan_dispatch_planned, moe_plan_combine) and launched by one moe_plan_run:
the same kernels as the Python calls without their per-call argument checks and
marshalling, which extras.eager_binding_calls times.
extras.three_launch_layout_dispatch_ws times the step with moe_layout (three
kernels) + moe_dispatch_ws (plan kernel + pack kernel), and the token-order
moe_dispatch is timed in extras.dispatch_token_order.

Cache state: the timed steps cycle over --rotate (default 8) copies of the batch
at distinct addresses, so each step reads its inputs from HBM rather than from
the 256 MB memory-side cache (eight copies of x alone are 470 MB at S=4096); extras.warm_same_buffers repeats the timing with
one set of buffers. ceilings holds the library's own 1 GiB probes (write-only
fill, read-only stream, copy); each kernel also reports its bandwidth against
the ceiling of its own read/write mix, (r + w) / (r / read + w / fill), and
against the measured copy (frac_copy_ceiling).
extras.fused_layout_dispatch times the step with the layout and the pack in one
moe_layout_dispatch call (one kernel for decode-sized tables) through the
binding, and at decode sizes extras.plans_fused_layout_dispatch the same two
calls as pre-validated calls.
extras.graph_replay times the same step captured in HIP graphs (one per input
set): the device time per step without Python's launch overhead, which is what
bounds the event timings at decode sizes. extras.graph_replay_fused_layout_dispatch
does the same with the layout and the pack in one moe_layout_dispatch call (one
kernel for decode-sized tables); at decode sizes extras.graph_replay_16_steps_per_graph
puts 16 steps in one graph so that the replay's own launch cost is shared.

Timing: value and ms_per_step come from the K timed steps with nothing recorded
between the kernels (wall clock between two device synchronisations). The same
K steps then run again with an event before and after every call; kernels
holds those event statistics per call (layout, dispatch = the pack kernel, combine)
and for the sums layout+dispatch and layout+dispatch+combine, each with its
bytes, GB/s, fraction of 8 TB/s, tokens/s and fraction of its pattern ceiling.
Each event adds a few microseconds to the interval it bounds, so the event
figures are upper bounds on the kernel durations; ms_per_step_with_events is the
step time of that second pass; roofline.achieved uses its figure for the
dominant call. kernels_isolated then times each call alone, K launches back to
back over the same rotated inputs with one event at each end.

Algorithmic bytes (what the method must move; zero padding and the window
reservation are not traffic):
  layout   = topk_idx + is_token_in_rank + counts + slot bases + slot_idx + both prefix matrices
  dispatch = x + slot_idx + N * (payload + 12-byte triple [+ 4-byte scale for fp8])
  combine  = slot_idx + topk_weights + N * 2H (gathered rows) + y
with N the number of valid (token, k) entries.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1..5] [--rotate R]
       [--quant workload|none|fp8|int8] [--no-extras] [--no-cpu-baseline]
"""

import argparse
import dataclasses
import json
import os
import resource
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD specification
METRIC = "dispatch+combine GB/s and tokens/s on 1 MI355X; % of HBM peak (S=4096,H=7168,K=8)"
ROOT = os.path.dirname(os.path.abspath(__file__))


def algorithmic_bytes(w, C, n_valid):
    S, H, K, E, P = w.S, w.H, w.K, w.E, w.P
    layout = 4 * S * K + S * P + 4 * (P + E) + 4 * (P + 1 + E + 1) + 4 * S * K + 4 * (P + E) * C
    payload = 2 * H if w.quant == 0 else H
    dispatch = 2 * S * H + 4 * S * K + n_valid * (payload + 12 + (4 if w.quant else 0))
    combine = 4 * S * K + 4 * S * K + n_valid * 2 * H + 2 * S * H
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def code_digest(names):
    """sha256 of the kernel sources `names` (files under combine_moe_layout_02_amd/csrc, in order)
    with their comments removed, so that an edit to a comment does not retire the counters."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "combine_moe_layout_02_amd", "csrc", name), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(line.rstrip() for line in text.splitlines() if line.strip()).encode())
    return h.hexdigest()


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, if still current."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        rec = data.get(kernel_key)
        if not rec:
            return None
        if code_digest(rec["sources"]) != rec["code_sha256"]:
            return None  # the kernel changed since the counters were taken
        return rec["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(w, C, inp, expert_out, n_valid, min_seconds=10.0, max_reps=25):
    """The oracle as it stands, on the host cores: full steps of the same workload, repeated
    until about min_seconds of wall time have accumulated."""
    import oracle

    ru0 = resource.getrusage(resource.RUSAGE_SELF)
    t0 = time.perf_counter()
    reps = 0
    stage_s = {"layout": 0.0, "dispatch": 0.0, "combine": 0.0}
    while reps < max_reps and (reps == 0 or time.perf_counter() - t0 < min_seconds):
        ta = time.perf_counter()
        lay = oracle.layout(inp["topk_idx"], w.E, w.P, C)
        tb = time.perf_counter()
        oracle.dispatch_slots(inp["x"], lay["slot_idx"], w.quant, 0)
        tc = time.perf_counter()
        oracle.combine(expert_out, lay["slot_idx"], inp["topk_weights"])
        td = time.perf_counter()
        stage_s["layout"] += tb - ta
        stage_s["dispatch"] += tc - tb
        stage_s["combine"] += td - tc
        reps += 1
    wall = time.perf_counter() - t0
    ru1 = resource.getrusage(resource.RUSAGE_SELF)
    cpu = (ru1.ru_utime - ru0.ru_utime) + (ru1.ru_stime - ru0.ru_stime)
    total = sum(algorithmic_bytes(w, C, n_valid).values()) * reps
    return {
        "value": round(total / wall / 1e9, 3),
        "unit": "GB/s",
        "cores": max(1, round(cpu / wall)),
        "kind": "oracle",
        "sample": f"{reps} full steps (layout+dispatch+combine) of {w.describe()}, {wall:.1f} s wall, "
                  f"{cpu:.1f} s cpu, {reps * w.S / wall:.0f} tokens/s; numpy on one thread; host has "
                  f"{os.cpu_count()} logical cpus ({cpu_model()})",
        "stage_ms": {k: round(1e3 * v / reps, 3) for k, v in stage_s.items()},
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "cpu model unknown"


def ceilings(torch, moe, dev, mib=1024, iters=10):
    """The library's bandwidth probes over 1 GiB buffers (write-only fill, read-only stream, copy
    of read + write bytes), GB/s: the practical ceilings of the three access patterns next to the
    8 TB/s specification."""
    n = mib * 2**20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    moe.moe_probe_fill(src)
    out = {}
    for name, fn, nbytes in (("fill", lambda: moe.moe_probe_fill(dst), n),
                             ("read", lambda: moe.moe_probe_read(src, sink), n),
                             ("copy", lambda: moe.moe_probe_copy(src, dst), 2 * n)):
        fn()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(nbytes * iters / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    return out


def rw_split(w, C, n_valid):
    """(read, write) algorithmic bytes of each call, for the pattern ceilings."""
    S, H, K, E, P = w.S, w.H, w.K, w.E, w.P
    payload = 2 * H if w.quant == 0 else H
    return {
        "layout": (4 * S * K, S * P + 4 * (P + E) + 4 * (P + 1 + E + 1) + 4 * S * K + 4 * (P + E) * C),
        "dispatch": (2 * S * H + 4 * S * K, n_valid * (payload + 12 + (4 if w.quant else 0))),
        "combine": (8 * S * K + n_valid * 2 * H, 2 * S * H),
    }


def pattern_ceiling(ceil, r, wbytes):
    """Bandwidth ceiling of a call that reads r and writes wbytes bytes, if reads and writes share
    the memory one after the other at the probes' read and fill rates."""
    if not ceil:
        return None
    return (r + wbytes) / (r / ceil["read"] + wbytes / ceil["fill"])


def time_fused_eager(args, torch, moe, w, C, sets, lay, window, y, total_bytes):
    """The step with the layout and the pack through moe_layout_dispatch, launched eagerly like the
    timed steps (W warm-up, K steps between two device synchronisations, nothing in between)."""
    def step(i):
        x, topk, wts, eo = sets[i % len(sets)]
        moe.moe_layout_dispatch(topk, w.E, w.P, C, x, window, w.quant, 0, out=lay)
        moe.moe_combine(eo, lay.slot_idx, wts, y=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    return {"ms_per_step": round(ms, 4), "value": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.S / (ms * 1e-3), 1)}


def time_three_launch_eager(args, torch, moe, w, C, sets, lay, window, y, total_bytes, ws):
    """The step with moe_layout (three kernels) and moe_dispatch_ws (plan kernel + pack kernel), launched
    eagerly like the timed steps."""
    def step(i):
        x, topk, wts, eo = sets[i % len(sets)]
        moe.moe_layout(topk, w.E, w.P, C, out=lay)
        moe.moe_dispatch_ws(x, lay.slot_idx, window, ws, w.quant, 0)
        moe.moe_combine(eo, lay.slot_idx, wts, y=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    return {"ms_per_step": round(ms, 4), "value": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.S / (ms * 1e-3), 1)}


def time_eager_binding(args, torch, moe, w, C, sets, lay, window, y, total_bytes, lws):
    """The step's three calls through the Python binding (moe_layout_ws, moe_dispatch_planned,
    moe_combine: argument checks and marshalling on every call), launched like the timed steps."""
    def step(i):
        x, topk, wts, eo = sets[i % len(sets)]
        moe.moe_layout_ws(topk, w.E, w.P, C, lws, w.quant, out=lay)
        moe.moe_dispatch_planned(x, lay.slot_idx, window, lws, C, w.quant, 0)
        moe.moe_combine(eo, lay.slot_idx, wts, y=y)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    return {"ms_per_step": round(ms, 4), "value": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.S / (ms * 1e-3), 1)}


def time_plans_fused(args, torch, moe, w, C, sets, lay, window, y, total_bytes):
    """Decode sizes: the step as two pre-validated calls, the one-kernel layout + pack
    (moe_plan_layout_dispatch) and the combine, launched like the timed steps."""
    plans = [[moe.plan_layout_dispatch(topk, w.E, w.P, C, x, window, lay, w.quant, 0).run,
              moe.plan_combine(eo, lay.slot_idx, wts, y).run] for x, topk, wts, eo in sets]
    n = len(plans)
    for i in range(args.warmup):
        for run in plans[i % n]:
            run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        for run in plans[i % n]:
            run()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    return {"ms_per_step": round(ms, 4), "value": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.S / (ms * 1e-3), 1)}


def time_graph_replay(args, torch, moe, w, C, sets, lay, window, y, total_bytes, fused=False, per_graph=1,
                      lws=None):
    """The same step captured in HIP graphs and replayed: the device time of a step without the
    Python launch overhead, which dominates at decode sizes. per_graph = 1: one graph per input set,
    one step per replay; per_graph > 1: that many steps (cycling over the input sets) in one graph,
    so each replay's own launch cost is shared. fused: the layout and the pack through
    moe_layout_dispatch (one kernel when S*K <= 4096 and C <= 1024)."""
    def step(x, topk, wts, eo):
        if fused:
            moe.moe_layout_dispatch(topk, w.E, w.P, C, x, window, w.quant, 0, out=lay)
        else:
            moe.moe_layout_ws(topk, w.E, w.P, C, lws, w.quant, out=lay)
            moe.moe_dispatch_planned(x, lay.slot_idx, window, lws, C, w.quant, 0)
        moe.moe_combine(eo, lay.slot_idx, wts, y=y)

    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    groups = [[sets[i % len(sets)]] for i in range(len(sets))] if per_graph == 1 else \
        [[sets[i % len(sets)] for i in range(per_graph)]]
    for group in groups:
        with torch.cuda.stream(side):  # warm-up on the capture stream
            for x, topk, wts, eo in group:
                step(x, topk, wts, eo)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for x, topk, wts, eo in group:
                step(x, topk, wts, eo)
        graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        graphs[i % len(graphs)].replay()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    replays = max(1, args.steps // per_graph)
    torch.cuda.synchronize()
    e0.record()
    for i in range(replays):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (replays * per_graph)
    del graphs
    return {"ms_per_step": round(ms, 4), "value": round(total_bytes / (ms * 1e-3) / 1e9, 1),
            "tokens_per_s": round(w.S / (ms * 1e-3), 1)}


def time_unpack_padded(moe, torch, w, lay, window, n_valid, stream, A=16, iters=20):
    """moe_unpack_padded of the last dispatched window with expert_alignment A into the worst-case
    row count S*K + E*(A-1), which needs no count read back (outside the timed step)."""
    R = w.S * w.K + w.E * (A - 1)
    payload = 2 * w.H if w.quant == 0 else w.H
    out = None
    ms = []
    for i in range(iters + 3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = moe.moe_unpack_padded(window, lay.expert_slot_base, w.S, w.K, w.H, w.quant, A, R, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    per_row = payload + 12 + (4 if w.quant else 0)
    nbytes = n_valid * per_row + R * per_row + 8 * (w.E + 1) + 4
    avg_us = 1e3 * float(np.mean(ms))
    return {"alignment": A, "rows": R, "avg_us": round(avg_us, 2), "bytes": nbytes,
            "GB/s": round(nbytes / avg_us / 1e3, 1), "frac_hbm_peak": round(nbytes / avg_us / 1e3 / HBM_PEAK_GBS, 4)}


def time_two_pass_combine(moe, torch, w, lay, window, inputs, n_valid, gather_bytes, stream, iters=20):
    """The page's combine form next to the gather: scatter the expert rows to staging row t*K + k
    by the triples (from moe_unpack of the dispatched window), then reduce K contiguous rows.
    Outside the timed step; the staging rows are 512-byte aligned as on the page."""
    x, topk, wts, eo = inputs
    moe.moe_layout(topk, w.E, w.P, w.C, out=lay)
    moe.moe_dispatch(x, lay.slot_idx, window, w.quant, 0)
    idx = moe.moe_unpack(window, lay.expert_slot_base[w.E:], w.S, w.K, w.H, w.quant).expand_idx
    stride = -(-2 * w.H // 512) * 512
    staging = torch.empty(w.S * w.K * stride, dtype=torch.uint8, device=eo.device)
    y = torch.empty((w.S, w.H), dtype=torch.bfloat16, device=eo.device)
    t_sc, t_st = [], []
    for i in range(iters + 3):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        moe.moe_combine_scatter(eo, idx, lay.expert_slot_base[w.E:], w.S, w.K, staging=staging,
                                staging_stride_bytes=stride)
        e[1].record(stream)
        moe.moe_combine_staged(staging, lay.slot_idx, wts, w.H, staging_stride_bytes=stride, y=y)
        e[2].record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            t_sc.append(e[0].elapsed_time(e[1]))
            t_st.append(e[1].elapsed_time(e[2]))
    sc_bytes = n_valid * (2 * w.H + 2 * w.H + 12) + 4
    sc_us, st_us = 1e3 * float(np.mean(t_sc)), 1e3 * float(np.mean(t_st))
    return {"scatter_us": round(sc_us, 2), "scatter_bytes": sc_bytes,
            "scatter_GB/s": round(sc_bytes / sc_us / 1e3, 1),
            "staged_us": round(st_us, 2), "staged_GB/s": round(gather_bytes / st_us / 1e3, 1),
            "total_us": round(sc_us + st_us, 2)}


def time_dedup(moe, torch, w, C, lay, window, inputs, n_valid, kfold_pack_bytes, stream, iters=20):
    """DeepEP's per-rank deduplicated dispatch next to the K-fold pack: rank rows, the dedup pack
    (one row per token and destination rank) and the receive-side expansion to expert-major rows
    (which equals moe_unpack of the K-fold window). Outside the timed step; reuses the window."""
    x, topk, wts, eo = inputs
    moe.moe_layout(topk, w.E, w.P, C, out=lay)
    rr = moe.moe_rank_rows(topk, lay, w.E, w.P, C)
    exp = moe.moe_expand_dedup(window, rr.rank_row_idx, lay.slot_idx, lay.expert_slot_base[w.E:], w.P, w.H,
                               w.quant)
    torch.cuda.synchronize()
    m = int(rr.rank_token_base[w.P].item())
    ms = {"rank_rows": [], "dispatch_dedup": [], "expand_dedup": []}
    for i in range(iters + 3):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        moe.moe_rank_rows(topk, lay, w.E, w.P, C, out=rr)
        e[1].record(stream)
        moe.moe_dispatch_dedup(x, rr.rank_row_idx, topk, w.E, w.P, window, w.quant)
        e[2].record(stream)
        moe.moe_expand_dedup(window, rr.rank_row_idx, lay.slot_idx, lay.expert_slot_base[w.E:], w.P, w.H,
                             w.quant, out=exp)
        e[3].record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            for j, k in enumerate(ms):
                ms[k].append(e[j].elapsed_time(e[j + 1]))
    row = (2 * w.H + 12) if w.quant == 0 else (w.H + 16)
    pack_bytes = 2 * w.S * w.H + 8 * w.S * w.K + m * row
    expand_bytes = m * row + n_valid * row + 4 * w.S * w.K + 8 * n_valid + 4
    out = {"rows": m, "rows_per_token": round(m / w.S, 3),
           "write_bytes_vs_kfold": round(m / n_valid, 4)}
    for k, nb in (("rank_rows", None), ("dispatch_dedup", pack_bytes), ("expand_dedup", expand_bytes)):
        us = 1e3 * float(np.mean(ms[k]))
        out[k] = {"avg_us": round(us, 2)}
        if nb:
            out[k].update({"bytes": nb, "GB/s": round(nb / us / 1e3, 1),
                           "frac_hbm_peak": round(nb / us / 1e3 / HBM_PEAK_GBS, 4)})
    return out


def time_fp8_workload_pack(args, torch, moe, dev, window, stream):
    """The fp8 DynamicQuant pack on its own workload (S=4096, H=7168, E=256, P=8, K=8, x ~ 2*N(0,1)
    with 1% outliers x50): moe_dispatch_ws in fp8 mode, K launches back to back over --rotate copies
    of x (cold), one event at each end; its algorithmic bytes and fraction of 8 TB/s."""
    from workloads import WORKLOADS, make_inputs

    w4 = WORKLOADS[4]
    inp = make_inputs(w4, with_expert_out=False)
    n_valid = int(((inp["topk_idx"] >= 0) & (inp["topk_idx"] < w4.E)).sum())
    x0 = torch.from_numpy(inp["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    xs = [x0] + [x0.clone() for _ in range(1, max(1, args.rotate))]
    lay4 = moe.moe_layout(torch.from_numpy(inp["topk_idx"]).to(dev), w4.E, w4.P, w4.C)
    nws = moe.moe_dispatch_workspace_bytes(w4.S, w4.K, w4.quant)
    ws4 = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    for i in range(3):
        moe.moe_dispatch_ws(xs[i % len(xs)], lay4.slot_idx, window, ws4, w4.quant, 0)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        moe.moe_dispatch_ws(xs[i % len(xs)], lay4.slot_idx, window, ws4, w4.quant, 0)
    e1.record(stream)
    torch.cuda.synchronize()
    avg_us = 1e3 * e0.elapsed_time(e1) / args.steps
    nb = algorithmic_bytes(w4, w4.C, n_valid)["dispatch"]
    gbs = nb / (avg_us * 1e-6) / 1e9
    del xs, x0
    return {"workload": w4.describe(), "avg_us": round(avg_us, 2), "bytes": nb, "GB/s": round(gbs, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "input_sets": max(1, args.rotate),
            "timing": "K launches back to back, events at both ends"}


def time_unpack(moe, torch, w, lay, window, n_valid, stream, iters=20):
    """moe_unpack of the last dispatched window (outside the timed step): the grouped-GEMM input."""
    payload = 2 * w.H if w.quant == 0 else w.H
    out = None
    ms = []
    for i in range(iters + 3):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        out = moe.moe_unpack(window, lay.expert_slot_base[w.E:], w.S, w.K, w.H, w.quant, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            ms.append(e0.elapsed_time(e1))
    per_row = payload + 12 + (4 if w.quant else 0)
    nbytes = 2 * n_valid * per_row + 4
    avg_us = 1e3 * float(np.mean(ms))
    return {"avg_us": round(avg_us, 2), "bytes": nbytes, "GB/s": round(nbytes / avg_us / 1e3, 1),
            "frac_hbm_peak": round(nbytes / avg_us / 1e3 / HBM_PEAK_GBS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # 100 warm-up steps (about 18 ms at workload 3): with 10 the first timed steps still run 1-2% slower
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--channels", type=int, default=None)
    ap.add_argument("--rotate", type=int, default=8,
                    help="input sets cycled over the timed steps, each a copy of the seeded batch at its "
                         "own addresses, so that no step finds its inputs in the 256 MB memory-side cache "
                         "(1 = the same buffers every step)")
    ap.add_argument("--quant", choices=["workload", "none", "fp8", "int8"], default="workload",
                    help="dispatch payload type (default: the workload's own)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (unpack of the dispatched window)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run an elementwise fp32 negate of this many MiB (reads and writes "
                         "exactly that many bytes), to scale rocprofv3 memory counters")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the work; multi-GPU runs are not part of this "
              "build (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_moe_layout_02_amd as moe
    from workloads import WORKLOADS, draw_expert_out, make_inputs

    w = WORKLOADS[args.config]
    if args.quant != "workload":
        w = dataclasses.replace(w, quant={"none": 0, "fp8": 1, "int8": 2}[args.quant])
    C = args.channels or w.C
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    inp = make_inputs(w, with_expert_out=False)
    valid = (inp["topk_idx"] >= 0) & (inp["topk_idx"] < w.E)
    n_valid = int(valid.sum())
    eo_host = draw_expert_out(w.seed + 1000, n_valid, w.H)

    def to_dev(bits):
        return torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)

    # input sets: copies of the seeded batch at distinct addresses. Streaming loads and stores do not
    # stay in the memory-side cache, but x is read with the default policy, so the copies of x
    # together must exceed the cache's 256 MB for every timed step to read its inputs from HBM
    # (cold). Set 0 alone gives the warm case.
    base = (to_dev(inp["x"]), torch.from_numpy(inp["topk_idx"]).to(dev),
            torch.from_numpy(inp["topk_weights"]).to(dev), to_dev(eo_host))
    sets = [base] + [tuple(t.clone() for t in base) for _ in range(1, max(1, args.rotate))]
    lay = moe.empty_layout(w.S, w.K, w.E, w.P, C, dev)
    window = torch.empty(moe.moe_window_bytes(w.S, w.K, w.H), dtype=torch.uint8, device=dev)
    nws = moe.moe_dispatch_workspace_bytes(w.S, w.K, w.quant)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    nlws = moe.moe_layout_dispatch_workspace_bytes(w.S, w.K, w.E, w.P, C, w.quant)
    lws = torch.empty(nlws, dtype=torch.uint8, device=dev) if nlws else None
    y = torch.empty((w.S, w.H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # the step's three calls, checked once per input set (moe_plan_*); each launch is one moe_plan_run
    plans = {}

    def plans_of(st):
        key = id(st[0])
        if key not in plans:
            x, topk, wts, eo = st
            plans[key] = (moe.plan_layout_ws(topk, w.E, w.P, C, lay, lws, w.quant).run,
                          moe.plan_dispatch_planned(x, lay.slot_idx, window, lws, C, w.quant, 0).run,
                          moe.plan_combine(eo, lay.slot_idx, wts, y).run)
        return plans[key]

    for st in sets:
        plans_of(st)

    def step(i, sets_used):
        layout, dispatch, combine = plans_of(sets_used[i % len(sets_used)])
        layout()
        dispatch()
        combine()

    def timed(sets_used):
        """W untimed then K timed steps cycling over sets_used, timed by the wall clock between two
        device synchronisations with nothing recorded between the kernels; then the same K steps
        again with an event between every two kernels for the per-kernel statistics (each event
        adds a few microseconds to the step, so that pass is not the step time)."""
        for i in range(args.warmup):
            step(i, sets_used)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i, sets_used)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            e = ev[i]
            layout, dispatch, combine = plans_of(sets_used[i % len(sets_used)])
            e[0].record(stream)
            layout()
            e[1].record(stream)
            dispatch()
            e[2].record(stream)
            combine()
            e[3].record(stream)
        torch.cuda.synchronize()
        elapsed_events = time.perf_counter() - t1
        ms = {k: [] for k in ("layout", "dispatch", "combine")}
        for e in ev:
            ms["layout"].append(e[0].elapsed_time(e[1]))
            ms["dispatch"].append(e[1].elapsed_time(e[2]))
            ms["combine"].append(e[2].elapsed_time(e[3]))
        ms["layout+dispatch"] = [a + b for a, b in zip(ms["layout"], ms["dispatch"])]
        ms["layout+dispatch+combine"] = [a + b for a, b in zip(ms["layout+dispatch"], ms["combine"])]
        nb = dict(nbytes)
        nb["layout+dispatch"] = nbytes["layout"] + nbytes["dispatch"]
        nb["layout+dispatch+combine"] = nb["layout+dispatch"] + nbytes["combine"]
        kernels = {}
        for k, v in ms.items():
            avg_us = 1e3 * float(np.mean(v))
            gbs = nb[k] / (avg_us * 1e-6) / 1e9
            kernels[k] = {
                "avg_us": round(avg_us, 2), "min_us": round(1e3 * float(np.min(v)), 2),
                "median_us": round(1e3 * float(np.median(v)), 2), "bytes": nb[k],
                "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                "tokens_per_s": round(w.S / (avg_us * 1e-6), 1),
            }
            pc = pattern_ceilings.get(k)
            if pc:
                kernels[k]["frac_pattern_ceiling"] = round(gbs / pc, 4)
            if ceil:
                kernels[k]["frac_copy_ceiling"] = round(gbs / ceil["copy"], 4)
        return kernels, 1e3 * elapsed / args.steps, 1e3 * elapsed_events / args.steps

    def isolated(sets_used, calls):
        """Each call alone, K launches back to back cycling over sets_used, one event at each end:
        the average duration of one launch (with the short gaps between queued launches)."""
        out = {}
        for name, fn in calls.items():
            for i in range(3):
                fn(sets_used[i % len(sets_used)])
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                fn(sets_used[i % len(sets_used)])
            e1.record(stream)
            torch.cuda.synchronize()
            avg_us = 1e3 * e0.elapsed_time(e1) / args.steps
            gbs = nbytes[name] / (avg_us * 1e-6) / 1e9 if name in nbytes else None
            out[name] = {"avg_us": round(avg_us, 2)}
            if gbs is not None:
                out[name].update({"bytes": nbytes[name], "GB/s": round(gbs, 1),
                                  "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
                pc = pattern_ceilings.get(name)
                if pc:
                    out[name]["frac_pattern_ceiling"] = round(gbs / pc, 4)
        return out

    calls = {
        "layout": lambda st: plans_of(st)[0](),
        "dispatch": lambda st: plans_of(st)[1](),
        "combine": lambda st: plans_of(st)[2](),
    }

    nbytes = algorithmic_bytes(w, C, n_valid)
    ceil = None if args.no_extras else ceilings(torch, moe, dev)
    split = rw_split(w, C, n_valid)
    pattern_ceilings = {}
    if ceil:
        for k, (r, wb) in split.items():
            pattern_ceilings[k] = pattern_ceiling(ceil, r, wb)
        for k, parts in (("layout+dispatch", ("layout", "dispatch")),
                         ("layout+dispatch+combine", ("layout", "dispatch", "combine"))):
            r = sum(split[p][0] for p in parts)
            wb = sum(split[p][1] for p in parts)
            pattern_ceilings[k] = pattern_ceiling(ceil, r, wb)
    kernels, ms_per_step, ms_per_step_events = timed(sets)
    kernels_isolated = isolated(sets, calls)
    total_bytes = sum(nbytes.values())
    value = total_bytes / (ms_per_step * 1e-3) / 1e9
    dom = max(("dispatch", "combine"), key=lambda k: kernels[k]["avg_us"])
    planned = moe.moe_dispatch_workspace_bytes(w.S, w.K, w.quant) > 0
    plan_by_layout = planned and -(-w.S // C) * w.K <= 1024  # else moe_dispatch_planned runs the plan kernel
    kernel_key = {"dispatch": {0: "pack_bf16_planned" if planned else "pack_bf16", 1: "pack_fp8",
                               2: "pack_int8"}[w.quant],
                  "combine": "combine"}[dom]
    traffic = traffic_from_profiles(f"{kernel_key}:{w.name}")
    roofline = {
        "bound": "hbm", "kernel": kernel_key,
        "launches": ("plan + pack kernels of one moe_dispatch_planned call" if dom == "dispatch" and planned
                     and not plan_by_layout else "one kernel"),
        "achieved": kernels[dom]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(kernels[dom]["GB/s"] / HBM_PEAK_GBS, 4), "traffic": traffic,
        "algorithmic_bytes_per_launch": nbytes[dom],
        "avg_launch_us": kernels[dom]["avg_us"],
        "timing": "events before and after the call in each of the K timed steps (the kernels' stream)",
        "isolated_avg_launch_us": kernels_isolated[dom]["avg_us"],
    }
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "bf16", 1: "fp8-e4m3+bf16", 2: "int8+bf16"}[w.quant],
        "data": "synthetic",
        "config": {"workload": w.describe() + f" C={C}", "S": w.S, "H": w.H, "E": w.E, "P": w.P,
                   "K": w.K, "C": C, "quant": {0: "none", 1: "fp8_e4m3_dynamic", 2: "int8_dynamic"}[w.quant],
                   "seed": w.seed, "input_sets": len(sets),
                   "parallelism": "single GPU (P virtual ranks)"},
        "tokens_per_s": round(w.S / (ms_per_step * 1e-3), 1),
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step_with_events": round(ms_per_step_events, 4),
        "kernels": kernels,
        "kernels_isolated": kernels_isolated,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if ceil:
        out["ceilings"] = dict(ceil, unit="GB/s", method="library probes (include/moe_probe.h) over 1 GiB; "
                               "copy counts read + write bytes", pattern_ceiling_GB_s={
                                   k: round(v, 1) for k, v in pattern_ceilings.items()})
    if not args.no_extras:
        out["extras"] = {}
        tok = isolated(sets, {"dispatch": lambda st: moe.moe_dispatch(st[0], lay.slot_idx, window, w.quant, 0)})
        out["extras"]["dispatch_token_order"] = tok["dispatch"]
        if len(sets) > 1:
            warm, warm_ms, _ = timed(sets[:1])
            out["extras"]["warm_same_buffers"] = {
                "value": round(total_bytes / (warm_ms * 1e-3) / 1e9, 1), "ms_per_step": round(warm_ms, 4),
                "kernels": {k: {f: v[f] for f in ("avg_us", "GB/s", "frac_hbm_peak")} for k, v in warm.items()}}
        out["extras"]["fused_layout_dispatch"] = time_fused_eager(args, torch, moe, w, C, sets, lay, window,
                                                                  y, total_bytes)
        out["extras"]["three_launch_layout_dispatch_ws"] = time_three_launch_eager(
            args, torch, moe, w, C, sets, lay, window, y, total_bytes, ws)
        out["extras"]["eager_binding_calls"] = time_eager_binding(args, torch, moe, w, C, sets, lay, window, y,
                                                                  total_bytes, lws)
        out["extras"]["graph_replay"] = time_graph_replay(args, torch, moe, w, C, sets, lay, window, y,
                                                          total_bytes, lws=lws)
        fused = time_graph_replay(args, torch, moe, w, C, sets, lay, window, y, total_bytes, fused=True)
        fused["one_kernel_layout_dispatch"] = w.S * w.K <= 4096 and C <= 1024
        out["extras"]["graph_replay_fused_layout_dispatch"] = fused
        if w.S * w.K <= 4096 and C <= 1024:  # decode sizes: the one-kernel layout + pack as a plan
            out["extras"]["plans_fused_layout_dispatch"] = time_plans_fused(args, torch, moe, w, C, sets, lay,
                                                                            window, y, total_bytes)
        if w.S * w.K <= 4096:  # decode sizes: 16 steps per graph, the replay's own cost shared
            out["extras"]["graph_replay_16_steps_per_graph"] = {
                "separate": time_graph_replay(args, torch, moe, w, C, sets, lay, window, y, total_bytes,
                                              per_graph=16, lws=lws),
                "fused_layout_dispatch": time_graph_replay(args, torch, moe, w, C, sets, lay, window, y,
                                                           total_bytes, fused=True, per_graph=16)}
        if w.name == "dsv3_prefill":
            out["extras"]["fp8_dynquant_pack"] = time_fp8_workload_pack(args, torch, moe, dev, window, stream)
        out["extras"]["unpack"] = time_unpack(moe, torch, w, lay, window, n_valid, stream)
        out["extras"]["unpack_padded"] = time_unpack_padded(moe, torch, w, lay, window, n_valid, stream)
        out["extras"]["two_pass_combine"] = time_two_pass_combine(moe, torch, w, lay, window, sets[0],
                                                                  n_valid, nbytes["combine"], stream)
        out["extras"]["dedup_dispatch"] = time_dedup(moe, torch, w, C, lay, window, sets[0], n_valid,
                                                     nbytes["dispatch"], stream)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, C, inp, eo_host, n_valid)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
