#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel dispatch layout + dispatch pack +
combine on one MI355X.

A step is one pass of the whole path (ep_layout, ep_dispatch, ep_combine)
over one batch: the prefill workload, 4,096 tokens x hidden 7,168, 256 experts
in 8 groups over 8 logical ranks, top-4 groups then top-8 experts, FP8
dispatch with one scale per 128 channels, BF16 combine (the DeepEP V1 Legacy
guide's §2.1 normal-kernel benchmark shape).  The decode workload (128 tokens,
top-8, FP8; §2.2's low-latency shape) is timed the same way and reported in
the same JSON line.

Inputs are seeded synthetic data resident in HBM before timing starts.  Each
timed step is bracketed by two HIP events on the stream the kernels run on;
before each step an untimed read of 1 GiB evicts the 256 MB Infinity Cache,
so the figures are cold-HBM figures ("warm" figures, without the eviction,
are reported beside them).  Throughput counts the algorithmic bytes of the
method (reads + writes it must do), not allocation, poisoning or the expert
output generation.

Prints ONE JSON line.  With --gpus > 1 it exits: the path runs on one GPU.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak, AMD's published figure
FUSED_MAX_TOKENS = 256  # ep_layout_dispatch is one launch up to this many tokens
PROFILES = os.path.join(ROOT, "profiles")


def algorithmic_bytes(n, h, k, e, r, p, use_fp8, scale_format=0):
    """Bytes the method must move per call, by phase.

    layout : read topk_idx (8 B per entry); write expert_slot (4 B per entry),
             rank_slot (4 B) and the u8 mask per (token, rank), the two count
             arrays and the offsets.
    pack   : read x once per token, topk_idx + expert_slot per entry; write
             per valid entry one row (H bytes FP8 or 2H bytes BF16), its
             source index (4 B) and, for FP8, H/128 fp32 scales (UE8M0:
             ceil(H/512) 32-bit words).
    combine: read one bf16 expert row per valid entry and idx + slot + weight
             per entry; write one bf16 output row per token."""
    b = 1 if use_fp8 else 2
    layout = 12 * n * k + 5 * n * r + 4 * (2 * e + r + 1)
    g = h // 128
    scale_bytes = 0 if not use_fp8 else 4 * ((g + 3) // 4) if scale_format == 2 else 4 * g
    pack = 2 * n * h + 12 * n * k + p * (b * h + 4 + scale_bytes)
    combine = 2 * p * h + 16 * n * k + 2 * n * h
    return {"layout": layout, "dispatch": pack, "combine": combine,
            "total": layout + pack + combine}


def kernel_source_digest():
    """Digest of every HIP source and header of the library (and its public
    headers): counter readings are only reused while it is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_ep_layout_02_amd", "csrc")
    inc = os.path.join(ROOT, "include")
    for d in (csrc, inc):
        for f in sorted(os.listdir(d)):
            if f.endswith((".hip", ".h", ".cpp")):
                with open(os.path.join(d, f), "rb") as fh:
                    h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload_name, kernel, digest):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_name}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_digest:\s*(\w+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != digest:
        return None
    return float(t.group(1))


def percentile(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def run_workload(wid, steps, warmup, scrub_bytes, say, batch=10):
    """Times the path on workload ``wid``.  Passes (each of ``steps``
    iterations, an untimed cache eviction before each iteration):

    cold    : the step is ep_layout_dispatch then ep_combine, events only
              before and after it -> the value;
    three   : the same step as ep_layout, ep_dispatch, ep_combine;
    graph   : the step captured once in a HIP graph and replayed;
    phases  : an event between the two calls as well (each event record
              delays the next launch by a few us: upper bounds);
    kernels : ``batch`` back-to-back launches of one entry point between two
              events -> average launch duration per entry point (the roofline);
    warm    : ``steps`` steps back to back, no eviction, two events overall.

    The eviction reads a buffer larger than the 256 MB Infinity Cache, so the
    cache holds clean unrelated lines and every input is in HBM (evicting by
    writing would leave dirty lines whose write-back lands in the next
    kernel)."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    shape = ep.shape_of(w)
    say(f"workload {w.name}: generating inputs")
    inp = W.make_inputs(w)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    topk_weights = torch.from_numpy(inp["topk_weights"]).to(dev)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev)
    buf = ep.allocate(shape, dev, parts=("layout", "dispatch", "combine"))
    g = torch.Generator(device=dev)
    g.manual_seed(2000 + wid)
    # expert outputs: bf16 N(0, 1) in every row (rows past a count are never read)
    y = torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16,
                    device=dev, generator=g).view(torch.int16)
    # eviction buffer: float32 so the reduction reads it in place (no cast copy)
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)
    P = inp["num_valid"]
    nbytes = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, P,
                               w.use_fp8)

    # every launch goes to torch's current stream (also while a graph is captured)
    def layout():
        ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])

    def dispatch():
        ep.ep_dispatch(shape, x, topk_idx, buf["expert_slot"], buf["recv_x"], buf["recv_scales"],
                       buf["recv_src_idx"], buf["status"])

    def combine():
        ep.ep_combine(shape, y, topk_idx, topk_weights, buf["expert_slot"], buf["combined_x"],
                      buf["status"])

    def layout_dispatch():
        ep.ep_layout_dispatch(shape, topk_idx, x, buf["num_tokens_per_rank"],
                              buf["num_tokens_per_expert"], buf["is_token_in_rank"],
                              buf["expert_slot"], buf["rank_slot"], buf["expert_offset"],
                              buf["workspace"], buf["recv_x"], buf["recv_scales"],
                              buf["recv_src_idx"], buf["status"])

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    # the timing loops re-issue prepared calls (arguments checked and
    # converted once, on torch's current stream); the graph capture below
    # uses the plain binding, which takes the capture stream
    plain = {"layout": layout, "dispatch": dispatch, "combine": combine,
             "layout_dispatch": layout_dispatch}
    layout = ep.prepare(ep.ep_layout, shape, topk_idx, buf["num_tokens_per_rank"],
                        buf["num_tokens_per_expert"], buf["is_token_in_rank"], buf["expert_slot"],
                        buf["rank_slot"], buf["expert_offset"], buf["workspace"], buf["status"])
    dispatch = ep.prepare(ep.ep_dispatch, shape, x, topk_idx, buf["expert_slot"], buf["recv_x"],
                          buf["recv_scales"], buf["recv_src_idx"], buf["status"])
    combine = ep.prepare(ep.ep_combine, shape, y, topk_idx, topk_weights, buf["expert_slot"],
                         buf["combined_x"], buf["status"])
    layout_dispatch = ep.prepare(ep.ep_layout_dispatch, shape, topk_idx, x,
                                 buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                                 buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                                 buf["expert_offset"], buf["workspace"], buf["recv_x"],
                                 buf["recv_scales"], buf["recv_src_idx"], buf["status"])

    def new_events(n):
        # torch creates an event's handle at its first record: record each
        # once here so that no handle is created inside a timed region
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)
        return evs

    say(f"workload {w.name}: {warmup} warmup steps")
    for _ in range(warmup):
        layout_dispatch()
        combine()
        evict()
        layout()
        dispatch()
        combine()
        evict()
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())} during warmup")

    # the step: ep_layout_dispatch, then ep_combine (the library's one-call
    # layout and pack; its outputs are exactly those of ep_layout and
    # ep_dispatch); the same step as three calls is timed alongside
    def step():
        layout_dispatch()
        combine()

    def step_three_calls():
        layout()
        dispatch()
        combine()

    say(f"workload {w.name}: {steps} timed steps, cache evicted before each")
    evs = [new_events(2) for _ in range(steps)]
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()  # no collector pause while the host enqueues a timed step
    t0 = time.perf_counter()
    for e in evs:
        evict()
        e[0].record(stream)
        step()
        e[1].record(stream)
    torch.cuda.synchronize()
    wall_cold = time.perf_counter() - t0
    gc.enable()
    cold = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    say(f"workload {w.name}: cold step times (us): " + " ".join(f"{v:.1f}" for v in cold))

    say(f"workload {w.name}: {steps} timed steps as three calls")
    evs = [new_events(2) for _ in range(steps)]
    for e in evs:
        evict()
        e[0].record(stream)
        step_three_calls()
        e[1].record(stream)
    torch.cuda.synchronize()
    cold_three = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]

    # The step without the latency an event marker adds before the next
    # launch: (eviction + step) minus (eviction alone), each between two
    # events, so both carry one marker.  An untimed eviction first takes the
    # previous step's dirty lines, so both timed evictions start alike.
    say(f"workload {w.name}: {steps} pairs of eviction alone and eviction + step")
    evs = [new_events(4) for _ in range(steps)]
    for e in evs:
        evict()
        e[0].record(stream)
        evict()
        e[1].record(stream)
        e[2].record(stream)
        evict()
        step()
        e[3].record(stream)
    torch.cuda.synchronize()
    evict_only = statistics.median([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    evict_step = statistics.median([e[2].elapsed_time(e[3]) * 1e3 for e in evs])
    net = {"eviction_us_median": round(evict_only, 2),
           "eviction_plus_step_us_median": round(evict_step, 2),
           "step_us": round(evict_step - evict_only, 2)}

    say(f"workload {w.name}: {steps} steps with an event between the two calls")
    evs = [new_events(3) for _ in range(steps)]
    for e in evs:
        evict()
        e[0].record(stream)
        layout_dispatch()
        e[1].record(stream)
        combine()
        e[2].record(stream)
    torch.cuda.synchronize()
    phases = {"layout_dispatch": [e[0].elapsed_time(e[1]) * 1e3 for e in evs],
              "combine": [e[1].elapsed_time(e[2]) * 1e3 for e in evs]}

    say(f"workload {w.name}: {batch} back-to-back launches per entry point, {steps} times")
    kernels = {}
    for name, fn in (("layout", layout), ("dispatch", dispatch),
                     ("layout_dispatch", layout_dispatch), ("combine", combine)):
        evs = [new_events(2) for _ in range(steps)]
        for e in evs:
            evict()
            e[0].record(stream)
            for _ in range(batch):
                fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        kernels[name] = [e[0].elapsed_time(e[1]) * 1e3 / batch for e in evs]

    say(f"workload {w.name}: the step captured in a HIP graph, {steps} replays")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        plain["layout_dispatch"]()
        plain["combine"]()
    stream.wait_stream(side)
    with torch.cuda.graph(graph):
        plain["layout_dispatch"]()
        plain["combine"]()
    torch.cuda.synchronize()
    evs = [new_events(2) for _ in range(steps)]
    for e in evs:
        evict()
        e[0].record(stream)
        graph.replay()
        e[1].record(stream)
    torch.cuda.synchronize()
    graph_cold = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    del graph

    say(f"workload {w.name}: {steps} steps back to back (warm), prepared and plain calls")
    warm = {}
    for kind, fns in (("prepared", (layout_dispatch, combine)),
                      ("prepared_three_calls", (layout, dispatch, combine)),
                      ("plain_three_calls", (plain["layout"], plain["dispatch"], plain["combine"]))):
        e = new_events(2)
        for _ in range(5):  # untimed, so the GPU is busy when timing starts
            for fn in fns:
                fn()
        torch.cuda.synchronize()
        e[0].record(stream)
        h0 = time.perf_counter()
        for _ in range(steps):
            for fn in fns:
                fn()
        h1 = time.perf_counter()
        e[1].record(stream)
        torch.cuda.synchronize()
        warm[kind] = {"us_per_step": round(e[0].elapsed_time(e[1]) * 1e3 / steps, 2),
                      "host_enqueue_us_per_step": round((h1 - h0) * 1e6 / steps, 2)}
    warm_us = warm["prepared"]["us_per_step"]
    # a plain copy of known size, for scaling counter readings of a profile run
    if scrub is not None:
        half = scrub.numel() // 2
        scrub[half:].copy_(scrub[:half])
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")

    def stats(v, b):
        med = statistics.median(v)
        return {"us_median": round(med, 2), "us_mean": round(statistics.fmean(v), 2),
                "us_p10": round(percentile(v, 10), 2), "us_p90": round(percentile(v, 90), 2),
                "gbps_median": round(b / (med * 1e-6) / 1e9, 1)}

    nb_ld = nbytes["layout"] + nbytes["dispatch"]
    entry_bytes = {"layout": nbytes["layout"], "dispatch": nbytes["dispatch"],
                   "layout_dispatch": nb_ld, "combine": nbytes["combine"]}
    return {
        "workload": w, "bytes": nbytes, "num_valid": P,
        "cold": stats(cold, nbytes["total"]),
        "cold_three_calls": stats(cold_three, nbytes["total"]),
        "graph_cold": stats(graph_cold, nbytes["total"]),
        "cold_net_of_marker": dict(net, gbps=round(nbytes["total"] / (net["step_us"] * 1e-6) / 1e9, 1)),
        "phases": {k: stats(v, entry_bytes[k]) for k, v in phases.items()},
        "kernels": {k: stats(v, entry_bytes[k]) for k, v in kernels.items()},
        "warm_us_per_step": round(warm_us, 2),
        "warm": warm,
        "wall_cold_s": wall_cold,
        "inputs": inp,
    }


def receive_layout_bytes(n, h, k, r, p, rows_sent, pad_rows, use_fp8, scale_format=0):
    """Algorithmic bytes of the other receive layouts, by entry point.

    dispatch_normal : read x once, rank_slot, topk_idx, topk_weights; write per
                      (token, rank) row the payload, scales, its source index
                      and K routing entries (8 B id + 4 B weight);
    combine_normal  : read rank_slot, one bf16 row and K weights per
                      (token, rank) row; write the bf16 output and K weights
                      per token;
    dispatch_expand : the per-expert pack's bytes plus the padding rows
                      (payload, scales and source index each);
    combine_expand  : the per-expert combine's bytes."""
    b = 1 if use_fp8 else 2
    g = h // 128
    scale_bytes = 0 if not use_fp8 else 4 * ((g + 3) // 4) if scale_format == 2 else 4 * g
    row = b * h + scale_bytes + 4
    return {
        "dispatch_normal": 2 * n * h + 4 * n * r + 12 * n * k + rows_sent * (row + 12 * k),
        "combine_normal": 4 * n * r + rows_sent * (2 * h + 4 * k) + n * (2 * h + 4 * k),
        "dispatch_expand": 2 * n * h + 12 * n * k + (p + pad_rows) * row,
        "combine_expand": 2 * p * h + 16 * n * k + 2 * n * h,
    }


def _recorded_event_pair(stream):
    """Two timing events, each recorded once (torch creates an event's handle
    at its first record), so no handle is created inside a timed region."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0, e1


def _timed_batches(fn, steps, batch, evict, stream):
    """Average duration of one call: ``batch`` back-to-back calls between two
    events after an untimed eviction, ``steps`` times."""
    import torch

    times = []
    e0, e1 = _recorded_event_pair(stream)
    for _ in range(steps):
        evict()
        e0.record(stream)
        for _ in range(batch):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / batch)
    return statistics.fmean(times)


def _timed_cold(fn, steps, evict, stream):
    """Median duration of one call with a cold Infinity Cache: an untimed
    eviction, then two events around the call, ``steps`` times.  The events
    add a few us of launch latency, so this is an upper bound on the kernel
    time (the rocprofv3 trace of the same run gives the kernel-only time)."""
    import torch

    times = []
    e0, e1 = _recorded_event_pair(stream)
    for _ in range(steps):
        evict()
        e0.record(stream)
        fn()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    return statistics.median(times)


def time_receive_layouts(wid, steps, scrub_bytes, say, alignment=128, batch=10):
    """The normal-mode and expand paths on workload ``wid``: each entry point
    timed alone, cold (one launch after an eviction, the same protocol as the
    bench's step) and back to back (``batch`` launches after an eviction:
    once a kernel writes more than the 256 MB Infinity Cache holds, each
    launch also pays the write-back of the previous one's lines), and the
    whole layout + dispatch + combine step of each mode, cold."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    shape = ep.shape_of(w, expert_alignment=alignment)
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    topk_weights = torch.from_numpy(inp["topk_weights"]).to(dev)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev)
    buf = ep.allocate(shape, dev, parts=("layout", "combine", "normal", "expand"))
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    def layout():
        ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])

    def dispatch_normal():
        ep.ep_dispatch_normal(shape, x, topk_idx, topk_weights, buf["rank_slot"],
                              buf["recv_x_normal"], buf["recv_scales_normal"], buf["recv_topk_idx"],
                              buf["recv_topk_weights"], buf["recv_src_idx_normal"], buf["status"])

    g = torch.Generator(device=dev)
    g.manual_seed(2100 + wid)
    R, M, H = w.num_ranks, w.num_max_dispatch_tokens_per_rank, w.hidden
    y_normal = torch.randn((R, M, H), dtype=torch.bfloat16, device=dev, generator=g).view(torch.int16)
    T = ep.expand_rows(shape)
    y_expand = torch.randn((T, H), dtype=torch.bfloat16, device=dev, generator=g).view(torch.int16)

    def combine_normal():
        ep.ep_combine_normal(shape, y_normal, buf["rank_slot"], buf["recv_topk_weights"],
                             buf["combined_x"], buf["combined_topk_weights"], buf["status"])

    def dispatch_expand():
        ep.ep_dispatch_expand(shape, x, topk_idx, buf["expert_slot"], buf["expert_offset"],
                              buf["num_tokens_per_expert"], buf["recv_x_expand"],
                              buf["recv_scales_expand"], buf["recv_src_idx_expand"], buf["status"])

    def combine_expand():
        ep.ep_combine_expand(shape, y_expand, topk_idx, topk_weights, buf["expert_slot"],
                             buf["expert_offset"], buf["combined_x"], buf["status"])

    layout()
    dispatch_normal()
    dispatch_expand()
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    rows_sent = int(buf["num_tokens_per_rank"].sum().item())
    used = int(buf["expert_offset"][-1].item())
    P = inp["num_valid"]
    nb = receive_layout_bytes(w.num_tokens, H, w.num_topk, R, P, rows_sent, used - P, w.use_fp8)
    out = {"workload": w.name, "expert_alignment": alignment, "rows_sent_normal": rows_sent,
           "expand_rows_used": used, "expand_padding_rows": used - P, "bytes": nb}
    for name, fn in (("dispatch_normal", dispatch_normal), ("combine_normal", combine_normal),
                     ("dispatch_expand", dispatch_expand), ("combine_expand", combine_expand)):
        say(f"{name} {w.name}: {steps} cold launches, {steps} x {batch} back to back")
        cold = _timed_cold(fn, steps, evict, stream)
        b2b = _timed_batches(fn, steps, batch, evict, stream)
        out[name] = {"us_cold_median": round(cold, 2),
                     "gbps_cold": round(nb[name] / (cold * 1e-6) / 1e9, 1),
                     "frac_of_peak_cold": round(nb[name] / (cold * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                     "us_back_to_back_mean": round(b2b, 2),
                     "gbps_back_to_back": round(nb[name] / (b2b * 1e-6) / 1e9, 1)}
    for mode, d, c in (("normal", dispatch_normal, combine_normal),
                       ("expand", dispatch_expand, combine_expand)):
        def step():
            layout()
            d()
            c()
        say(f"{mode} step {w.name}: {steps} steps")
        out[f"step_us_cold_{mode}"] = round(_timed_cold(step, steps, evict, stream), 2)
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    return out


def time_config(wid, steps, warmup, scrub_bytes, say, allocations=1):
    """The whole step (ep_layout_dispatch, then ep_combine) on another
    workload, cold (eviction before each step, two events around it): median
    and mean us, and algorithmic GB/s at the mean, against the 60 % of peak
    bar; the median of the same step as three calls beside it.

    With allocations > 1 the receive buffer and the expert outputs are freed
    and allocated again that many times in all, and the median step of each
    allocation is reported as well: on buffers of tens of GB the physical
    pages behind an allocation move the pack and the combine by up to about
    13 %, with the same code and virtual layout.  The headline figures are
    those of the first allocation."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    shape = ep.shape_of(w)
    say(f"workload {w.name}: generating inputs")
    inp = W.make_inputs(w)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    topk_weights = torch.from_numpy(inp["topk_weights"]).to(dev)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev)
    buf = ep.allocate(shape, dev, parts=("layout", "dispatch", "combine"))
    g = torch.Generator(device=dev)
    g.manual_seed(2400 + wid)
    y = torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16,
                    device=dev, generator=g).view(torch.int16)
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    def combine():
        ep.ep_combine(shape, y, topk_idx, topk_weights, buf["expert_slot"], buf["combined_x"],
                      buf["status"])

    def step():
        # the bench's step: ep_layout_dispatch, then ep_combine
        ep.ep_layout_dispatch(shape, topk_idx, x, buf["num_tokens_per_rank"],
                              buf["num_tokens_per_expert"], buf["is_token_in_rank"],
                              buf["expert_slot"], buf["rank_slot"], buf["expert_offset"],
                              buf["workspace"], buf["recv_x"], buf["recv_scales"],
                              buf["recv_src_idx"], buf["status"])
        combine()

    def step_three_calls():
        ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])
        ep.ep_dispatch(shape, x, topk_idx, buf["expert_slot"], buf["recv_x"], buf["recv_scales"],
                       buf["recv_src_idx"], buf["status"])
        combine()

    def cold_steps(fn=step):
        for _ in range(warmup):
            fn()
            evict()
        torch.cuda.synchronize()
        times = []
        e0, e1 = _recorded_event_pair(stream)
        for _ in range(steps):
            evict()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3)
        if int(buf["status"].item()) != 0:
            raise RuntimeError(f"device status {int(buf['status'].item())}")
        return times

    say(f"workload {w.name}: {steps} cold steps")
    times = cold_steps()
    say(f"workload {w.name}: {steps} cold steps as three calls")
    three = cold_steps(step_three_calls)
    by_allocation = [round(statistics.median(times), 2)]
    for a in range(1, allocations):
        # the same shapes and contents in newly allocated memory
        rx_shape, rx_dtype = buf["recv_x"].shape, buf["recv_x"].dtype
        del buf["recv_x"], y
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        buf["recv_x"] = torch.empty(rx_shape, dtype=rx_dtype, device=dev)
        g.manual_seed(2400 + wid)
        y = torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16,
                        device=dev, generator=g).view(torch.int16)
        say(f"workload {w.name}: allocation {a + 1} of {allocations}, {steps} cold steps")
        by_allocation.append(round(statistics.median(cold_steps()), 2))
    nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                           inp["num_valid"], w.use_fp8)["total"]
    mean = statistics.fmean(times)
    out = {"us_median": round(statistics.median(times), 2), "us_mean": round(mean, 2),
           "bytes": nb, "gbps_at_mean": round(nb / (mean * 1e-6) / 1e9, 1),
           "frac_of_peak": round(nb / (mean * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
           "bar_60pct_us": round(nb / (0.6 * PEAK_HBM_GBPS * 1e9) * 1e6, 1),
           "us_median_three_calls": round(statistics.median(three), 2)}
    if allocations > 1:
        out["us_median_by_allocation"] = by_allocation
        out["frac_of_peak_by_allocation"] = [round(nb / (u * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
                                             for u in by_allocation]
    return out


# the other workloads timed as whole cold steps (workload id -> JSON key)
OTHER_CONFIGS = {4: "large_16384x7168_bf16", 5: "skewed_4096x4096"}


def calibration_copy():
    """A plain copy of 512 MiB (torch copy_, which the runtime runs as its own
    copy kernel): the known-size reference that scales the HBM counters of a
    profiling run."""
    import torch

    src = torch.ones(1 << 29, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def time_copy_ceiling(steps, say):
    """A plain device-to-device copy of 2 GiB (torch copy_, which the runtime
    runs as its own copy kernel): the rate a streaming half-read, half-write
    pattern reaches on this GPU, as context for the step's GB/s.  The buffers
    are far larger than the 256 MB Infinity Cache, so no eviction is needed."""
    import torch

    n = 1 << 31
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    say(f"plain copy of {n >> 20} MiB, {steps} times")
    for _ in range(2):
        dst.copy_(src)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:  # handles are created at the first record, outside the timed region
        e[0].record(stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    for e in evs:
        e[0].record(stream)
        dst.copy_(src)
        e[1].record(stream)
    torch.cuda.synchronize()
    us = statistics.median([e[0].elapsed_time(e[1]) * 1e3 for e in evs])
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * n / (us * 1e-6) / 1e9
    return {"bytes_read": n, "bytes_written": n, "us_median": round(us, 1),
            "gbps_read_plus_write": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_HBM_GBPS, 4)}


def gpu_clocks():
    """Current and top shader (sclk) and memory (mclk) clock levels of the
    GPUs, from the kernel driver's power-management files (each lists the
    levels in MHz, the current one marked with '*'); when those are not
    readable, from rocm-smi.  None when neither source answers."""
    import glob
    import subprocess

    out = {}
    for dev_dir in sorted(glob.glob("/sys/class/drm/card*/device")):
        entry = {}
        for name in ("pp_dpm_sclk", "pp_dpm_mclk"):
            try:
                with open(os.path.join(dev_dir, name)) as f:
                    levels = [ln.strip() for ln in f if ln.strip()]
            except OSError:
                continue
            cur = [ln for ln in levels if ln.endswith("*")]
            mhz = [int(re.findall(r"(\d+)\s*[Mm][Hh]z", ln)[0]) for ln in levels
                   if re.findall(r"(\d+)\s*[Mm][Hh]z", ln)]
            entry[name[7:]] = {"current": cur[0] if cur else None, "max_mhz": max(mhz) if mhz else None}
        if entry:
            out[dev_dir.split("/")[-2]] = entry
    if out:
        return {"source": "/sys/class/drm/*/device/pp_dpm_{sclk,mclk}", "levels": out}
    try:
        res = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                             timeout=30)
        if res.returncode == 0 and res.stdout.strip().startswith("{"):
            return {"source": "rocm-smi --showclocks --json", "levels": json.loads(res.stdout)}
    except (OSError, subprocess.SubprocessError, ValueError):
        pass
    return None


def device_info():
    """The device and software the figures were measured on."""
    import torch

    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip,
            "torch": torch.__version__, "clocks": gpu_clocks()}


def time_gating(wid, steps, scrub_bytes, say):
    """Group-limited gating on workload ``wid``'s own router scores with the
    summed-score rule (top groups by the ordered binary32 sum of their
    scores, normalised sigmoid weights), which reproduces the workload's
    routing exactly (checked here): ep_group_limited_topk alone, cold; the
    whole step with the gating in front (gating + layout + dispatch +
    combine), cold; and the same step without the gating in the same run.
    The gating's algorithmic bytes: read the scores (4 B per (token,
    expert)), write topk_idx (8 B) and topk_weights (4 B) per entry."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    shape = ep.shape_of(w)
    N, E, K, H = w.num_tokens, w.num_experts, w.num_topk, w.hidden
    G, TG = w.num_groups, w.topk_groups
    say(f"gating {w.name}: generating inputs")
    inp = W.make_inputs(w)
    scores = torch.from_numpy(inp["router_scores"]).to(dev)
    topk_idx = torch.empty((N, K), dtype=torch.int64, device=dev)
    topk_weights = torch.empty((N, K), dtype=torch.float32, device=dev)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(2300 + wid)
    y = torch.randn((E, w.expert_capacity, H), dtype=torch.bfloat16, device=dev,
                    generator=g).view(torch.int16)
    buf = ep.allocate(shape, dev, parts=("layout", "dispatch", "combine"))
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    def gate():
        ep.ep_group_limited_topk(shape, G, TG, ep.EP_GATE_SUM_SIGMOID, scores, topk_idx,
                                 topk_weights)

    def path():
        ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])
        ep.ep_dispatch(shape, x, topk_idx, buf["expert_slot"], buf["recv_x"], buf["recv_scales"],
                       buf["recv_src_idx"], buf["status"])
        ep.ep_combine(shape, y, topk_idx, topk_weights, buf["expert_slot"], buf["combined_x"],
                      buf["status"])

    def step():
        gate()
        path()

    step()
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    if not np.array_equal(topk_idx.cpu().numpy(), inp["topk_idx"]):
        raise RuntimeError("the gating did not reproduce the workload's routing")
    nb = 4 * N * E + 12 * N * K
    say(f"ep_group_limited_topk {w.name}: {steps} cold launches, {steps} gated steps")
    us = _timed_cold(gate, steps, evict, stream)
    return {"rule": "group score = ordered binary32 sum; weights = normalised sigmoids",
            "num_groups": G, "topk_groups": TG, "bytes": nb,
            "picks_equal_the_workload_routing": True,
            "us_cold_median": round(us, 2), "gbps_cold": round(nb / (us * 1e-6) / 1e9, 1),
            "step_us_cold_with_gating": round(_timed_cold(step, steps, evict, stream), 2),
            "step_us_cold_without_gating": round(_timed_cold(path, steps, evict, stream), 2)}


def time_combine_bias(wid, steps, scrub_bytes, say):
    """ep_combine with and without the shared expert's bias row (one more bf16
    row read per token), cold single launches after an eviction."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    shape = ep.shape_of(w)
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    topk_weights = torch.from_numpy(inp["topk_weights"]).to(dev)
    buf = ep.allocate(shape, dev, parts=("layout", "combine"))
    ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                 buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                 buf["expert_offset"], buf["workspace"], buf["status"])
    g = torch.Generator(device=dev)
    g.manual_seed(2200 + wid)
    y = torch.randn((w.num_experts, w.expert_capacity, w.hidden), dtype=torch.bfloat16, device=dev,
                    generator=g).view(torch.int16)
    bias = torch.randn((w.num_tokens, w.hidden), dtype=torch.bfloat16, device=dev,
                       generator=g).view(torch.int16)
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    P = inp["num_valid"]
    nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, P,
                           w.use_fp8)["combine"]
    out = {}
    for label, b in (("plain", None), ("bias", bias)):
        say(f"ep_combine {label} {w.name}: {steps} cold launches")
        fn = lambda: ep.ep_combine(shape, y, topk_idx, topk_weights, buf["expert_slot"],
                                   buf["combined_x"], buf["status"], bias=b)
        us = _timed_cold(fn, steps, evict, stream)
        nbytes = nb + (2 * w.num_tokens * w.hidden if b is not None else 0)
        out[label] = {"us_cold_median": round(us, 2), "bytes": nbytes,
                      "gbps_cold": round(nbytes / (us * 1e-6) / 1e9, 1)}
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    return out


def logfmt_bytes(n, h, k, p):
    """Algorithmic bytes of the LogFMT entry points: the encoder reads one bf16
    expert row and the (id, slot) entry per valid entry's row and writes its
    codes (1 B per channel) and headers (8 B per 128 channels); the LogFMT
    combine reads those codes and headers per valid entry plus idx + slot +
    weight per entry, and writes one bf16 output row per token."""
    payload = h + 8 * (h // 128)
    return {"encode": p * (2 * h + payload) + 12 * n * k,
            "combine_logfmt": p * payload + 16 * n * k + 2 * n * h}


def time_logfmt(wid, steps, scrub_bytes, say, batch=10):
    """The LogFMT combine payload on workload ``wid``: the encoder (expert
    side) and the LogFMT combine, each cold (one launch after an eviction)
    and back to back, beside the BF16 combine of the same expert outputs in
    the same run.  Expert outputs are bf16 N(0, 1) in every row."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w.scaled(w.num_tokens, 128))  # the routing; no activations needed
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    shape = ep.shape_of(w)
    N, H, K, E, S = w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.expert_capacity
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    topk_weights = torch.from_numpy(inp["topk_weights"]).to(dev)
    buf = ep.allocate(shape, dev, parts=("layout", "combine", "logfmt"))
    ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                 buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                 buf["expert_offset"], buf["workspace"], buf["status"])
    g = torch.Generator(device=dev)
    g.manual_seed(2500 + wid)
    y = torch.randn((E, S, H), dtype=torch.bfloat16, device=dev, generator=g).view(torch.int16)
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)

    def evict():
        if scrub is not None:
            torch.sum(scrub, dim=0, out=scrub_out)

    def encode():
        ep.ep_logfmt_encode(shape, y, topk_idx, buf["expert_slot"], buf["logfmt_codes"],
                            buf["logfmt_headers"], buf["status"])

    def combine_logfmt():
        ep.ep_combine_logfmt(shape, buf["logfmt_codes"], buf["logfmt_headers"], topk_idx,
                             topk_weights, buf["expert_slot"], buf["combined_x"], buf["status"])

    def combine_bf16():
        ep.ep_combine(shape, y, topk_idx, topk_weights, buf["expert_slot"], buf["combined_x"],
                      buf["status"])

    encode()
    combine_logfmt()
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    P = inp["num_valid"]
    nb = logfmt_bytes(N, H, K, P)
    nb["combine_bf16"] = algorithmic_bytes(N, H, K, E, w.num_ranks, P, w.use_fp8)["combine"]
    out = {"workload": w.name, "bytes": nb,
           "combine_bytes_saved": nb["combine_bf16"] - nb["combine_logfmt"]}
    for name, fn in (("encode", encode), ("combine_logfmt", combine_logfmt),
                     ("combine_bf16", combine_bf16)):
        say(f"{name} {w.name}: {steps} cold launches, {steps} x {batch} back to back")
        cold = _timed_cold(fn, steps, evict, stream)
        b2b = _timed_batches(fn, steps, batch, evict, stream)
        out[name] = {"us_cold_median": round(cold, 2), "us_back_to_back_mean": round(b2b, 2),
                     "gbps_back_to_back": round(nb[name] / (b2b * 1e-6) / 1e9, 1),
                     "frac_of_peak_back_to_back": round(nb[name] / (b2b * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    torch.cuda.synchronize()
    if int(buf["status"].item()) != 0:
        raise RuntimeError(f"device status {int(buf['status'].item())}")
    return out


def time_scale_formats(wid, steps, scrub_bytes, say, batch=10):
    """ep_dispatch alone on workload ``wid`` with each FP8 scale format:
    ``batch`` back-to-back launches between two events after an untimed
    eviction, ``steps`` times -> average launch duration."""
    import torch
    from combine_ep_layout_02_amd import ep
    from combine_ep_layout_02_amd import workloads as W

    w = W.WORKLOADS[wid]
    inp = W.make_inputs(w)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    topk_idx = torch.from_numpy(inp["topk_idx"]).to(dev)
    x = torch.from_numpy(inp["x_bits"].view(np.int16)).to(dev)
    scrub = torch.ones(scrub_bytes // 4, dtype=torch.float32, device=dev) if scrub_bytes else None
    scrub_out = torch.zeros((), dtype=torch.float32, device=dev)
    out = {}
    for fmt, label in ((ep.EP_SCALE_FP32, "fp32"), (ep.EP_SCALE_POW2, "pow2"),
                       (ep.EP_SCALE_UE8M0, "ue8m0")):
        shape = ep.shape_of(w, fmt)
        buf = ep.allocate(shape, dev, parts=("layout", "dispatch"))
        ep.ep_layout(shape, topk_idx, buf["num_tokens_per_rank"], buf["num_tokens_per_expert"],
                     buf["is_token_in_rank"], buf["expert_slot"], buf["rank_slot"],
                     buf["expert_offset"], buf["workspace"], buf["status"])
        say(f"ep_dispatch {w.name} scale format {label}: {steps} x {batch} launches")
        times = []
        e0, e1 = _recorded_event_pair(stream)
        for _ in range(steps):
            if scrub is not None:
                torch.sum(scrub, dim=0, out=scrub_out)
            e0.record(stream)
            for _ in range(batch):
                ep.ep_dispatch(shape, x, topk_idx, buf["expert_slot"], buf["recv_x"],
                               buf["recv_scales"], buf["recv_src_idx"], buf["status"])
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / batch)
        if int(buf["status"].item()) != 0:
            raise RuntimeError(f"device status {int(buf['status'].item())}")
        nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                               inp["num_valid"], True, fmt)["dispatch"]
        us = statistics.fmean(times)
        out[label] = {"us_mean": round(us, 2), "gbps": round(nb / (us * 1e-6) / 1e9, 1),
                      "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
        del buf
    return out


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


CPU_BASELINE_WORKLOADS = (1, 2, 3, 5, 4)


def cpu_baseline(reps, say, workloads=CPU_BASELINE_WORKLOADS):
    """The CPU oracle as it stands (plain single-threaded C) on each
    workload's own inputs: layout, pack and combine, each timed inside the C
    library on buffers allocated beforehand, so allocation is not in the
    figures.  The combine reads identity-expert outputs (each routed row holds
    its token's bf16 row, placed before timing).  Median of ``reps`` runs per
    phase; one run for the 16,384-token workload, which takes seconds.  The
    ``value`` is the prefill workload's GB/s at the sum of its phase
    medians."""
    import oracle
    from combine_ep_layout_02_amd import workloads as W

    o = oracle.get()
    per = {}
    for wid in workloads:
        w = W.WORKLOADS[wid]
        say(f"cpu oracle {w.name}: inputs")
        inp = W.make_inputs(w)
        idx, x = inp["topk_idx"], inp["x_bits"]
        lay = o.layout(idx, w.num_experts, w.num_ranks)
        S = max(1, int(lay["num_tokens_per_expert"].max()))
        y = np.zeros((w.num_experts, S, w.hidden), np.uint16)
        for k in range(w.num_topk):
            m = idx[:, k] >= 0
            y[idx[m, k], lay["expert_slot"][m, k]] = x[m]
        n = 1 if wid == 4 else reps
        runs = []
        for r in range(n):
            say(f"cpu oracle {w.name}: run {r + 1}/{n}")
            secs, st = o.timed_path(x, idx, inp["topk_weights"], y, w.num_experts, w.num_ranks, S,
                                    w.use_fp8)
            if st != 0:
                raise RuntimeError(f"oracle status {st} on {w.name}")
            runs.append(secs)
        del y
        med = [statistics.median(r[i] for r in runs) for i in range(3)]
        nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                               inp["num_valid"], w.use_fp8)
        per[w.name] = {"layout_ms": round(med[0] * 1e3, 3), "pack_ms": round(med[1] * 1e3, 3),
                       "combine_ms": round(med[2] * 1e3, 3),
                       "step_ms": round(sum(med) * 1e3, 3), "runs": n,
                       "gbps": round(nb["total"] / sum(med) / 1e9, 3)}
    head_name = "prefill_4096x7168" if "prefill_4096x7168" in per else next(iter(per))
    head = per[head_name]
    return {"value": head["gbps"], "unit": "GB/s", "cores": 1, "threads": 1, "kind": "oracle",
            "sample": f"every workload once through layout + pack + combine, median of {reps} runs "
                      f"per phase (1 for large_16384x7168); the value is {head_name} "
                      f"({head['step_ms']:.0f} ms per step); single-threaded C, phases timed "
                      "inside the library on preallocated buffers",
            "cpu_model": cpu_model(), "logical_cpus": os.cpu_count(), "per_workload": per}


# The profiling commands whose outputs the summaries in profiles/ come from.
# $REPO is the repository root, $OUT the directory a profiling run writes to
# and ${WID} the workload of a --configs-only run (4 or 5);
# `bench.py --summarize-profiles $OUT` reads that directory back.
PROFILE_COMMANDS = {
    "layouts_trace": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -T -f csv "
                     "-d $OUT/prof_layouts -o trace -- python3 $REPO/bench.py "
                     "--receive-layouts-only --steps 20 --quiet",
    "trace": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -T -f csv "
             "-d $OUT/prof_trace -o trace -- python3 $REPO/bench.py --steps 30 "
             "--warmup 5 --no-cpu-baseline --no-scale-formats --no-receive-layouts "
             "--no-other-configs --quiet",
    "configs_trace": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --kernel-trace --stats -T -f csv "
                     "-d $OUT/prof_cfg${WID}_trace -o trace -- python3 $REPO/bench.py "
                     "--configs-only ${WID} --steps 20 --warmup 3 --quiet",
    "configs_FETCH_SIZE": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -T -f csv "
                          "-d $OUT/prof_cfg${WID}_FETCH_SIZE -o pmc -- python3 $REPO/bench.py "
                          "--configs-only ${WID} --steps 3 --warmup 1 --quiet",
    "configs_WRITE_SIZE": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -T -f csv "
                          "-d $OUT/prof_cfg${WID}_WRITE_SIZE -o pmc -- python3 $REPO/bench.py "
                          "--configs-only ${WID} --steps 3 --warmup 1 --quiet",
    "FETCH_SIZE": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc FETCH_SIZE -T -f csv "
                  "-d $OUT/prof_FETCH_SIZE -o pmc -- python3 $REPO/bench.py --steps 3 "
                  "--warmup 1 --no-cpu-baseline --no-decode --no-scale-formats --no-receive-layouts "
                  "--no-other-configs --no-copy-ceiling --quiet",
    "WRITE_SIZE": "cd /tmp && export TMPDIR=/tmp && rocprofv3 --pmc WRITE_SIZE -T -f csv "
                  "-d $OUT/prof_WRITE_SIZE -o pmc -- python3 $REPO/bench.py --steps 3 "
                  "--warmup 1 --no-cpu-baseline --no-decode --no-scale-formats --no-receive-layouts "
                  "--no-other-configs --no-copy-ceiling --quiet",
}


def _grid_threads(n, h, kind):
    """Grid size (threads) of a kernel on a workload: pack and combine run one
    wave per (token, 1024-channel chunk), four waves per block; the layout
    kernels one lane per token, 256 tokens per block, and the assign kernel
    one more block (the totals) when there are several token blocks."""
    if kind in ("layout_count", "layout_assign", "layout_local"):
        blocks = max(1, -(-n // 256))
        extra = 1 if kind == "layout_assign" and blocks > 1 else 0
        return (blocks + extra) * 256
    if kind == "pack_local":  # one block per token plus the totals block
        return (n + 1) * 256
    if kind == "fused":  # one block per token plus the totals block: 512 threads up to
        # 256 tokens, 256 threads above
        return (n + 1) * (512 if n <= 256 else 256)
    return -(-(n * -(-h // 1024)) // 4) * 256


def summarize_profiles(out_dir):
    """Write short text summaries of a profiling run (the commands in
    PROFILE_COMMANDS, outputs under ``out_dir``) into profiles/: those of the
    headline runs, the receive-layout run and the other workloads' runs,
    whichever are present."""
    written = []
    if os.path.isdir(os.path.join(out_dir, "prof_trace")):
        written += summarize_headline_profiles(out_dir)
    written += summarize_layout_profiles(out_dir)
    written += summarize_config_profiles(out_dir)
    return written


def summarize_headline_profiles(out_dir):
    """Summaries of the prefill and decode kernels from the headline trace
    and counter runs (``prof_trace``, ``prof_FETCH_SIZE``, ``prof_WRITE_SIZE``)."""
    import csv

    from combine_ep_layout_02_amd import workloads as W

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def bench_json(log):
        for line in reversed(open(log).read().splitlines()):
            if line.startswith("{"):
                return json.loads(line)
        raise RuntimeError(f"no bench JSON line in {log}")

    trace = rows(os.path.join(out_dir, "prof_trace", "trace_kernel_trace.csv"))
    stats = rows(os.path.join(out_dir, "prof_trace", "trace_kernel_stats.csv"))
    pmc = {c: rows(os.path.join(out_dir, f"prof_{c}", "pmc_counter_collection.csv"))
           for c in ("FETCH_SIZE", "WRITE_SIZE")}
    digests = {bench_json(os.path.join(out_dir, f"prof_{c}.log"))["roofline"]["kernel_source_digest"]
               for c in ("FETCH_SIZE", "WRITE_SIZE", "trace")}
    if len(digests) != 1:
        raise RuntimeError("profile runs were taken on different kernel sources")
    digest = digests.pop()
    traced = bench_json(os.path.join(out_dir, "prof_trace.log"))
    # calibration: the bench's plain copy of a known size (512 MiB read, 512 MiB written)
    copy_bytes = 512 << 20
    cal = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        vals = [float(r["Counter_Value"]) for r in pmc[c] if "copyBuffer" in r["Kernel_Name"]]
        top = max(vals)
        cal[c] = (top, copy_bytes / 1024.0 / top)
    stats_txt = "\n".join(f"  {r['Name']:<48} calls={r['Calls']:>4} avg_ns={float(r['AverageNs']):>12.0f} "
                          f"min_ns={r['MinNs']:>9} max_ns={r['MaxNs']:>9}" for r in stats)
    written = []
    for wid in (3, 2):
        w = W.WORKLOADS[wid]
        inp = W.make_inputs(w.scaled(w.num_tokens, 128))
        p = inp["num_valid"]
        nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks, p,
                               w.use_fp8)
        # (kernel, grid kind, entry point, summary name); the pack is the FP8
        # instantiation of pack_kernel on dense rows
        # the prefill combine runs the multi-item kernel (more items than one
        # round of resident waves covers), the decode combine the one-item one
        nb = dict(nb, layout_dispatch=nb["layout"] + nb["dispatch"])
        # (kernel, grid kind, entry point, summary name, counter summary?);
        # the bench's step runs ep_layout_dispatch (local ranks + the pack of
        # local_kernel at prefill, the one-launch layout_pack_kernel at
        # decode), the per-entry passes run the three ordinary calls
        for kname, kind, phase, short, with_pmc in (
                ("combine_multi_kernel", "any", "combine", "combine", True),
                ("combine_kernel", "combine", "combine", "combine", True),
                ("pack_kernel", "pack", "dispatch", "pack_fp8", True),
                ("pack_local_kernel", "pack_local", "layout_dispatch", "pack_local_fp8", True),
                ("layout_local_kernel", "layout_local", "layout_dispatch", "layout_local", False),
                ("layout_assign_kernel", "layout_assign", "layout", "layout_assign", False),
                ("layout_count_kernel", "layout_count", "layout", "layout_count", False),
                ("layout_pack_kernel", "fused", "layout_dispatch", "layout_pack", False)):
            grid = None if kind == "any" else str(_grid_threads(w.num_tokens, w.hidden, kind))
            if grid is None:  # the workload's launches of this kernel, whatever their grid
                mine = [r for r in trace if r["Kernel_Name"] == kname]
                grids = {r["Grid_Size_X"] for r in mine}
                if wid != 3 or len(grids) != 1:
                    continue
                grid = grids.pop()
            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                    if r["Kernel_Name"] == kname and r["Grid_Size_X"] == grid]
            if not durs:
                continue
            ex = traced["extra"] if wid == 3 else traced["extra"]["decode_128x7168"]
            same_run = ex["kernel_avg_us_back_to_back"][phase]
            lines = [
                f"# {kname}, workload {w.name}",
                f"# N={w.num_tokens} H={w.hidden} K={w.num_topk} E={w.num_experts} R={w.num_ranks} "
                f"S={w.expert_capacity} {'FP8' if w.use_fp8 else 'BF16'} dispatch; grid {grid} threads",
                f"kernel_source_digest: {digest}",
                "",
                "## rocprofv3 kernel trace (kernel-only durations of every dispatch in the run)",
                f"command: {PROFILE_COMMANDS['trace']}",
                f"dispatches: {len(durs)}",
                f"avg_us: {statistics.fmean(durs):.2f}",
                f"median_us: {statistics.median(durs):.2f}",
                f"min_us: {min(durs):.2f}  max_us: {max(durs):.2f}",
                f"bench_avg_launch_us_same_run: {same_run['us_mean']}"
                f" ({phase} entry point, back-to-back launches timed with HIP events)",
            ]
            if wid == 3:
                lines += [f"algorithmic_bytes_per_launch ({phase} entry point): {nb[phase]}",
                          f"achieved_GBps_at_trace_avg: {nb[phase] / statistics.fmean(durs) / 1e3:.1f}"
                          if with_pmc else "achieved_GBps_at_trace_avg: n/a (one of two kernels)"]
            lines += ["", "## rocprofv3 --stats (all kernels of the run, both workloads)", stats_txt]
            path = os.path.join(PROFILES, f"{short}_{w.name}_trace.txt")
            with open(path, "w") as f:
                f.write("\n".join(lines) + "\n")
            written.append(path)
            if wid != 3 or not with_pmc:
                continue
            per = {}
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                vals = [float(r["Counter_Value"]) for r in pmc[c]
                        if r["Kernel_Name"] == kname and r["Grid_Size"] == grid]
                per[c] = statistics.median(vals)
            hbm = (per["FETCH_SIZE"] * cal["FETCH_SIZE"][1] + per["WRITE_SIZE"] * cal["WRITE_SIZE"][1]) * 1024
            lines = [
                f"# {kname}, workload {w.name}: HBM traffic from rocprofv3 counters",
                f"kernel_source_digest: {digest}",
                f"command_fetch: {PROFILE_COMMANDS['FETCH_SIZE']}",
                f"command_write: {PROFILE_COMMANDS['WRITE_SIZE']}",
                "calibration: the bench's plain copy of 512 MiB (torch copy_, __amd_rocclr_copyBuffer) "
                "reads and writes 524288 KiB",
                f"  FETCH_SIZE on the copy: {cal['FETCH_SIZE'][0]:.0f} KiB -> factor {cal['FETCH_SIZE'][1]:.4f}",
                f"  WRITE_SIZE on the copy: {cal['WRITE_SIZE'][0]:.0f} KiB -> factor {cal['WRITE_SIZE'][1]:.4f}",
                f"FETCH_SIZE_KiB_per_dispatch (median): {per['FETCH_SIZE']:.0f}",
                f"WRITE_SIZE_KiB_per_dispatch (median): {per['WRITE_SIZE']:.0f}",
                f"hbm_bytes_per_launch: {hbm:.0f}",
                f"algorithmic_bytes_per_launch: {nb[phase]}",
                f"traffic_over_algorithmic: {hbm / nb[phase]:.4f}",
            ]
            path = os.path.join(PROFILES, f"{short}_{w.name}_pmc.txt")
            with open(path, "w") as f:
                f.write("\n".join(lines) + "\n")
            written.append(path)
    return written


def summarize_config_profiles(out_dir):
    """Summaries of the large and skewed workloads' kernels from the
    ``--configs-only`` runs (``prof_cfg<WID>_trace``, ``_FETCH_SIZE``,
    ``_WRITE_SIZE`` and their logs), if present: kernel-trace durations of
    each kernel of the step, and HBM bytes per launch from the two counters,
    each scaled by its reading on the run's 512 MiB calibration copy."""
    import csv

    from combine_ep_layout_02_amd import workloads as W

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    def bench_json(log):
        for line in reversed(open(log).read().splitlines()):
            if line.startswith("{"):
                return json.loads(line)
        raise RuntimeError(f"no bench JSON line in {log}")

    written = []
    for wid in OTHER_CONFIGS:
        tdir = os.path.join(out_dir, f"prof_cfg{wid}_trace")
        if not os.path.isdir(tdir):
            continue
        w = W.WORKLOADS[wid]
        fig = bench_json(os.path.join(out_dir, f"prof_cfg{wid}_trace.log"))
        digest = fig["kernel_source_digest"]
        trace = rows(os.path.join(tdir, "trace_kernel_trace.csv"))
        inp = W.make_inputs(w.scaled(w.num_tokens, 128))
        nb = algorithmic_bytes(w.num_tokens, w.hidden, w.num_topk, w.num_experts, w.num_ranks,
                               inp["num_valid"], w.use_fp8)
        pmc = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            pdir = os.path.join(out_dir, f"prof_cfg{wid}_{c}")
            if os.path.isdir(pdir):
                pmc[c] = rows(os.path.join(pdir, "pmc_counter_collection.csv"))
                d = bench_json(os.path.join(out_dir, f"prof_cfg{wid}_{c}.log"))["kernel_source_digest"]
                if d != digest:
                    raise RuntimeError("profile runs were taken on different kernel sources")
        cal = {}
        for c, rs in pmc.items():
            top = max(float(r["Counter_Value"]) for r in rs if "copyBuffer" in r["Kernel_Name"])
            cal[c] = (top, (512 << 20) / 1024.0 / top)
        nb = dict(nb, layout_dispatch=nb["layout"] + nb["dispatch"])
        # the step's kernels (ep_layout_dispatch: local ranks, then the pack
        # that adds the prefix; ep_combine), then those of the three calls
        kernels = [("layout_local_kernel", "layout_local", "layout"),
                   ("pack_local_kernel", "pack_local", "layout_dispatch"),
                   ("layout_count_kernel", "layout_count", "layout"),
                   ("layout_assign_kernel", "layout_assign", "layout"),
                   ("pack_kernel", "pack", "dispatch"),
                   ("combine_kernel", "combine", "combine"),
                   ("combine_multi_kernel", "combine", "combine")]
        for kname, short, phase in kernels:
            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                    if r["Kernel_Name"] == kname]
            if not durs:
                continue
            grids = sorted({r["Grid_Size_X"] for r in trace if r["Kernel_Name"] == kname})
            med = statistics.median(durs)
            lines = [
                f"# {kname}, workload {w.name} (cold steps: an eviction read of 1 GiB before each)",
                f"# N={w.num_tokens} H={w.hidden} K={w.num_topk} E={w.num_experts} R={w.num_ranks} "
                f"S={w.expert_capacity} {'FP8' if w.use_fp8 else 'BF16'} dispatch; grid {', '.join(grids)} "
                "threads",
                f"kernel_source_digest: {digest}",
                "",
                "## rocprofv3 kernel trace (kernel-only durations of every dispatch in the run)",
                f"command: {PROFILE_COMMANDS['configs_trace'].replace('${WID}', str(wid))}",
                f"dispatches: {len(durs)}",
                f"avg_us: {statistics.fmean(durs):.2f}",
                f"median_us: {med:.2f}",
                f"min_us: {min(durs):.2f}  max_us: {max(durs):.2f}",
                f"bench_same_run: whole cold step {fig['figures']['us_median']} us median "
                f"({fig['figures']['frac_of_peak']} of 8 TB/s at the mean)",
            ]
            if phase != "layout":
                lines += [f"algorithmic_bytes_per_launch ({phase} entry point): {nb[phase]}",
                          f"achieved_GBps_at_trace_median: {nb[phase] / med / 1e3:.1f}"]
            elif kname == "layout_local_kernel":
                lines += [f"algorithmic_bytes_per_launch (layout outputs; the kernel writes local ranks "
                          f"that the pack completes): {nb['layout']}"]
            else:
                lines += [f"algorithmic_bytes_per_launch (layout entry point, both kernels): {nb['layout']}"]
            if len(pmc) == 2 and phase != "layout":
                per = {}
                for c, rs in pmc.items():
                    per[c] = statistics.median(float(r["Counter_Value"]) for r in rs
                                               if r["Kernel_Name"] == kname)
                hbm = (per["FETCH_SIZE"] * cal["FETCH_SIZE"][1] + per["WRITE_SIZE"] * cal["WRITE_SIZE"][1]) * 1024
                lines += [
                    "",
                    "## HBM traffic from rocprofv3 counters (one run per counter)",
                    f"command_fetch: {PROFILE_COMMANDS['configs_FETCH_SIZE'].replace('${WID}', str(wid))}",
                    f"command_write: {PROFILE_COMMANDS['configs_WRITE_SIZE'].replace('${WID}', str(wid))}",
                    "calibration: the run's plain copy of 512 MiB (torch copy_, __amd_rocclr_copyBuffer) "
                    "reads and writes 524288 KiB",
                    f"  FETCH_SIZE on the copy: {cal['FETCH_SIZE'][0]:.0f} KiB -> factor {cal['FETCH_SIZE'][1]:.4f}",
                    f"  WRITE_SIZE on the copy: {cal['WRITE_SIZE'][0]:.0f} KiB -> factor {cal['WRITE_SIZE'][1]:.4f}",
                    f"FETCH_SIZE_KiB_per_dispatch (median): {per['FETCH_SIZE']:.0f}",
                    f"WRITE_SIZE_KiB_per_dispatch (median): {per['WRITE_SIZE']:.0f}",
                    f"hbm_bytes_per_launch: {hbm:.0f}",
                    f"traffic_over_algorithmic: {hbm / nb[phase]:.4f}",
                ]
            path = os.path.join(PROFILES, f"{short}_{w.name}.txt")
            with open(path, "w") as f:
                f.write("\n".join(lines) + "\n")
            written.append(path)
    return written


def summarize_layout_profiles(out_dir):
    """Summaries of the normal-mode and expand kernels from the
    ``--receive-layouts-only`` trace run (``prof_layouts``), if present: every
    dispatch of each kernel in that run (cold single launches and
    back-to-back batches) and the figures the bench printed in the same run."""
    import csv

    tdir = os.path.join(out_dir, "prof_layouts")
    log = os.path.join(out_dir, "prof_layouts.log")
    if not os.path.isdir(tdir) or not os.path.exists(log):
        return []
    with open(os.path.join(tdir, "trace_kernel_trace.csv")) as f:
        trace = list(csv.DictReader(f))
    figures = None
    for line in reversed(open(log).read().splitlines()):
        if line.startswith("{"):
            figures = json.loads(line)
            break
    if figures is None:
        raise RuntimeError(f"no JSON line in {log}")
    rl = figures["receive_layouts_4096x7168"]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    written = []
    # in this run the per-expert kernels only serve the expand layout
    for kname, entry, short in (("pack_normal_kernel", "dispatch_normal", "pack_normal"),
                                ("combine_normal_kernel", "combine_normal", "combine_normal"),
                                ("pack_kernel", "dispatch_expand", "pack_expand"),
                                ("combine_multi_kernel", "combine_expand", "combine_expand")):
        # a dispatch right after another kernel (the eviction, or the layout
        # in a step) ran cold; one right after itself ran back to back
        cold, b2b = [], []
        for i, r in enumerate(trace):
            if r["Kernel_Name"] != kname:
                continue
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            after_self = i > 0 and trace[i - 1]["Kernel_Name"] == kname
            (b2b if after_self else cold).append(d)
        durs = sorted(cold + b2b)
        if not durs:
            continue
        nb = rl["bytes"][entry]
        med = statistics.median(cold) if cold else statistics.median(durs)
        lines = [
            f"# {kname} ({entry}), workload {rl['workload']}, expert_alignment "
            f"{rl['expert_alignment']}",
            f"kernel_source_digest: {figures['kernel_source_digest']}",
            "",
            "## rocprofv3 kernel trace (kernel-only durations of every dispatch in the run: "
            "cold single launches and back-to-back batches)",
            f"command: {PROFILE_COMMANDS['layouts_trace']}",
            f"dispatches: {len(durs)} ({len(cold)} after another kernel = cold, {len(b2b)} right "
            f"after itself = back to back)",
            f"avg_us_all: {statistics.fmean(durs):.2f}",
            f"median_us_cold: {med:.2f}",
            f"median_us_back_to_back: {statistics.median(b2b) if b2b else float('nan'):.2f}",
            f"min_us: {durs[0]:.2f}  max_us: {durs[-1]:.2f}",
            f"algorithmic_bytes_per_launch: {nb}",
            f"achieved_GBps_at_cold_median: {nb / med / 1e3:.1f}",
            f"bench_same_run: cold {rl[entry]['us_cold_median']} us (events around one launch), "
            f"back to back {rl[entry]['us_back_to_back_mean']} us",
            f"rows_sent_normal: {rl['rows_sent_normal']}  expand_rows_used: {rl['expand_rows_used']}  "
            f"expand_padding_rows: {rl['expand_padding_rows']}",
        ]
        path = os.path.join(PROFILES, f"{short}_{rl['workload']}_trace.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    gt = figures.get("gating_4096x256")
    durs = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
                  if r["Kernel_Name"] == "gate_kernel")
    if gt and durs:
        med = statistics.median(durs)
        lines = [
            f"# gate_kernel (ep_group_limited_topk), {gt['num_groups']} groups, top "
            f"{gt['topk_groups']} groups, prefill shape (4096 tokens, 256 experts, top-8)",
            f"kernel_source_digest: {figures['kernel_source_digest']}",
            "",
            "## rocprofv3 kernel trace (every dispatch in the run: cold launches and gated steps)",
            f"command: {PROFILE_COMMANDS['layouts_trace']}",
            f"dispatches: {len(durs)}",
            f"median_us: {med:.2f}",
            f"min_us: {durs[0]:.2f}  max_us: {durs[-1]:.2f}",
            f"algorithmic_bytes_per_launch: {gt['bytes']}",
            f"achieved_GBps_at_trace_median: {gt['bytes'] / med / 1e3:.1f}",
            f"bench_same_run: cold {gt['us_cold_median']} us (events around one launch); gated step "
            f"{gt['step_us_cold_with_gating']} us",
        ]
        path = os.path.join(PROFILES, "gate_prefill_4096x7168_trace.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    return written


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--scrub-mib", type=int, default=1024)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-scale-formats", action="store_true",
                    help="skip the per-variant timings (ep_dispatch per FP8 scale format, "
                         "ep_combine with the shared expert's bias, the LogFMT payload)")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the cold steps of the large and skewed workloads")
    ap.add_argument("--no-receive-layouts", action="store_true",
                    help="skip the normal-mode and expand-layout timings")
    ap.add_argument("--receive-layouts-only", action="store_true",
                    help="time only the normal-mode and expand paths (a profiling run) and print "
                         "their figures as the JSON line")
    ap.add_argument("--configs-only", metavar="WID", type=int, choices=(4, 5),
                    help="time only the cold steps of one other workload (4: large, 5: skewed) "
                         "and a 512 MiB calibration copy (a profiling run), and print their "
                         "figures as the JSON line")
    ap.add_argument("--no-copy-ceiling", action="store_true",
                    help="skip the 2 GiB plain-copy context figure (counter runs calibrate on "
                         "the bench's 512 MiB copy and must see no other copy)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ summaries from a profiling run's output directory and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        for path in summarize_profiles(args.summarize_profiles):
            print(path)
        return

    def say(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.gpus != 1:
        print(f"bench.py runs the path on one GPU; --gpus {args.gpus} is not supported "
              "(the logical EP ranks are regions of one GPU's HBM).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    from combine_ep_layout_02_amd import ep

    ep.lib()  # fail loudly if the HIP library is missing
    scrub_bytes = args.scrub_mib << 20
    if args.configs_only:
        cfg = time_config(args.configs_only, args.steps, args.warmup, scrub_bytes, say)
        torch.cuda.empty_cache()
        calibration_copy()
        print(json.dumps({"workload": OTHER_CONFIGS[args.configs_only], "figures": cfg,
                          "kernel_source_digest": kernel_source_digest()}), flush=True)
        return
    if args.receive_layouts_only:
        print(json.dumps({"receive_layouts_4096x7168": time_receive_layouts(
            3, args.steps, scrub_bytes, say),
            "gating_4096x256": time_gating(3, args.steps, scrub_bytes, say),
            "kernel_source_digest": kernel_source_digest()}), flush=True)
        return
    prefill = run_workload(3, args.steps, args.warmup, scrub_bytes, say)
    decode = None if args.no_decode else run_workload(2, args.steps, args.warmup, scrub_bytes, say)

    w = prefill["workload"]
    total_us = prefill["cold"]["us_mean"]
    value = prefill["bytes"]["total"] / (total_us * 1e-6) / 1e9
    comb_us = prefill["kernels"]["combine"]["us_mean"]
    digest = kernel_source_digest()
    roofline = {
        "bound": "hbm",
        "kernel": "combine_multi_kernel (ep_combine; 14 items per wave at this size)",
        "achieved": round(prefill["bytes"]["combine"] / (comb_us * 1e-6) / 1e9, 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(prefill["bytes"]["combine"] / (comb_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "traffic": committed_traffic(w.name, "combine", digest),
        "algorithmic_bytes_per_launch": prefill["bytes"]["combine"],
        "avg_launch_us": round(comb_us, 2),
        "kernel_source_digest": digest,
    }
    pack_us = prefill["kernels"]["dispatch"]["us_mean"]
    extra = {
        "step": "ep_layout_dispatch then ep_combine (cold: the Infinity Cache evicted before each)",
        "step_us_cold": prefill["cold"],
        "step_us_cold_three_calls": prefill["cold_three_calls"],
        "step_us_cold_hip_graph": prefill["graph_cold"],
        "step_cold_net_of_event_marker": prefill["cold_net_of_marker"],
        "phases_us_with_events_between": prefill["phases"],
        "kernel_avg_us_back_to_back": prefill["kernels"],
        "step_us_warm": prefill["warm_us_per_step"],
        "warm_steps_by_call_kind": prefill["warm"],
        "bytes_per_step": prefill["bytes"],
        "dispatch_frac_of_peak": round(prefill["bytes"]["dispatch"] / (pack_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
        "gate_60pct_of_peak_us": round(prefill["bytes"]["total"] / (0.6 * PEAK_HBM_GBPS * 1e9) * 1e6, 1),
        "frac_of_peak_whole_step": round(value / PEAK_HBM_GBPS, 4),
        "wall_s_incl_eviction": round(prefill["wall_cold_s"], 4),
    }
    if not args.no_scale_formats:
        extra["dispatch_by_scale_format_4096x7168"] = time_scale_formats(
            3, min(args.steps, 20), scrub_bytes, say)
        extra["combine_shared_expert_bias_4096x7168"] = time_combine_bias(
            3, min(args.steps, 20), scrub_bytes, say)
        for wid, key in ((3, "logfmt_combine_4096x7168"), (2, "logfmt_combine_128x7168")):
            extra[key] = time_logfmt(wid, min(args.steps, 20), scrub_bytes, say)
    if not args.no_other_configs:
        torch.cuda.empty_cache()
        for wid, key in OTHER_CONFIGS.items():
            extra[key] = time_config(wid, min(args.steps, 20), min(args.warmup, 3), scrub_bytes, say,
                                     allocations=3 if wid == 4 else 1)
            torch.cuda.empty_cache()
    if not args.no_receive_layouts:
        extra["receive_layouts_4096x7168"] = time_receive_layouts(
            3, min(args.steps, 20), scrub_bytes, say)
        extra["gating_4096x256"] = time_gating(3, min(args.steps, 20), scrub_bytes, say)
    extra["device"] = device_info()
    if not args.no_copy_ceiling:
        extra["copy_2GiB_context"] = time_copy_ceiling(min(args.steps, 20), say)
    if decode is not None:
        extra["decode_128x7168"] = {
            "step_us_cold": decode["cold"], "step_us_cold_three_calls": decode["cold_three_calls"],
            "step_us_cold_hip_graph": decode["graph_cold"],
            "step_cold_net_of_event_marker": decode["cold_net_of_marker"],
            "phases_us_with_events_between": decode["phases"],
            "kernel_avg_us_back_to_back": decode["kernels"],
            "step_us_warm": decode["warm_us_per_step"], "bytes_per_step": decode["bytes"],
            "warm_steps_by_call_kind": decode["warm"],
        }
    line = {
        "metric": "dispatch+combine achieved HBM GB/s (4096 tok x hidden 7168, FP8 dispatch, BF16 combine)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_us / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 (FP8 E4M3FN / BF16 storage)",
        "data": "synthetic (seeded numpy inputs; expert outputs bf16 N(0,1) from a seeded torch generator)",
        "config": {"workload": w.name, "num_tokens": w.num_tokens, "hidden": w.hidden,
                   "num_topk": w.num_topk, "num_experts": w.num_experts, "num_ranks": w.num_ranks,
                   "routing": "group-limited top-4 of 8 groups, top-8 experts",
                   "num_max_dispatch_tokens_per_rank": w.num_max_dispatch_tokens_per_rank,
                   "expert_capacity": w.expert_capacity, "dispatch": "fp8_e4m3fn, 1 scale / 128 ch",
                   "combine": "bf16, fp32 accumulate", "parallelism": "1 GPU, 8 logical EP ranks"},
        "roofline": roofline,
        "cpu_baseline": None,
        "extra": extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_reps, say)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
