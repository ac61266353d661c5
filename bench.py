"""Benchmark of the MoE dispatch + combine path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3_prefill]

One step = moe_route_dispatch (top-k, counts, scan, scatter/FP8) +
moe_combine over one batch of the workload's synthetic inputs, all resident
in HBM. The stand-in experts run once before timing (they are not part of
the path).
Before every step a 1 GiB scratch buffer is written so the step starts with
a cold Infinity Cache; that write is outside the timed events. Dispatch and
combine are timed with HIP events on the stream the kernels are launched on.

Each timed step is bracketed by one pair of events (an event marker in the
middle of the stream leaves a bubble of a few microseconds, so the dispatch /
combine split is measured in a second pass with a marker between the two).

Prints one JSON line. value = effective HBM GB/s = algorithmic bytes of
dispatch + combine / step time, median over steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import subprocess
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
PEAK_FP8_TFLOPS = 5000.0     # dense MFMA, fp8
PROFILES = os.path.join(ROOT, "profiles")
COMBINE_SRC = os.path.join(ROOT, "combine_moe_route_amd", "csrc", "combine.hip")
SCATTER_SRC = os.path.join(ROOT, "combine_moe_route_amd", "csrc", "dispatch.hip")
GEMM_SRC = os.path.join(ROOT, "combine_moe_route_amd", "csrc", "grouped_gemm.hip")


def algorithmic_bytes(T, H, E, k, R, fp8):
    """Bytes the method must move (no re-reads, no workspace).

    dispatch: logits 4TE + x 2TH + payload R*H*b (pad rows included)
              + scales 4R*H/128 (FP8) + topk_idx/topk_w/dst_row 12Tk + row_src 4R
    combine:  gathered rows 2Tk*H + y 2TH + dst_row/topk_w 8Tk
    """
    b = 1 if fp8 else 2
    d = 4 * T * E + 2 * T * H + R * H * b + (4 * R * (H // 128) if fp8 else 0) + 12 * T * k + 4 * R
    c = 2 * T * k * H + 2 * T * H + 8 * T * k
    return d, c


def src_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def read_traffic(kernel, workload, src_path):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/counters_<workload>.md: FETCH_SIZE and WRITE_SIZE scaled
    by a 1 GiB copy), if the counters were taken on the current kernel source;
    else None."""
    p = os.path.join(PROFILES, f"counters_{workload}.md")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m = re.search(rf"{kernel} source_sha256_16:\s*([0-9a-f]{{16}})", text)
    t = re.search(rf"{kernel} traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != src_hash(src_path):
        return None
    return float(t.group(1))


def pct(a, q):
    return float(np.percentile(np.asarray(a), q))


def run_gpu(w, steps, warmup, cold=True, sender=False):
    import torch

    from combine_moe_route_amd import (alloc_dispatch, moe_combine, moe_dispatch_max_rows,
                                       moe_harness_expert_scale, moe_route_dispatch)
    from moe_synth import gen_inputs

    dev = torch.device("cuda:0")
    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    topk_idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    bufs = alloc_dispatch(w.T, w.H, w.E, w.k, w.groups, w.row_align, w.fp8, dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    cap = moe_dispatch_max_rows(w.T, w.E, w.k, w.row_align)
    expert_out = torch.empty((cap, w.H), dtype=torch.bfloat16, device=dev)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    # stand-in experts once (outside the path, untimed)
    moe_route_dispatch(logits, x, w.k, w.groups, w.row_align, w.fp8, bufs, topk_idx, topk_w)
    moe_harness_expert_scale(bufs, topk_idx, w.E, w.fp8, expert_out=expert_out)
    torch.cuda.synchronize()
    R = int(bufs.expert_offsets[-1].item())

    stream = torch.cuda.current_stream(dev)

    def step(e=None, split=False):
        # e: events [start, after dispatch, end]; the middle one is recorded
        # only when split is set, because every event marker leaves a
        # few-microsecond bubble in the stream
        if cold:
            scratch.fill_(1)
        if e is not None:
            e[0].record(stream)
        moe_route_dispatch(logits, x, w.k, w.groups, w.row_align, w.fp8, bufs, topk_idx, topk_w)
        if split:
            e[1].record(stream)
        moe_combine(expert_out, bufs.dst_row, topk_w, y)
        if e is not None:
            e[2].record(stream)

    for _ in range(warmup):
        step()
    # timed steps: one event pair per step
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = [a[0].elapsed_time(a[2]) * 1e3 for a in ev]           # microseconds
    # split steps: dispatch (route included) / combine intervals (combine's
    # interval is the combine kernel alone: its start marker follows
    # dispatch's last kernel)
    sp = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(sp[i], split=True)
    torch.cuda.synchronize()
    disp = [a[0].elapsed_time(a[1]) * 1e3 for a in sp]
    comb = [a[1].elapsed_time(a[2]) * 1e3 for a in sp]
    out = dict(R=R, total=total, disp=disp, comb=comb, wall_s=wall)
    if sender and w.groups > 1:
        out["sender"] = run_sender(w, steps, cold, scratch, stream, expert_out, bufs, topk_idx,
                                   topk_w, y)
    return out


def run_sender(w, steps, cold, scratch, stream, expert_out, bufs, topk_idx, topk_w, y_recv):
    """Combine with sender-side partial sums (one bf16 row per token and
    destination group), timed like the main path, with its wire bytes and its
    error against the exact weighted sum on a token sample."""
    import torch

    from combine_moe_route_amd import moe_combine_recv, moe_combine_send
    dev = expert_out.device
    partial = torch.empty((w.T, w.k, w.H), dtype=torch.bfloat16, device=dev)
    count = torch.empty(w.T, dtype=torch.int32, device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(-2, steps):
        if cold:
            scratch.fill_(1)
        if i >= 0:
            ev[i][0].record(stream)
        moe_combine_send(expert_out, bufs.dst_row, topk_w, topk_idx, w.E, w.groups, partial, count)
        if i >= 0:
            ev[i][1].record(stream)
        moe_combine_recv(partial, count, y)
        if i >= 0:
            ev[i][2].record(stream)
    torch.cuda.synchronize()
    send = statistics.median([a[0].elapsed_time(a[1]) * 1e3 for a in ev])
    recv = statistics.median([a[1].elapsed_time(a[2]) * 1e3 for a in ev])
    rows = int(count.sum().item())
    # error of both variants against the exact sum, on 256 sampled tokens
    g = torch.Generator().manual_seed(0)
    toks = torch.randperm(w.T, generator=g)[:256].to(dev)
    dr = bufs.dst_row[toks].long()
    live = (dr >= 0)
    rowsv = expert_out[dr.clamp(min=0)].double()
    wts = torch.where(live, topk_w[toks].double(), torch.zeros((), dtype=torch.float64, device=dev))
    exact = (wts[:, :, None] * rowsv).sum(1)
    err_recv = (y_recv[toks].double() - exact).abs().mean().item()
    err_send = (y[toks].double() - exact).abs().mean().item()
    return dict(us_send=round(send, 2), us_recv=round(recv, 2), us_total=round(send + recv, 2),
                wire_rows=rows, wire_rows_receiver_only=int((bufs.dst_row >= 0).sum().item()),
                wire_bytes=rows * 2 * w.H,
                wire_saving=round(1 - rows / max(1, int((bufs.dst_row >= 0).sum().item())), 4),
                mean_abs_err=err_send, mean_abs_err_receiver_only=err_recv)


def time_steps(step, steps, warmup, cold, scratch, stream):
    """Median of `steps` event-timed calls of step() (cache flushed before each)."""
    import torch
    for _ in range(warmup):
        if cold:
            scratch.fill_(1)
        step()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        if cold:
            scratch.fill_(1)
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) * 1e3 for a, b in ev])


def run_grouped_gemm(w, N, steps, warmup, cold=True):
    """The grouped FP8 GEMM that consumes the dispatch's padded segments:
    every expert's rows times that expert's [N, H] E4M3 weights (128x128
    block scales). Weights are drawn on the device from a seeded torch
    generator, uniform over the finite E4M3 codes (the GEMM's speed does not
    depend on the values). Flops are counted on live rows only (2*T*k*N*H);
    the pad rows the 128-row tiles also compute count against the rate."""
    import torch

    from combine_moe_route_amd import (alloc_dispatch, moe_dispatch, moe_grouped_gemm_fp8,
                                       moe_grouped_gemm_workspace_bytes, moe_route_topk)
    from moe_synth import gen_inputs

    dev = torch.device("cuda:0")
    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    topk_idx, _ = moe_route_topk(logits, w.k)
    bufs = alloc_dispatch(w.T, w.H, w.E, w.k, w.groups, w.row_align, True, dev)
    moe_dispatch(x, topk_idx, w.E, w.groups, w.row_align, True, bufs)
    a = bufs.out.view(torch.uint8)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    wq = torch.randint(0, 254, (w.E, N, w.H), dtype=torch.uint8, device=dev, generator=g)
    for e in range(w.E):                         # skip the NaN codes 0x7F, 0xFF
        wq[e] += (wq[e] >= 0x7F).to(torch.uint8)
    ws = (torch.rand((w.E, N // 128, w.H // 128), device=dev, generator=g) + 0.5) * 2.0 ** -8
    R_cap = a.shape[0]
    y = torch.empty((R_cap, N), dtype=torch.bfloat16, device=dev)
    work = torch.empty(moe_grouped_gemm_workspace_bytes(R_cap, w.E), dtype=torch.uint8, device=dev)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    R = int(bufs.expert_offsets[-1].item())

    def step():
        moe_grouped_gemm_fp8(a, bufs.out_scales, bufs.expert_offsets, wq, ws, y, work)

    us = time_steps(step, steps, warmup, cold, scratch, stream)
    flops = 2.0 * w.T * w.k * N * w.H
    flops_padded = 2.0 * R * N * w.H
    tflops = flops / (us * 1e-6) / 1e12
    hbm = w.E * N * w.H + w.E * (N // 128) * (w.H // 128) * 4 + R * w.H + R * (w.H // 128) * 4 \
        + R * N * 2
    return dict(
        workload=w.name, N=N, K=w.H, rows=R, rows_live=w.T * w.k,
        us=round(us, 1), tflops=round(tflops, 1),
        tflops_padded_rows=round(flops_padded / (us * 1e-6) / 1e12, 1),
        roofline={"kernel": "k_grouped_gemm_fp8", "bound": "mfma", "achieved": round(tflops, 1),
                  "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                  "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                  "traffic": read_traffic("k_grouped_gemm_fp8", "grouped_gemm_" + w.name, GEMM_SRC),
                  "flops_per_launch": flops},
        hbm_bytes_algorithmic=hbm,
        hbm_gbps_algorithmic=round(hbm / (us * 1e-6) / 1e9, 1),
        weights="uniform finite E4M3 codes, block scales U[0.5,1.5)*2^-8 (seeded torch generator)",
    )


def run_graph(w, steps):
    """Route + dispatch + combine captured once in a HIP graph and replayed:
    the GPU-side time of a launch-bound step without the host's per-launch
    cost. warm = events around `steps` back-to-back replays; cold = one event
    pair per replay with the 1 GiB write before it."""
    import torch

    from combine_moe_route_amd import (alloc_dispatch, moe_combine, moe_dispatch_max_rows,
                                       moe_harness_expert_scale, moe_route_dispatch)
    from moe_synth import gen_inputs

    dev = torch.device("cuda:0")
    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    topk_idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    topk_w = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    bufs = alloc_dispatch(w.T, w.H, w.E, w.k, w.groups, w.row_align, w.fp8, dev)
    cap = moe_dispatch_max_rows(w.T, w.E, w.k, w.row_align)
    expert_out = torch.empty((cap, w.H), dtype=torch.bfloat16, device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    moe_route_dispatch(logits, x, w.k, w.groups, w.row_align, w.fp8, bufs, topk_idx, topk_w)
    moe_harness_expert_scale(bufs, topk_idx, w.E, w.fp8, expert_out=expert_out)

    def step():
        moe_route_dispatch(logits, x, w.k, w.groups, w.row_align, w.fp8, bufs, topk_idx, topk_w)
        moe_combine(expert_out, bufs.dst_row, topk_w, y)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for _ in range(20):
        g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(steps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) * 1e3 / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 200))]
    for a, b in ev:
        scratch.fill_(1)
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    cold = [a.elapsed_time(b) * 1e3 for a, b in ev]
    return dict(us_total_warm_mean=round(warm, 2), us_total_cold=round(statistics.median(cold), 2),
                us_total_cold_p10=round(pct(cold, 10), 2), us_total_cold_p90=round(pct(cold, 90), 2))


def run_routing_variants(steps, warmup, cold=True):
    """Shared expert on the 16384-token FP8 workload; load-proportional
    replicas on the skewed 4096-token workload."""
    import torch

    from combine_moe_route_amd import (alloc_dispatch, moe_combine, moe_dispatch,
                                       moe_dispatch_max_rows, moe_harness_expert_scale,
                                       moe_route_replicas, moe_route_topk, moe_route_topk_shared)
    from moe_synth import WORKLOADS, gen_inputs
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    res = {}

    # (a) one shared expert, always chosen, weight 1
    w = WORKLOADS["dsv3_prefill"]
    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    E2, k2 = w.E + 1, w.k + 1
    idx = torch.empty((w.T, k2), dtype=torch.int32, device=dev)
    wt = torch.empty((w.T, k2), dtype=torch.float32, device=dev)
    bufs = alloc_dispatch(w.T, w.H, E2, k2, 1, w.row_align, w.fp8, dev)
    eo = torch.empty((moe_dispatch_max_rows(w.T, E2, k2, w.row_align), w.H), dtype=torch.bfloat16,
                     device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    moe_route_topk_shared(logits, w.k, 1, 1.0, idx, wt)
    moe_dispatch(x, idx, E2, 1, w.row_align, w.fp8, bufs)
    moe_harness_expert_scale(bufs, idx, E2, w.fp8, expert_out=eo)
    torch.cuda.synchronize()
    R = int(bufs.expert_offsets[-1].item())

    def step_shared():
        moe_route_topk_shared(logits, w.k, 1, 1.0, idx, wt)
        moe_dispatch(x, idx, E2, 1, w.row_align, w.fp8, bufs)
        moe_combine(eo, bufs.dst_row, wt, y)
    us = time_steps(step_shared, steps, warmup, cold, scratch, stream)
    bd, bc = algorithmic_bytes(w.T, w.H, E2, k2, R, w.fp8)
    res["shared_expert"] = dict(workload=w.name, experts=E2, slots=k2, rows=R, us_total=round(us, 2),
                                gbps=round((bd + bc) / (us * 1e-6) / 1e9, 1),
                                pct_of_peak=round(100 * (bd + bc) / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2))
    del bufs, eo, x, logits, idx, wt, y

    # (b) replicas proportional to the observed load of each expert
    w = WORKLOADS["kimi_prefill"]
    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    moe_route_topk(logits, w.k, idx, wt)
    b0 = moe_dispatch(x, idx, w.E, 1, w.row_align, w.fp8)
    counts = b0.expert_counts.cpu().numpy().astype(np.int64)
    mean = w.T * w.k / w.E
    copies = np.maximum(1, np.ceil(counts / mean)).astype(np.int64)
    base = torch.from_numpy(np.concatenate([[0], np.cumsum(copies)]).astype(np.int32)).to(dev)
    Ep = int(copies.sum())
    bufs = alloc_dispatch(w.T, w.H, Ep, w.k, 1, w.row_align, w.fp8, dev)
    eo = torch.empty((moe_dispatch_max_rows(w.T, Ep, w.k, w.row_align), w.H), dtype=torch.bfloat16,
                     device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    moe_route_replicas(idx, w.E, base)
    moe_dispatch(x, idx, Ep, 1, w.row_align, w.fp8, bufs)
    moe_harness_expert_scale(bufs, idx, Ep, w.fp8, expert_out=eo)
    torch.cuda.synchronize()
    max_after = int(bufs.expert_counts.max().item())

    def step_rep():
        moe_route_topk(logits, w.k, idx, wt)
        moe_route_replicas(idx, w.E, base)
        moe_dispatch(x, idx, Ep, 1, w.row_align, w.fp8, bufs)
        moe_combine(eo, bufs.dst_row, wt, y)
    us = time_steps(step_rep, steps, warmup, cold, scratch, stream)
    bd, bc = algorithmic_bytes(w.T, w.H, Ep, w.k, w.T * w.k, w.fp8)
    res["replicas"] = dict(workload=w.name, logical_experts=w.E, physical_experts=Ep,
                           max_rows_per_expert_before=int(counts.max()),
                           max_rows_per_expert_after=max_after, us_total=round(us, 2),
                           gbps=round((bd + bc) / (us * 1e-6) / 1e9, 1))
    return res


def cu_budget(w, steps, co="bf16"):
    """Dispatch + combine restricted to N CUs through CU-masked streams, and
    the same steps overlapped with a GEMM confined to the other CUs. co =
    "bf16": a plain 8192^3 bf16 GEMM (torch.matmul); co = "grouped": the
    grouped FP8 GEMM of the expert projection (N = 4096) on a second
    micro-batch's dispatch output (seed + 1), i.e. one micro-batch's experts
    running while the other's dispatch and combine run. The last row (CUs 0)
    runs both on plain streams that share every CU."""
    import ctypes

    import torch

    from combine_moe_route_amd import (alloc_dispatch, moe_combine, moe_dispatch,
                                       moe_dispatch_max_rows, moe_harness_expert_scale,
                                       moe_route_dispatch, moe_route_topk)
    from moe_synth import gen_inputs
    hip = ctypes.CDLL("libamdhip64.so")
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    made = []

    def masked(cus):
        mask = (ctypes.c_uint32 * ((n_cu + 31) // 32))()
        for c in cus:
            mask[c // 32] |= 1 << (c % 32)
        h = ctypes.c_void_p()
        err = hip.hipExtStreamCreateWithCUMask(ctypes.byref(h), len(mask), mask)
        if err != 0:
            raise RuntimeError(f"hipExtStreamCreateWithCUMask failed: {err}")
        made.append(h)
        return torch.cuda.ExternalStream(h.value, device=dev)

    x_np, l_np = gen_inputs(w)
    x = torch.from_numpy(x_np.view(np.int16)).view(torch.bfloat16).to(dev)
    logits = torch.from_numpy(l_np).to(dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    bufs = alloc_dispatch(w.T, w.H, w.E, w.k, w.groups, w.row_align, w.fp8, dev)
    eo = torch.empty((moe_dispatch_max_rows(w.T, w.E, w.k, w.row_align), w.H), dtype=torch.bfloat16,
                     device=dev)
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
    moe_route_topk(logits, w.k, idx, wt)
    moe_dispatch(x, idx, w.E, w.groups, w.row_align, w.fp8, bufs)
    moe_harness_expert_scale(bufs, idx, w.E, w.fp8, expert_out=eo)
    torch.cuda.synchronize()
    bytes_step = sum(algorithmic_bytes(w.T, w.H, w.E, w.k, int(bufs.expert_offsets[-1].item()),
                                       w.fp8))
    gen = torch.Generator(device=dev).manual_seed(0)
    if co == "grouped":
        from combine_moe_route_amd import moe_grouped_gemm_fp8, moe_grouped_gemm_workspace_bytes
        w2 = w.with_(seed=w.seed + 1)
        x2_np, l2_np = gen_inputs(w2)
        x2 = torch.from_numpy(x2_np.view(np.int16)).view(torch.bfloat16).to(dev)
        idx2, _ = moe_route_topk(torch.from_numpy(l2_np).to(dev), w.k)
        bufs2 = alloc_dispatch(w.T, w.H, w.E, w.k, w.groups, w.row_align, True, dev)
        moe_dispatch(x2, idx2, w.E, w.groups, w.row_align, True, bufs2)
        a2 = bufs2.out.view(torch.uint8)
        gemm_n = 4096
        wq = torch.randint(0, 254, (w.E, gemm_n, w.H), dtype=torch.uint8, device=dev, generator=gen)
        for e in range(w.E):
            wq[e] += (wq[e] >= 0x7F).to(torch.uint8)
        wsc = (torch.rand((w.E, gemm_n // 128, w.H // 128), device=dev, generator=gen) + 0.5) * 2.0 ** -8
        y2 = torch.empty((a2.shape[0], gemm_n), dtype=torch.bfloat16, device=dev)
        work2 = torch.empty(moe_grouped_gemm_workspace_bytes(a2.shape[0], w.E), dtype=torch.uint8,
                            device=dev)
        gemm_name = f"grouped FP8 GEMM, second micro-batch (seed {w2.seed}), N {gemm_n}, K {w.H}"
    else:
        ga = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev, generator=gen)
        gb = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev, generator=gen)
        gc = torch.empty((8192, 8192), dtype=torch.bfloat16, device=dev)
        gemm_name = "bf16 8192x8192x8192 (torch.matmul)"
    torch.cuda.synchronize()

    def moe_step():
        moe_route_dispatch(logits, x, w.k, w.groups, w.row_align, w.fp8, bufs, idx, wt)
        moe_combine(eo, bufs.dst_row, wt, y)

    def gemm():
        if co == "grouped":
            moe_grouped_gemm_fp8(a2, bufs2.out_scales, bufs2.expert_offsets, wq, wsc, y2, work2)
        else:
            torch.matmul(ga, gb, out=gc)

    def timed(fn, reps, stream):
        with torch.cuda.stream(stream):
            fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                fn()
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    full = torch.cuda.current_stream(dev)
    t_moe_full = timed(moe_step, steps, full)
    t_gemm_full = timed(gemm, steps, full)
    gemm_reps = max(1, round(steps * t_moe_full / t_gemm_full))
    rows = []
    for n in (32, 64, 128, 192, 256, 0):
        # consecutive mask bits are spread over the XCDs (a mask that leaves an
        # XCD without CUs is rejected), so [0, n) is an even n-CU budget;
        # n = 0: two plain streams, both free to use every CU
        print(f"[bench] cu budget {n}", file=sys.stderr, flush=True)
        if n == 0:
            s_moe, s_rest = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)
            rest = True
            t_moe, t_gemm = t_moe_full, t_gemm_full
        else:
            cus = list(range(min(n, n_cu)))
            rest = list(range(min(n, n_cu), n_cu))
            s_moe = masked(cus)
            t_moe = timed(moe_step, steps, s_moe)
        row = dict(cus=n if n else "all (shared)", us_moe_step=round(t_moe, 1))
        if n:
            # the budget's own ceiling: a 1 GiB device copy on the same CUs
            with torch.cuda.stream(s_moe):
                cpy = copy_bandwidth()
            row.update(copy_GBps_on_budget=round(cpy, 1),
                       us_moe_step_at_copy_rate=round(
                           (bytes_step / (cpy * 1e9)) * 1e6, 1))
        if rest:
            if n:
                s_rest = masked(rest)
                t_gemm = timed(gemm, gemm_reps, s_rest)
            # overlap: both streams start after one marker, run concurrently
            start = torch.cuda.Event()
            start.record(full)
            s_moe.wait_event(start)
            s_rest.wait_event(start)
            e_m, e_g = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(full)
            with torch.cuda.stream(s_moe):
                for _ in range(steps):
                    moe_step()
                e_m.record(s_moe)
            with torch.cuda.stream(s_rest):
                for _ in range(gemm_reps):
                    gemm()
                e_g.record(s_rest)
            torch.cuda.synchronize()
            makespan = max(e0.elapsed_time(e_m), e0.elapsed_time(e_g)) * 1e3
            seq = steps * t_moe_full + gemm_reps * t_gemm_full
            row.update(us_gemm_on_rest=round(t_gemm, 1), us_moe_steps_end=round(e0.elapsed_time(e_m) * 1e3, 1),
                       us_gemms_end=round(e0.elapsed_time(e_g) * 1e3, 1),
                       us_makespan=round(makespan, 1), us_sequential_full_gpu=round(seq, 1),
                       overlap_speedup=round(seq / makespan, 3))
        rows.append(row)
        torch.cuda.synchronize()
        while made:
            hip.hipStreamDestroy(made.pop())
    return dict(workload=w.name, moe_steps=steps, gemm=gemm_name, gemm_reps=gemm_reps,
                us_moe_step_full_gpu=round(t_moe_full, 1), us_gemm_full_gpu=round(t_gemm_full, 1),
                budgets=rows)


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """Device-to-device copy bandwidth (read + write bytes / time) on torch's
    current stream."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(3)
    b.copy_(a)
    torch.cuda.current_stream().synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def _host_cpu():
    """(logical CPUs this process may run on, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count()
    model = "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    return n, model


def _oracle_legs(ws, x, l):
    """One oracle pass: (route+dispatch seconds, combine seconds, rows)."""
    import oracle
    t0 = time.perf_counter()
    idx, wt = oracle.route_topk(l, ws.k)
    d = oracle.dispatch(x, idx, ws.E, ws.groups, ws.row_align, ws.fp8)
    t1 = time.perf_counter()
    eo = np.ascontiguousarray(x[np.maximum(d.row_src, 0) // ws.k])
    t2 = time.perf_counter()
    oracle.combine(eo, d.dst_row, wt)
    t3 = time.perf_counter()
    return t1 - t0, t3 - t2, d.num_rows


def cpu_baseline(w, max_tokens, reps=3):
    """The CPU oracle as it stands on a bounded token sample of the same
    workload: routing + dispatch + combine, its experts replaced by the token
    rows themselves (identity) so no oracle time goes to them. Two builds of
    the one source: single-threaded, and OpenMP over tokens (the histogram and
    the scan stay serial) on every host thread it is given. Each leg's time is
    the median of reps runs; value is the OpenMP build's rate."""
    import oracle
    from moe_synth import gen_inputs
    ws = w.with_(T=min(w.T, max_tokens))
    x, l = gen_inputs(ws)
    n_cpu, model = _host_cpu()
    legs = {}
    prev = oracle.variant()
    try:
        for v in ("plain", "omp"):
            oracle.set_variant(v)
            runs = [_oracle_legs(ws, x, l) for _ in range(reps)]
            td = float(np.median([r[0] for r in runs]))
            tc = float(np.median([r[1] for r in runs]))
            bd, bc = algorithmic_bytes(ws.T, ws.H, ws.E, ws.k, runs[0][2], ws.fp8)
            legs[v] = dict(value=round((bd + bc) / (td + tc) / 1e9, 4), threads=oracle.threads(),
                           route_dispatch_s=round(td, 4), combine_s=round(tc, 4))
    finally:
        oracle.set_variant(prev)
    par, one = legs["omp"], legs["plain"]
    return dict(value=par["value"], unit="GB/s", cores=par["threads"], kind="oracle",
                sample=(f"{ws.T} of {w.T} tokens of {w.name} (H={ws.H}, E={ws.E}, k={ws.k}); "
                        f"C oracle built with OpenMP, {par['threads']} threads; median of {reps} "
                        f"runs per leg: route+dispatch {par['route_dispatch_s']:.3f} s, "
                        f"combine {par['combine_s']:.3f} s"),
                single_thread=dict(value=one["value"], unit="GB/s", cores=1,
                                   route_dispatch_s=one["route_dispatch_s"],
                                   combine_s=one["combine_s"]),
                host=dict(nproc=n_cpu, cpu_model=model))


def summarize(w, r):
    bd, bc = algorithmic_bytes(w.T, w.H, w.E, w.k, r["R"], w.fp8)
    tot = r["total"]
    dmed = statistics.median(r["disp"])
    cmed = statistics.median(r["comb"])
    tmed = statistics.median(tot)
    return dict(
        bytes_dispatch=bd, bytes_combine=bc, rows=r["R"],
        us_dispatch=round(dmed, 2), us_combine=round(cmed, 2), us_total=round(tmed, 2),
        us_total_p10=round(pct(tot, 10), 2), us_total_p90=round(pct(tot, 90), 2),
        gbps=round((bd + bc) / (tmed * 1e-6) / 1e9, 1),
        gbps_dispatch=round(bd / (dmed * 1e-6) / 1e9, 1),
        gbps_combine=round(bc / (cmed * 1e-6) / 1e9, 1),
        pct_of_peak=round(100 * (bd + bc) / (tmed * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2),
    )


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--also", default="kimi_prefill",
                    help="comma-separated extra workloads reported under 'other' ('' for none)")
    ap.add_argument("--decode", default="mixtral_decode,dsv3_decode",
                    help="decode workloads reported under 'decode', cold and warm ('' for none)")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--warm", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the routing-variant measurements reported under 'next'")
    ap.add_argument("--cpu-tokens", type=int, default=16384)
    ap.add_argument("--gemm-n", type=int, default=4096,
                    help="output width of the grouped FP8 GEMM leg (0 skips it)")
    ap.add_argument("--gemm-only", action="store_true",
                    help="only run the grouped FP8 GEMM leg")
    ap.add_argument("--cu-budget", action="store_true",
                    help="only run the CU-budget / overlap experiment")
    ap.add_argument("--cu-budget-gemm", default="bf16", choices=("bf16", "grouped"),
                    help="co-runner of the CU-budget experiment")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run 1 GiB device copies (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this path runs on one GPU; multi-GPU runs are not part of "
                                   "it (the path shards by tokens; each GPU would run this "
                                   "same step on its own share)", "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    from moe_synth import WORKLOADS

    if args.cu_budget:
        print(json.dumps({"cu_budget": cu_budget(WORKLOADS[args.workload], args.steps,
                                                 args.cu_budget_gemm)}), flush=True)
        return

    if args.calib_copy:
        print(json.dumps({"copy_GBps": round(copy_bandwidth(), 1), "bytes_per_copy": 1 << 30}),
              flush=True)
        return

    w = WORKLOADS[args.workload]
    if args.gemm_only:
        print(json.dumps({"grouped_gemm_fp8": run_grouped_gemm(w, args.gemm_n or 4096, args.steps,
                                                               args.warmup, cold=not args.warm)}),
              flush=True)
        return
    print(f"[bench] {w.name}: T={w.T} H={w.H} E={w.E} k={w.k} G={w.groups} A={w.row_align} "
          f"fp8={w.fp8} steps={args.steps} warmup={args.warmup}", file=sys.stderr, flush=True)
    r = run_gpu(w, args.steps, args.warmup, cold=not args.warm, sender=True)
    s = summarize(w, r)
    print(f"[bench] {json.dumps(s)}", file=sys.stderr, flush=True)

    others = {}
    for name in [n for n in args.also.split(",") if n and n != w.name]:
        wo = WORKLOADS[name]
        print(f"[bench] {name}", file=sys.stderr, flush=True)
        others[name] = summarize(wo, run_gpu(wo, args.steps, args.warmup, cold=not args.warm))
    # Decode batches (128 tokens): launch- and latency-bound, their working
    # sets fit the 256 MB Infinity Cache, so both a cold (1 GiB write before
    # each step) and a warm figure are given.
    decode = {}
    for name in [n for n in args.decode.split(",") if n]:
        wd = WORKLOADS[name]
        print(f"[bench] {name} (decode, {args.decode_steps} steps)", file=sys.stderr, flush=True)
        cold_s = summarize(wd, run_gpu(wd, args.decode_steps, 20, cold=True))
        warm_s = summarize(wd, run_gpu(wd, args.decode_steps, 20, cold=False))
        keys = ("us_dispatch", "us_combine", "us_total", "us_total_p10",
                "us_total_p90", "gbps")
        decode[name] = dict(rows=cold_s["rows"], bytes_total=cold_s["bytes_dispatch"] + cold_s["bytes_combine"],
                            cold={k: cold_s[k] for k in keys}, warm={k: warm_s[k] for k in keys},
                            graph=run_graph(wd, args.decode_steps))
    copy_gbps = round(copy_bandwidth(), 1)

    comb_avg_us = statistics.mean(r["comb"])
    achieved = s["bytes_combine"] / (comb_avg_us * 1e-6) / 1e9
    traffic = read_traffic("k_combine", w.name, COMBINE_SRC)

    out = {
        "metric": "dispatch+combine µs and effective HBM GB/s (% of peak), 1 MI355X",
        "value": s["gbps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(s["us_total"] / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 dispatch / bf16 combine, fp32 math" if w.fp8 else "bf16, fp32 math",
        "data": "synthetic (seeded numpy; x~N(0,1) bf16, logits~N(0,1) fp32)",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "k": w.k,
                   "groups": w.groups, "row_align": w.row_align,
                   "cache": "warm" if args.warm else "cold (1 GiB write before each step)"},
        "us_dispatch": s["us_dispatch"],
        "us_combine": s["us_combine"], "us_total": s["us_total"],
        "us_total_p10": s["us_total_p10"], "us_total_p90": s["us_total_p90"],
        "pct_of_peak": s["pct_of_peak"],
        "gbps_dispatch": s["gbps_dispatch"], "gbps_combine": s["gbps_combine"],
        "bytes": {"dispatch": s["bytes_dispatch"], "combine": s["bytes_combine"], "rows": s["rows"]},
        "copy_GBps_measured": copy_gbps,
        "wall_s_timed_region": round(r["wall_s"], 4),
        "roofline": {"kernel": "k_combine", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "us_avg": round(comb_avg_us, 2)},
        "other": others,
        "decode": decode,
        "next": {"sender_side_combine": r.get("sender")},
    }
    if not args.no_variants:
        print("[bench] routing variants", file=sys.stderr, flush=True)
        out["next"].update(run_routing_variants(args.steps, args.warmup, cold=not args.warm))
    if args.gemm_n and w.fp8:
        print("[bench] grouped FP8 GEMM", file=sys.stderr, flush=True)
        out["next"]["grouped_gemm_fp8"] = run_grouped_gemm(w, args.gemm_n, args.steps,
                                                          args.warmup, cold=not args.warm)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
