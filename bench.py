#!/usr/bin/env python3
"""Effective HBM bandwidth of the fused Q4_K dequantize-GEMV on one MI355X.

Workload (one "step" = one decoded token's weight stream at batch 1): the
TinyLlama-1.1B-shaped Q4_K projections of 22 layers (q, o 2048x2048; k, v
256x2048; gate, up 5632x2048; down 2048x5632) followed by the 2048->32000 LM
head: 155 GEMVs, 582 MB of distinct packed weights (more than the 256 MB
last-level cache, so every step streams them from HBM). Weights, activations
and outputs are seeded synthetic data resident in HBM before timing starts.

Weights are held in the library's tile-major order (every 64-row tile stored
block column by block column; qwg_pack_q4k_tiles repacks the row-major tensors
once, before timing; each 144-byte block is unchanged, and the byte count is the
same because every shape here is a whole number of tiles). The headline runs the
step as one grouped launch through the C ABI (qwg_group_run over the 155
independent GEMVs). Further schedules of the same step are timed and reported
beside it: "grouped_row_major" (the same launch on the row-major tensors),
"layered" (the launches a decoder whose layers depend on each other would make:
per layer q|k|v grouped, o, gate|up grouped, down; then the LM head: 89
launches) and "per_call" (155 qwg_gemv_q4k_tiled calls).

Reported: value = algorithmic bytes of the step (weights + x + y) / wall time
per step, in GB/s; the roofline object for the grouped kernel (algorithmic bytes
/ average launch time from HIP events on its stream around the timed loop of
back-to-back launches); and the CPU oracle's throughput on the host cores
(cpu_baseline).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--headline-only]
       python bench.py --workload iq3_stream|iq3_xxs|codebooks|encode|lm_head [--steps K] [--warmup W]
The second form measures the other hot-path rows on their own (one JSON line each, for the
record and for profiling): "iq3_stream" = the same 155 GEMV shapes in the IQ3 container as one
grouped launch (IQ3 tile layout; the row-major launch beside it); "iq3_xxs" = IQ3_XXS blocks in
llama.cpp's byte order (single GEMVs row-major and repacked, and the stream repacked); "codebooks" =
the same stream and single shapes in IQ3_S and IQ4_XS (tile layout); "encode" = the IQ3 container
encoder on the IQ3 configuration's matrices (an ALU-bound roofline); "lm_head" = the 32000x2048 Q4_K LM head at batch 1..8 (qwg_gemv_q4k,
qwg_gemv_q4k_tiled, qwg_gemm_q4k), cycling over enough weight copies that every launch streams
from HBM rather than the last-level cache.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ["quantized_weight_decode_gemv_amd/csrc/q4k.hip",
                  "quantized_weight_decode_gemv_amd/csrc/qwg_device.h",
                  "quantized_weight_decode_gemv_amd/csrc/qwg_internal.h"]
# HBM bytes per grouped launch of the stream (tile layout), from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE
# runs of this script, each scaled by the same counter on a plain device copy of known size
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0; see profiles/q4k_stream_c5_grouped.md). Valid only for
# the kernel sources with this hash; otherwise traffic is reported as null.
TRAFFIC = {"sources_sha256": "8a57f09c07b571c93b58da4189b9872cba6a05b5229ec48c661a85c9721536bc",
           "fetch_bytes": 594760417, "write_bytes": 1704960}


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes():
    if TRAFFIC["sources_sha256"] and TRAFFIC["sources_sha256"] == kernel_sources_sha256():
        return TRAFFIC["fetch_bytes"] + TRAFFIC["write_bytes"]
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The clocks take ~150-200 back-to-back steps (~20 ms) to settle (measured: launches 1-50
    # average 113 us, 151-200 95 us, then 89-92 us), so the default warm-up covers that.
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time budget for the oracle baseline")
    ap.add_argument("--print-kernel-hash", action="store_true",
                    help="print the hash of the kernel sources the traffic figure is tied to")
    ap.add_argument("--workload", default="q4k_stream",
                    choices=["q4k_stream", "iq3_stream", "iq3_xxs", "codebooks", "encode", "lm_head",
                             "batched"],
                    help="q4k_stream: the headline (default); the others: see the module docstring")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline launch (no row-major, layered or per-call "
                         "schedules), so a kernel trace holds nothing else of that kernel")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 10 plain device-to-device copies of MIB "
                         "MiB (reference for scaling hardware traffic counters) and exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_copy": 4 * n,
                      "copy_calibration_bytes_written_per_copy": 4 * n, "copies": 10}), flush=True)


def main():
    args = parse()
    if args.print_kernel_hash:
        print(kernel_sources_sha256())
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the GEMV path has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.workload == "iq3_stream":
        bench_iq3_stream(args)
        return
    if args.workload == "lm_head":
        bench_lm_head(args)
        return
    if args.workload == "iq3_xxs":
        bench_iq3_xxs(args)
        return
    if args.workload == "codebooks":
        bench_codebooks(args)
        return
    if args.workload == "encode":
        bench_encode(args)
        return
    if args.workload == "batched":
        bench_batched(args)
        return

    import numpy as np
    import torch

    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = qwg.lib()

    probs = synth.config(5)
    t0 = time.time()
    host_w = [synth.weights(p) for p in probs]
    host_x = [synth.inputs(p) for p in probs]
    W = [torch.from_numpy(w).to(dev) for w in host_w]
    X = [torch.from_numpy(x).to(dev) for x in host_x]
    Y = [torch.empty(p.n_out, dtype=torch.float32, device=dev) for p in probs]
    WT = [qwg.pack_q4k_tiles(w, p.n_in) for p, w in zip(probs, W)]
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream(dev)
    sptr = ctypes.c_void_p(stream.cuda_stream)
    step_bytes = sum(p.algorithmic_bytes for p in probs)
    weight_bytes = sum(p.weight_bytes for p in probs)

    group = qwg.Q4kGroup(zip(WT, X, Y), tiled=True)
    Y_rows = [torch.empty_like(y) for y in Y]
    group_rows = qwg.Q4kGroup(zip(W, X, Y_rows))
    layered = []
    i = 0
    while i < len(probs):
        name = probs[i].name.split(".")[-1]
        if name in ("q", "gate"):
            n = 3 if name == "q" else 2
            layered.append(qwg.Q4kGroup(zip(WT[i:i + n], X[i:i + n], Y[i:i + n]), tiled=True))
            i += n
        else:
            layered.append(qwg.Q4kGroup([(WT[i], X[i], Y[i])], tiled=True))
            i += 1
    calls = [(y.data_ptr(), x.data_ptr(), w.data_ptr(), p.n_in, p.n_out)
             for p, w, x, y in zip(probs, WT, X, Y)]
    gemv = L.qwg_gemv_q4k_tiled

    def step_grouped():
        group.run(stream)

    def step_layered(s=stream):
        for g in layered:
            g.run(s)

    def step_per_call(s=stream):
        sp = ctypes.c_void_p(s.cuda_stream)
        for yp, xp, wp, n_in, n_out in calls:
            rc = gemv(yp, xp, wp, n_in, n_out, sp)
            if rc:
                raise RuntimeError(f"qwg_gemv_q4k_tiled failed: {rc}")

    def graph_of(fn):
        """fn(stream) captured once in a HIP graph on a side stream; one eager call
        there first sets up that stream's split-sum workspace (no allocation or
        memset is recorded). Returns the graph and whether three replays, with
        eager runs in between, each reproduced the eager outputs bit for bit."""
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            fn(side)
        torch.cuda.synchronize()
        ok = True
        for _ in range(3):
            fn(stream)
            torch.cuda.synchronize()
            ref = [y.clone() for y in Y]
            for y in Y:
                y.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            ok = ok and all(torch.equal(a, b) for a, b in zip(ref, Y))
        return graph, ok

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    # Headline: wall clock over the timed loop. Roofline: HIP events on the
    # launch stream around the same loop (back-to-back launches, so this is the
    # average launch duration). An event pair around every launch inflates
    # the figure by ~10 us: the markers between launches break the
    # back-to-back dispatch.
    for _ in range(args.warmup):
        step_grouped()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step_grouped()
    ev1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = 1e3 * sec
    value = step_bytes / sec / 1e9
    achieved = step_bytes / (kernel_ms * 1e-3) / 1e9

    schedules = {}
    if not args.headline_only:
        sec_rows = timed(lambda: group_rows.run(stream), args.steps, args.warmup)
        sec_layered = timed(step_layered, max(5, args.steps // 5), 2)
        sec_percall = timed(step_per_call, max(5, args.steps // 5), 2)
        # The same two schedules replayed from HIP graphs (the launches are
        # recorded once; the GPU still runs one kernel per launch).
        graph_layered, ok_layered = graph_of(step_layered)
        graph_percall, ok_percall = graph_of(step_per_call)
        sec_layered_g = timed(graph_layered.replay, max(5, args.steps // 5), 2)
        sec_percall_g = timed(graph_percall.replay, max(5, args.steps // 5), 2)

    def sched(sec_, launches):
        return {"us_per_step": round(1e6 * sec_, 1), "GBps": round(step_bytes / sec_ / 1e9, 1),
                "pct_of_hbm_peak": round(100 * step_bytes / sec_ / 1e9 / HBM_PEAK_GBS, 1),
                "tokens_per_s": round(1.0 / sec_, 1), "launches": launches}

    schedules["grouped"] = sched(sec, 1)
    if not args.headline_only:
        schedules["grouped_row_major"] = sched(sec_rows, 1)
        schedules["layered"] = sched(sec_layered, len(layered))
        schedules["per_call"] = sched(sec_percall, len(calls))
        schedules["layered_graph"] = dict(sched(sec_layered_g, len(layered)),
                                          replays_match_eager=ok_layered)
        schedules["per_call_graph"] = dict(sched(sec_percall_g, len(calls)),
                                           replays_match_eager=ok_percall)

    result = {
        "metric": "effective HBM GB/s (% of MI355X peak) for Q4_K/IQ3 GEMV, batch 1",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "TinyLlama-1.1B Q4_K per-token weight stream, batch 1: 22 layers x "
                        "(q,o 2048x2048; k,v 256x2048; gate,up 5632x2048; down 2048x5632) + "
                        "LM head 32000x2048 = 155 GEMVs, one grouped launch (qwg_group_run), "
                        "weights in tile-major order",
            "layout": "tile-major Q4_K (qwg_pack_q4k_tiles, repacked once before timing)",
            "weight_bytes": weight_bytes,
            "algorithmic_bytes_per_step": step_bytes,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(1e3 / ms_per_step, 1),
            "tiles_per_launch": group.workgroups,
            "setup_s": round(setup_s, 1),
            "schedules": schedules,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_bytes(),
            "kernel": "q4k_stream_kernel<4,2> (grouped, 155 GEMVs per launch, tile layout)",
            "bytes_per_launch": step_bytes,
            "kernel_us": round(1e3 * kernel_ms, 2),
        },
    }

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(probs, host_w, host_x,
                                              (Y,) if args.headline_only else (Y, Y_rows),
                                              args.cpu_seconds)
    print(json.dumps(result), flush=True)


def _event_us(fn, stream, steps, warmup):
    """Average time of fn() over `steps` back-to-back calls, from HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / steps


def _graph_us(call, n, stream, rounds):
    """Device time per call of call(0..n-1) captured once in a HIP graph (on a side
    stream, after one eager pass there sets up its split-sum workspace) and
    replayed `rounds` times back to back, from HIP events on `stream`: the
    kernels' own rate without the host's per-call cost. Also returns whether a
    replay left the outputs the eager pass wrote."""
    import torch
    side = torch.cuda.Stream(stream.device)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        outs = [call(k) for k in range(n)]
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for k in range(n):
            call(k)
    torch.cuda.synchronize()
    for o in outs:
        o.fill_(float("nan"))
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(a, b) for a, b in zip(ref, outs))
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(rounds):
        graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    return 1e3 * a.elapsed_time(b) / (rounds * n), same


def bench_iq3_stream(args):
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probs = synth.config(6)
    grid = torch.from_numpy(synth.iq3_grid()).to(dev)
    W = [torch.from_numpy(synth.weights(p)).to(dev) for p in probs]
    X = [torch.from_numpy(synth.inputs(p)).to(dev) for p in probs]
    Y = [torch.empty(p.n_out, dtype=torch.float32, device=dev) for p in probs]
    WT = [qwg.pack_iq3_tiles(w, p.n_in) for p, w in zip(probs, W)]
    group = qwg.Iq3Group(zip(WT, X, Y), grid, tiled=True)
    group_rows = qwg.Iq3Group(zip(W, X, [torch.empty_like(y) for y in Y]), grid)
    stream = torch.cuda.current_stream(dev)
    step_bytes = sum(p.algorithmic_bytes for p in probs)
    us = _event_us(lambda: group.run(stream), stream, args.steps, args.warmup)
    us_rows = _event_us(lambda: group_rows.run(stream), stream, args.steps, args.warmup)
    gbs = step_bytes / us / 1e3
    print(json.dumps({
        "metric": "effective HBM GB/s, IQ3 GEMV stream, batch 1", "value": round(gbs, 2),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 4), "higher_is_better": True, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "TinyLlama-1.1B-shaped per-token stream in the 98-byte IQ3 "
                               "container: 155 GEMVs, one grouped launch (qwg_group_run), "
                               "weights in the IQ3 tile layout",
                   "layout": "IQ3 tile layout (qwg_pack_iq3_tiles, repacked once before timing)",
                   "algorithmic_bytes_per_step": step_bytes,
                   "row_major_us": round(us_rows, 2),
                   "row_major_GBs": round(step_bytes / us_rows / 1e3, 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "kernel": "iq3_stream_kernel<8,2,tile layout> (grouped)",
                     "kernel_us": round(us, 2)}}), flush=True)


def bench_iq3_xxs(args):
    """IQ3_XXS blocks in llama.cpp's byte order: the two single GEMV shapes of the
    IQ3 configuration (5632x2048, 2048x5632; cold weights, copies cycled), row-major
    in that order, row-major in the container order, and repacked to the tile
    layout (also replayed from a HIP graph, which leaves out the host's per-call
    cost); then the per-token stream's 155 GEMVs repacked from that order as one
    grouped launch."""
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    grid = torch.from_numpy(synth.iq3_xxs_grid()).to(dev)
    copies = 64  # 64 x 4.4 MB: more than the last-level cache
    singles = {}
    i = [0]

    def cycle(fn):
        def run():
            fn(i[0] % copies)
            i[0] += 1
        return run

    for p in synth.config(4):
        wx = torch.from_numpy(synth.iq3_xxs_weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev)
        w5 = torch.from_numpy(synth.weights(p)).to(dev)
        x = torch.from_numpy(synth.inputs(p)).to(dev)
        y = torch.empty(p.n_out, device=dev)
        WX = wx.reshape(1, -1).repeat(copies, 1)
        W5 = w5.reshape(1, -1).repeat(copies, 1)
        WT = torch.stack([qwg.pack_iq3_xxs_tiles(wx, p.n_in)] * copies)
        us_x = _event_us(cycle(lambda k: qwg.gemv_iq3_xxs(WX[k], x, grid, out=y)), stream,
                         args.steps, args.warmup)
        us_5 = _event_us(cycle(lambda k: qwg.gemv_iq3(W5[k], x, grid, out=y)), stream,
                         args.steps, args.warmup)
        us_t = _event_us(cycle(lambda k: qwg.gemv_iq3_tiled(WT[k], x, grid, p.n_out, out=y)),
                         stream, args.steps, args.warmup)
        # the same calls replayed from a HIP graph (one output per copy, so the
        # replay can be checked against the eager pass)
        YG = torch.empty(copies, p.n_out, device=dev)
        us_g, same = _graph_us(lambda k: qwg.gemv_iq3_tiled(WT[k], x, grid, p.n_out, out=YG[k]),
                               copies, stream, max(1, args.steps // copies) * 4)
        b = p.algorithmic_bytes
        singles[p.name] = {"xxs_rows_us": round(us_x, 2), "xxs_rows_GBs": round(b / us_x / 1e3, 1),
                           "container_rows_us": round(us_5, 2),
                           "xxs_tiled_us": round(us_t, 2), "xxs_tiled_GBs": round(b / us_t / 1e3, 1),
                           "xxs_tiled_graph_us": round(us_g, 2),
                           "xxs_tiled_graph_GBs": round(b / us_g / 1e3, 1),
                           "graph_replays_match_eager": same}
        del YG
        del WX, W5, WT

    probs = synth.config(6)
    X = [torch.from_numpy(synth.inputs(p)).to(dev) for p in probs]
    Y = [torch.empty(p.n_out, dtype=torch.float32, device=dev) for p in probs]
    WT = [qwg.pack_iq3_xxs_tiles(torch.from_numpy(
        synth.iq3_xxs_weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev), p.n_in) for p in probs]
    group = qwg.Iq3Group(zip(WT, X, Y), grid, tiled=True)
    step_bytes = sum(p.algorithmic_bytes for p in probs)
    us = _event_us(lambda: group.run(stream), stream, args.steps, args.warmup)
    gbs = step_bytes / us / 1e3
    print(json.dumps({
        "metric": "effective HBM GB/s, IQ3_XXS (llama.cpp byte order) GEMV stream, batch 1",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 4), "higher_is_better": True,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "TinyLlama-1.1B-shaped per-token stream of IQ3_XXS blocks in "
                               "llama.cpp's byte order, repacked once (qwg_pack_iq3_xxs_tiles) "
                               "and run as one grouped launch; single GEMVs of the IQ3 "
                               "configuration beside it",
                   "algorithmic_bytes_per_step": step_bytes, "singles": singles},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "kernel": "iq3_stream_kernel<8,2,tile layout> (grouped)",
                     "kernel_us": round(us, 2)}}), flush=True)


def bench_codebooks(args):
    """IQ3_S and IQ4_XS (codebook.py page): the per-token stream's 155 GEMV
    shapes in each format, repacked to the tile layout, as one grouped launch;
    and the two single GEMV shapes of the IQ3 configuration with cold weights."""
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    fmts = {"iq3s": (synth.iq3s_weights, synth.iq3s_grid, 110, qwg.pack_iq3s_tiles,
                     qwg.gemv_iq3s_tiled, qwg.Iq3sGroup),
            "iq4xs": (synth.iq4xs_weights, synth.iq4nl_table, 136, qwg.pack_iq4xs_tiles,
                      qwg.gemv_iq4xs_tiled, qwg.Iq4xsGroup)}
    out = {}
    for name, (weights, table, nbytes, pack, gemv, Group) in fmts.items():
        tab = torch.from_numpy(table()).to(dev)
        probs = synth.config(6)
        X = [torch.from_numpy(synth.inputs(p)).to(dev) for p in probs]
        Y = [torch.empty(p.n_out, device=dev) for p in probs]
        W = [pack(torch.from_numpy(weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev), p.n_in)
             for p in probs]
        group = Group(zip(W, X, Y), tab)
        step = sum(p.n_out * (p.n_in // 256) * nbytes + 4 * (p.n_in + p.n_out) for p in probs)
        us = _event_us(lambda: group.run(stream), stream, args.steps, args.warmup)
        group.close()
        del W
        singles = {}
        copies = 64
        for p in synth.config(4):
            wt = pack(torch.from_numpy(weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev), p.n_in)
            WT = torch.stack([wt] * copies)
            x = torch.from_numpy(synth.inputs(p)).to(dev)
            y = torch.empty(p.n_out, device=dev)
            i = [0]

            def run():
                gemv(WT[i[0] % copies], x, tab, p.n_out, out=y)
                i[0] += 1
            u = _event_us(run, stream, args.steps, args.warmup)
            b = p.n_out * (p.n_in // 256) * nbytes + 4 * (p.n_in + p.n_out)
            singles[p.name] = {"us": round(u, 2), "GBs": round(b / u / 1e3, 1)}
            del WT
        out[name] = {"stream_us": round(us, 2), "stream_GBs": round(step / us / 1e3, 1),
                     "frac": round(step / us / 1e3 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_step": step, "singles": singles}
    best = max(out.values(), key=lambda v: v["stream_GBs"])
    print(json.dumps({
        "metric": "effective HBM GB/s, IQ3_S / IQ4_XS GEMV stream, batch 1",
        "value": best["stream_GBs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "TinyLlama-1.1B-shaped per-token stream (155 GEMVs) in the IQ3_S and "
                               "IQ4_XS formats, tile layout, one grouped launch each; single GEMVs "
                               "of the IQ3 configuration's shapes, cold weights", **out},
    }), flush=True)


# Vector-ALU operations per weight of the IQ3 encoder's search (the rest is
# negligible): 16 codes x 256 grid rows per group of four weights, each row
# 4 multiplies + 3 adds (q.g), a doubling and a subtract (g2 - 2 q.g), a
# compare and two selects (the running minimum) = 12 operations.
ENCODE_OPS_PER_WEIGHT = 16 * 256 * 12 / 4
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz: a wave64 fp32 instruction issues in
# two cycles on MI355X (the vendor's 157.3 TFLOP/s fp32 vector figure is this
# rate counting an FMA as two; the encoder itself sustains 0.45 wave64
# instructions per SIMD-cycle, more than a four-cycle issue allows). Its
# search uses no packed or fused forms.
VALU_PEAK_OPS = 256 * 4 * 32 * 2.4e9


def bench_encode(args):
    """The IQ3 container encoder on the IQ3 configuration's two matrices
    (5632x2048, 2048x5632) of seeded N(0, 0.02) weights."""
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    grid = torch.from_numpy(synth.iq3_grid()).to(dev)
    res = {}
    total_w, total_us = 0, 0.0
    steps, warm = max(3, args.steps // 30), max(2, args.warmup // 100)
    for p in synth.config(4):
        g = torch.Generator(device="cpu").manual_seed(180 + p.tensor)
        x = (torch.randn(p.n_out, p.n_in, generator=g) * 0.02).to(dev)
        out = torch.empty(p.n_out, p.n_in // 256 * 98, dtype=torch.uint8, device=dev)
        us = _event_us(lambda: qwg.encode_iq3(x, grid, out=out), stream, steps, warm)
        n = p.n_out * p.n_in
        res[p.name] = {"us": round(us, 1), "Mweights_per_s": round(n / us, 1)}
        total_w += n
        total_us += us
    ops = ENCODE_OPS_PER_WEIGHT * total_w / (total_us * 1e-6)
    print(json.dumps({
        "metric": "IQ3 container encode throughput (weights/s)",
        "value": round(total_w / total_us * 1e6, 1), "unit": "weights/s", "n_gpus": 1,
        "steps": steps, "warmup": warm, "higher_is_better": True, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwg_encode_iq3 on 5632x2048 and 2048x5632 N(0, 0.02) fp32 weights",
                   **res},
        "roofline": {"bound": "alu", "achieved": round(ops / 1e12, 2), "peak": VALU_PEAK_OPS / 1e12,
                     "unit": "Tops/s", "frac": round(ops / VALU_PEAK_OPS, 4),
                     "ops_per_weight": ENCODE_OPS_PER_WEIGHT, "kernel": "iq3_encode_kernel"},
    }), flush=True)


def bench_lm_head(args):
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    p = synth.config(3)[0]
    w = torch.from_numpy(synth.weights(p)).to(dev)
    copies = 16  # 16 x 36.9 MB: more than the last-level cache
    wr = w.reshape(1, -1).repeat(copies, 1)
    wt = torch.stack([qwg.pack_q4k_tiles(w, p.n_in)] * copies)
    xs = torch.from_numpy(synth.activations(p.n_in, 3, 1, batch=8)).to(dev)
    stream = torch.cuda.current_stream(dev)
    wbytes = p.weight_bytes
    out = {}
    i = [0]

    def cycle(fn):
        def run():
            fn(i[0] % copies)
            i[0] += 1
        return run

    for batch in range(1, 9):
        x = xs[:batch].contiguous()
        y = torch.empty(batch, p.n_out, device=dev)
        if batch == 1:
            us = _event_us(cycle(lambda k: qwg.gemv_q4k(wr[k].view(p.n_out, -1), x[0], out=y[0])),
                           stream, args.steps, args.warmup)
            ust = _event_us(cycle(lambda k: qwg.gemv_q4k_tiled(wt[k], x[0], p.n_out, out=y[0])),
                            stream, args.steps, args.warmup)
            out["b1_tiled_us"] = round(ust, 2)
        else:
            us = _event_us(cycle(lambda k: qwg.gemm_q4k(wr[k].view(p.n_out, -1), x, out=y)),
                           stream, args.steps, args.warmup)
            ust = _event_us(cycle(lambda k: qwg.gemm_q4k_tiled(wt[k], x, p.n_out, out=y)),
                            stream, args.steps, args.warmup)
            out[f"b{batch}_tiled_us"] = round(ust, 2)
        nbytes = wbytes + 4 * batch * (p.n_in + p.n_out)
        out[f"b{batch}_us"] = round(us, 2)
        out[f"b{batch}_GBs"] = round(nbytes / us / 1e3, 1)
    b8 = out["b8_us"]
    flops8 = 2.0 * 8 * p.n_in * p.n_out
    print(json.dumps({
        "metric": "LM head 32000x2048 Q4_K time per call, batch 1..8", "value": b8, "unit": "us (batch 8)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Q4_K LM head 2048->32000, cold weights (16 copies cycled)", **out,
                   "b8_TFLOPs": round(flops8 / b8 / 1e6, 2)},
    }), flush=True)


def bench_batched(args):
    """The per-token stream's 155 products for a batch of 2, 4 or 8 sequences at
    once: one batched group launch (qwg_group_create_q4k_batched[_tiled]) on the
    matrix cores, tile-layout and row-major weights. A step reads every weight once and the batch's
    activations and outputs: its algorithmic bytes are the weights plus
    4 * batch * (n_in + n_out) per GEMV."""
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probs = synth.config(5)
    W = [torch.from_numpy(synth.weights(p)).to(dev) for p in probs]
    WT = [qwg.pack_q4k_tiles(w, p.n_in) for p, w in zip(probs, W)]
    stream = torch.cuda.current_stream(dev)
    out = {}
    for batch in (2, 4, 8):
        X = [torch.from_numpy(synth.activations(p.n_in, 5, k, batch=batch)).to(dev)
             for k, p in enumerate(probs)]
        Y = [torch.empty(batch, p.n_out, device=dev) for p in probs]
        nbytes = sum(p.weight_bytes + 4 * batch * (p.n_in + p.n_out) for p in probs)
        for tiled, key in ((True, f"b{batch}"), (False, f"b{batch}_row_major")):
            group = qwg.Q4kBatchedGroup(zip(WT if tiled else W, X, Y), tiled=tiled)
            us = _event_us(lambda: group.run(stream), stream, args.steps, args.warmup)
            out[key] = {"us_per_step": round(us, 2), "tokens_per_s": round(batch / us * 1e6, 1),
                        "GBs": round(nbytes / us / 1e3, 1),
                        "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                        "algorithmic_bytes_per_step": nbytes, "workgroups": group.workgroups}
            group.close()
    b8 = out["b8"]
    print(json.dumps({
        "metric": "tokens/s, Q4_K per-token stream for a batch of sequences (matrix cores)",
        "value": b8["tokens_per_s"], "unit": "tokens/s (batch 8)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "TinyLlama-1.1B Q4_K per-token stream (155 products) for 2, 4 or 8 "
                               "sequences, one batched group launch, tile-layout weights (row-major "
                               "beside it)", **out},
        "roofline": {"bound": "hbm", "achieved": b8["GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": b8["frac"], "traffic": None,
                     "kernel": "q4k_mfma_group_kernel<8,1,tile layout> (batch 8, one launch)"},
    }), flush=True)


def cpu_baseline(probs, host_w, host_x, outputs, budget_s):
    """The oracle (plain C, fp64 dot, OpenMP over rows) on the host cores over the
    same per-token stream, repeated until the budget is spent; the GPU outputs of
    the last step of each layout are compared with it on the way (sampled rows)."""
    import numpy as np
    import oracle

    oracle.build(force=False)
    cores = oracle.get_threads()
    step_bytes = sum(p.algorithmic_bytes for p in probs)
    runs, t_total = 0, 0.0
    worst = 0.0
    rng = np.random.default_rng(0)
    while runs == 0 or t_total < budget_s:
        t0 = time.perf_counter()
        for j, (p, w, x) in enumerate(zip(probs, host_w, host_x)):
            y, s = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
            if runs == 0:
                rows = rng.integers(0, p.n_out, 16)
                for Y in outputs:
                    g = Y[j].cpu().numpy()[rows].astype(np.float64)
                    worst = max(worst, float(np.max(np.abs(g - y[rows]) / s[rows])))
        t_total += time.perf_counter() - t0
        runs += 1
    if worst > 2e-6:
        raise SystemExit(f"GPU output outside the 2e-6 bound vs the oracle (worst {worst:.3g})")
    return {
        "value": round(step_bytes * runs / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{runs} full per-token streams (155 GEMVs, {step_bytes / 1e6:.0f} MB each), "
                  f"{t_total:.1f} s; GPU rows checked, worst |dy|/sum|wx| = {worst:.2e}",
    }


if __name__ == "__main__":
    main()
