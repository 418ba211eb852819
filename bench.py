#!/usr/bin/env python3
"""Effective HBM bandwidth of the fused Q4_K dequantize-GEMV on one MI355X.

Workload (one "step" = one decoded token's weight stream at batch 1): the
TinyLlama-1.1B-shaped Q4_K projections of 22 layers (q, o 2048x2048; k, v
256x2048; gate, up 5632x2048; down 2048x5632) followed by the 2048->32000 LM
head: 155 GEMVs, 582 MB of distinct packed weights (more than the 256 MB
last-level cache, so every step streams them from HBM). Weights, activations
and outputs are seeded synthetic data resident in HBM before timing starts.

A decode step cannot run its products independently: per layer q|k|v read the
normalized x, o reads the attention output, gate|up the normalized residual,
down the SwiGLU activation, the next layer the updated x, and the LM head the
final norm (picoLM page, model_forward). The headline therefore runs the step
in that order, 89 dependent phases, as one layer-chain launch (qwg_chain_run:
a phase's products read their activations only after the previous phase has
stored all of its outputs); the activations themselves are the seeded inputs,
since the norms, attention and activations are not part of this library.
Weights are held in the library's tile-major order (qwg_pack_q4k_tiles repacks
the row-major tensors once, before timing; each 144-byte block is unchanged).

Reported beside the headline: the same order as 89 launches ("layered") and as
155 single calls ("per_call"), both also replayed from HIP graphs; and the 155
GEMVs as one launch with independent inputs ("grouped_independent", the stream
kernel's bandwidth ceiling, which no decode step can use). Every schedule writes
its own outputs, and every row of every output is checked against the oracle
before anything is timed (parity_max_ratio). Per-configuration records (C1-C4
single calls: median/p10/p90 per call, GB/s, parity, dequant bit mismatches)
and the CPU oracle's throughput (all cores and one pinned core) are in the
same line.

value = algorithmic bytes of the step (weights + x + y) / wall time per step of
the headline, in GB/s; roofline = the same bytes / the chain kernel's average
duration from HIP events on its stream around the timed loop.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--headline-only]
       python bench.py --workload iq3_stream|iq3_xxs|codebooks|encode|lm_head|batched|gemm_ab|dequant [--steps K] [--warmup W]
The second form measures the other hot-path rows on their own (one JSON line each, for the
record and for profiling): "iq3_stream" = the same 155 GEMV shapes in the IQ3 container as one
grouped launch (IQ3 tile layout; the row-major launch beside it); "iq3_xxs" = IQ3_XXS blocks in
llama.cpp's byte order (single GEMVs row-major and repacked, and the stream repacked); "codebooks" =
the same stream and single shapes in IQ3_S and IQ4_XS (tile layout); "encode" = the IQ3 container
encoder on the IQ3 configuration's matrices (an ALU-bound roofline); "lm_head" = the 32000x2048 Q4_K
LM head at batch 1..8 (qwg_gemv_q4k, qwg_gemv_q4k_tiled, qwg_gemm_q4k), cycling over enough weight
copies that every launch streams from HBM rather than the last-level cache; "batched" = the
per-token stream for 2, 4 and 8 sequences as one batched group launch; "gemm_ab" = an A/B of
the batched-GEMM engines (matrix-core pipeline with one or two columns per stage, the persistent
matrix-core stream, the vector-ALU engine with 4, 8 or 16 wavefronts per tile, and the automatic
choice) at batch 2..8 on the LM head and the layer shapes, cold weights; "dequant" =
dequant_q4k, _iq3, _iq3s and _iq4xs of the 32000x2048 LM-head matrix to fp32 (write-bound: 262 MB
written per call), checked bit for bit against the oracle's decode before timing.
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
KERNEL_SOURCES = ["quantized_weight_decode_gemv_amd/csrc/chain.hip",
                  "quantized_weight_decode_gemv_amd/csrc/q4k_dot.h",
                  "quantized_weight_decode_gemv_amd/csrc/qwg_device.h",
                  "quantized_weight_decode_gemv_amd/csrc/qwg_internal.h"]
# HBM bytes per layer-chain launch of the stream (tile layout), from rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE runs of this script, each scaled by the same counter on a plain device copy of known
# size (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0; see profiles/q4k_chain_c5.md). Valid only for the
# kernel sources with this hash; otherwise traffic is reported as null.
TRAFFIC = {"sources_sha256": "37d4448fcc5fa42791aced621d92b98d21b982e4f78577b6fa069164e4b8a3aa",
           "fetch_bytes": 620764864, "write_bytes": 6816768}


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
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="minimum CPU time budget for the oracle baseline")
    ap.add_argument("--print-kernel-hash", action="store_true",
                    help="print the hash of the kernel sources the traffic figure is tied to")
    ap.add_argument("--workload", default="q4k_stream",
                    choices=["q4k_stream", "configs", "iq3_stream", "iq3_xxs", "codebooks", "encode",
                             "lm_head", "batched", "gemm_ab", "dequant"],
                    help="q4k_stream: the headline (default); the others: see the module docstring")
    ap.add_argument("--headline-only", action="store_true",
                    help="run and time only the headline launch (no other schedules, no "
                         "per-configuration records), so a kernel trace holds nothing else of it")
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
    if args.workload == "configs":
        bench_configs(args)
        return
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
    if args.workload == "gemm_ab":
        bench_gemm_ab(args)
        return
    if args.workload == "dequant":
        bench_dequant(args)
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
    # Weights whose chained products keep their norms (the chain feeds each
    # product's output to the next); the other schedules use the same weights.
    host_w = [synth.q4k_chain_weights(p.n_out, p.n_in, p.cfg, p.tensor) for p in probs]
    host_x = [synth.inputs(p) for p in probs]
    W = [torch.from_numpy(w).to(dev) for w in host_w]
    X = [torch.from_numpy(x).to(dev) for x in host_x]
    WT = [qwg.pack_q4k_tiles(w, p.n_in) for p, w in zip(probs, W)]
    torch.cuda.synchronize()
    setup_s = time.time() - t0

    stream = torch.cuda.current_stream(dev)
    step_bytes = sum(p.algorithmic_bytes for p in probs)
    weight_bytes = sum(p.weight_bytes for p in probs)
    phases = layer_phases(probs)

    def outputs():
        return [torch.empty(p.n_out, dtype=torch.float32, device=dev) for p in probs]

    # Every schedule writes its own outputs, so each can be checked on its own.
    Y = {name: outputs() for name in ("chain", "layered", "per_call", "grouped_independent",
                                      "grouped_independent_row_major")}
    # The chain as a decode step: each product reads the output of the product
    # that stands in for its input (layer 0's q, k, v read the step input).
    src = synth.chain_sources(probs)
    XC = [X[0] if j < 0 else Y["chain"][j] for j in src]
    chain = qwg.Q4kChain([[(WT[i], XC[i], Y["chain"][i]) for i in ph] for ph in phases])
    layered = [qwg.Q4kGroup([(WT[i], X[i], Y["layered"][i]) for i in ph], tiled=True)
               for ph in phases]
    calls = [(y.data_ptr(), x.data_ptr(), w.data_ptr(), p.n_in, p.n_out)
             for p, w, x, y in zip(probs, WT, X, Y["per_call"])]
    grouped = qwg.Q4kGroup(zip(WT, X, Y["grouped_independent"]), tiled=True)
    grouped_rows = qwg.Q4kGroup(zip(W, X, Y["grouped_independent_row_major"]))
    gemv = L.qwg_gemv_q4k_tiled

    def step_chain(s=stream):
        chain.run(s)

    def step_layered(s=stream):
        for g in layered:
            g.run(s)

    def step_per_call(s=stream):
        sp = ctypes.c_void_p(s.cuda_stream)
        for yp, xp, wp, n_in, n_out in calls:
            rc = gemv(yp, xp, wp, n_in, n_out, sp)
            if rc:
                raise RuntimeError(f"qwg_gemv_q4k_tiled failed: {rc}")

    runners = {"chain": step_chain, "layered": step_layered, "per_call": step_per_call,
               "grouped_independent": lambda s=stream: grouped.run(s),
               "grouped_independent_row_major": lambda s=stream: grouped_rows.run(s)}
    if args.headline_only:
        runners = {"chain": step_chain}

    # One run of each schedule into NaN-filled outputs, checked on every row by
    # the oracle leg before anything is timed.
    for name, fn in runners.items():
        for y in Y[name]:
            y.fill_(float("nan"))
        fn()
    torch.cuda.synchronize()
    chain.status()
    gpu_out = {name: [y.cpu().numpy() for y in Y[name]] for name in runners}
    # the chain's actual inputs: the step input, or the producer's output
    chain_in = [host_x[0] if j < 0 else gpu_out["chain"][j] for j in src]
    per_config_gpu = None if args.headline_only else run_configs(dev, stream, args)

    parity, cpu, per_config = None, None, None
    if not args.no_cpu:
        cpu, parity, per_config = cpu_baseline_leg(probs, host_w, host_x, gpu_out, per_config_gpu,
                                                   args.cpu_seconds, inputs={"chain": chain_in})

    def graph_of(fn, outs):
        """fn(stream) captured once in a HIP graph on a side stream (after one
        eager call there, so that nothing is allocated during capture); returns
        the graph and whether three replays, with eager runs in between, each
        reproduced the eager outputs bit for bit."""
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
            ref = [y.clone() for y in outs]
            for y in outs:
                y.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            ok = ok and all(torch.equal(a, b) for a, b in zip(ref, outs))
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

    def sched(sec_, launches, chain_respecting, **extra):
        return {"us_per_step": round(1e6 * sec_, 1), "GBps": round(step_bytes / sec_ / 1e9, 1),
                "pct_of_hbm_peak": round(100 * step_bytes / sec_ / 1e9 / HBM_PEAK_GBS, 1),
                "tokens_per_s": round(1.0 / sec_, 1), "launches": launches,
                "respects_layer_chain": chain_respecting, **extra}

    # The other schedules first (this also brings the clocks up), the headline last.
    schedules = {}
    grouped_kernel_us = None
    if not args.headline_only:
        n = max(5, args.steps // 5)
        schedules["layered"] = sched(timed(step_layered, n, 2), len(layered), True)
        schedules["per_call"] = sched(timed(step_per_call, n, 2), len(calls), True)
        g_l, ok_l = graph_of(step_layered, Y["layered"])
        g_p, ok_p = graph_of(step_per_call, Y["per_call"])
        schedules["layered_graph"] = sched(timed(g_l.replay, n, 2), len(layered), True,
                                           replays_match_eager=ok_l)
        schedules["per_call_graph"] = sched(timed(g_p.replay, n, 2), len(calls), True,
                                            replays_match_eager=ok_p)
        # 155 GEMVs with independent inputs in one launch: the stream kernel's
        # bandwidth ceiling, not a decode step (a decoder's layers depend on
        # one another).
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(max(args.warmup, 200)):
            grouped.run(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for _ in range(args.steps):
            grouped.run(stream)
        ev1.record(stream)
        torch.cuda.synchronize()
        sec_g = (time.perf_counter() - t0) / args.steps
        grouped_kernel_us = 1e3 * ev0.elapsed_time(ev1) / args.steps
        schedules["grouped_independent"] = sched(sec_g, 1, False, kernel_us=round(grouped_kernel_us, 2))
        schedules["grouped_independent_row_major"] = sched(
            timed(lambda: grouped_rows.run(stream), args.steps, args.warmup), 1, False)
        for _ in range(200):   # keep the clocks up right before the headline
            chain.run(stream)

    # Headline: the layer-chain launch (the fastest schedule that respects the
    # dependency of each layer's products on the previous ones). Wall clock
    # over the timed loop; HIP events on the launch stream around the same
    # loop of back-to-back launches give the kernel's average duration.
    for _ in range(args.warmup):
        step_chain()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step_chain()
    ev1.record(stream)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / args.steps
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    chain.status()
    ms_per_step = 1e3 * sec
    value = step_bytes / sec / 1e9
    achieved = step_bytes / (kernel_ms * 1e-3) / 1e9
    schedules["chain"] = sched(sec, 1, True, kernel_us=round(1e3 * kernel_ms, 2),
                               phases=chain.launch_phases,
                               waits="tagged done words" if chain.tagged else "flag barriers",
                               inputs="each product reads its producer's output")

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
                        "LM head 32000x2048 = 155 GEMVs in the dependency order of a decode step "
                        "(per layer q|k|v, o, gate|up, down; then the LM head: 89 phases, each "
                        "starting when every tile of the phase before it is finished), each "
                        "product reading the output of the product standing in for its input "
                        "(q|k|v the previous layer's down, o q, gate|up o, down gate, the LM head "
                        "the last down), one layer-chain launch (qwg_chain_run), weights in "
                        "tile-major order",
            "layout": "tile-major Q4_K (qwg_pack_q4k_tiles, repacked once before timing)",
            "weight_bytes": weight_bytes,
            "algorithmic_bytes_per_step": step_bytes,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "tokens_per_s": round(1e3 / ms_per_step, 1),
            "setup_s": round(setup_s, 1),
            "schedules": schedules,
            "parity_max_ratio": parity,
            "per_config": per_config,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_bytes(),
            "kernel": "q4k_chain_kernel (layer chain, 155 GEMVs in 89 dependent phases, tile layout)",
            "bytes_per_launch": step_bytes,
            "kernel_us": round(1e3 * kernel_ms, 2),
        },
    }
    if grouped_kernel_us is not None:
        ga = step_bytes / (grouped_kernel_us * 1e-6) / 1e9
        result["roofline_stream_kernel"] = {
            "bound": "hbm", "achieved": round(ga, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ga / HBM_PEAK_GBS, 4),
            "kernel": "q4k_stream_kernel<4,2> (155 independent GEMVs per launch, tile layout: "
                      "the stream's bandwidth ceiling, not a decode step)",
            "kernel_us": round(grouped_kernel_us, 2)}
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def bench_configs(args):
    """One JSON line per configuration C1-C4 (single calls through the C ABI,
    cold weights): per call median / p10 / p90, GB/s, % of peak, the parity max
    ratio over all rows and the dequant bit-mismatch count (the per-config
    records of the default run, printed on their own)."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    gpu = run_configs(dev, stream, args)
    if args.no_cpu:
        recs = {k: v["rec"] for k, v in gpu.items()}
    else:
        recs = cpu_baseline_leg(None, None, None, {}, gpu, 0.0, configs_only=True)
    for cfg in ("C1", "C2", "C3", "C4"):
        members = {k: v for k, v in recs.items() if v["config"] == cfg}
        total_bytes = sum(v["algorithmic_bytes"] for v in members.values())
        total_us = sum(v["median_us"] for v in members.values())
        print(json.dumps({
            "metric": "effective HBM GB/s (% of MI355X peak) for Q4_K/IQ3 GEMV, batch 1",
            "config": cfg, "value": round(total_bytes / total_us / 1e3, 2), "unit": "GB/s",
            "n_gpus": 1, "dtype": "f32", "data": "synthetic", "higher_is_better": True,
            "pct_of_hbm_peak": round(100 * total_bytes / total_us / 1e3 / HBM_PEAK_GBS, 2),
            "calls": members}), flush=True)


def layer_phases(probs):
    """The per-token stream's GEMVs grouped into the phases of a decode step
    (picoLM model_forward: per layer q|k|v read the normalized x, o the attention
    output, gate|up the normalized residual, down the SwiGLU activation; then the
    LM head), as lists of indices."""
    phases, i = [], 0
    while i < len(probs):
        name = probs[i].name.split(".")[-1]
        n = 3 if name == "q" else 2 if name == "gate" else 1
        phases.append(list(range(i, i + n)))
        i += n
    return phases


def _percentiles(us):
    import numpy as np
    a = np.asarray(us)
    return {"median_us": round(float(np.median(a)), 2), "p10_us": round(float(np.percentile(a, 10)), 2),
            "p90_us": round(float(np.percentile(a, 90)), 2)}


def run_configs(dev, stream, args):
    """GPU side of the per-configuration records (C1-C4 as single calls through
    the C ABI): each call's duration from a HIP event pair around it, on
    weights cycled over enough copies (>= 1 GiB) that every call reads HBM;
    200 timed calls after 200 warm-up calls. Also one call into NaN-filled
    outputs, and the bit patterns of the dequantized matrix, for the oracle
    leg. Returns {name: {...}}."""
    import numpy as np
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    out = {}
    # (200 warm-up calls per case: these records are taken right after setup,
    # before the clocks have come up; with 20 the first case read 9.0 against 6.2 us)
    timed_calls, warm = 200, 200

    def cycle_time(call, copies):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(timed_calls)]
        for k in range(warm):
            call(k % copies)
        for k, (a, b) in enumerate(evs):
            a.record(stream)
            call((warm + k) % copies)
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    cases = []
    for p in synth.config(1) + synth.config(2) + synth.config(3) + synth.config(4):
        cases.append(p)
    for p in cases:
        w = synth.weights(p)
        x = synth.inputs(p)
        wd = torch.from_numpy(w).to(dev)
        xd = torch.from_numpy(np.ascontiguousarray(x)).to(dev)
        copies = max(1, -(-(1 << 30) // w.nbytes))
        wc = wd.reshape(1, -1).repeat(copies, 1).view(copies, *w.shape)
        if p.fmt == "iq3":
            grid = torch.from_numpy(synth.iq3_grid()).to(dev)
            y = torch.full((p.n_out,), float("nan"), device=dev)
            qwg.gemv_iq3(wd, xd, grid, out=y)
            deq = qwg.dequant_iq3(wd, grid)
            call = lambda k: qwg.gemv_iq3(wc[k], xd, grid, out=y)   # noqa: E731
            kernel = "qwg_gemv_iq3"
        elif p.batch > 1:
            y = torch.full((p.batch, p.n_out), float("nan"), device=dev)
            qwg.gemm_q4k(wd, xd, out=y)
            deq = None
            call = lambda k: qwg.gemm_q4k(wc[k], xd, out=y)   # noqa: E731
            kernel = f"qwg_gemm_q4k (batch {p.batch})"
        else:
            y = torch.full((p.n_out,), float("nan"), device=dev)
            qwg.gemv_q4k(wd, xd, out=y)
            deq = qwg.dequant_q4k(wd)
            call = lambda k: qwg.gemv_q4k(wc[k], xd, out=y)   # noqa: E731
            kernel = "qwg_gemv_q4k"
        torch.cuda.synchronize()
        y0 = y.cpu().numpy().copy()
        d0 = None if deq is None else deq.cpu().numpy().reshape(-1).view(np.uint32).copy()
        us = cycle_time(call, copies)
        cfg = {1: "C1", 2: "C2", 3: "C3", 4: "C4"}[p.cfg]
        rec = {"config": cfg, "kernel": kernel, "shape": [p.n_out, p.n_in], "batch": p.batch,
               "algorithmic_bytes": p.algorithmic_bytes, **_percentiles(us),
               "cold_copies": copies}
        rec["GBps_median"] = round(p.algorithmic_bytes / rec["median_us"] / 1e3, 1)
        rec["pct_of_hbm_peak"] = round(100 * rec["GBps_median"] / HBM_PEAK_GBS, 2)
        out[f"{cfg}.{p.name}"] = {"rec": rec, "y": y0, "deq_bits": d0, "problem": p}
        del wc
        torch.cuda.empty_cache()
    return out


def cpu_info():
    """CPU model, logical CPUs this process may use, and last-level cache size."""
    model, llc = None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        base = "/sys/devices/system/cpu/cpu0/cache"
        best = -1
        for idx in os.listdir(base):
            lvl_path = os.path.join(base, idx, "level")
            if os.path.exists(lvl_path):
                lvl = int(open(lvl_path).read())
                if lvl > best:
                    best = lvl
                    llc = f"L{lvl} " + open(os.path.join(base, idx, "size")).read().strip()
    except OSError:
        pass
    return {"cpu_model": model, "llc": llc, "cpus_usable": len(os.sched_getaffinity(0)),
            "cpus_online": os.cpu_count()}


def cpu_baseline_leg(probs, host_w, host_x, gpu_out, per_config_gpu, budget_s, configs_only=False,
                     inputs=None):
    """Everything that runs the oracle (plain C, fp64 dot, OpenMP over rows):
    (1) the full oracle result of the per-token stream, against which every row
    of every schedule's GPU output is checked (the bench stops if any row is
    outside |dy| <= 2e-6 * sum|w*x|); (2) the per-configuration parity (max
    ratio |dy| / sum|w*x|, dequant bit mismatches); (3) the CPU baseline: the
    oracle timed over the same stream on all usable host cores and on one
    pinned core (no GPU data is copied inside the timed loops)."""
    import numpy as np
    import oracle
    from quantized_weight_decode_gemv_amd import synth

    oracle.build(force=False)
    threads0 = oracle.get_threads()
    parity = {}
    ref = [] if configs_only else [oracle.gemv_q4k(w, x, p.n_in, p.n_out)
                                   for p, w, x in zip(probs, host_w, host_x)]
    for name, outs in gpu_out.items():
        worst = 0.0
        mine = ref
        if inputs and name in inputs:   # a schedule with its own inputs (the chained stream)
            mine = [oracle.gemv_q4k(w, np.ascontiguousarray(x), p.n_in, p.n_out)
                    for p, w, x in zip(probs, host_w, inputs[name])]
        for (yr, sr), yg in zip(mine, outs):
            d = np.abs(yg.astype(np.float64) - yr)
            worst = max(worst, float(np.max(np.where(np.isnan(d), np.inf, d) / np.maximum(sr, 1e-300))))
        parity[name] = worst
        if not worst <= 2e-6:
            raise SystemExit(f"schedule {name}: a GPU output row is outside the 2e-6 bound "
                             f"(worst {worst:.3g})")
    per_config = None
    if per_config_gpu:
        per_config = {}
        for key, item in per_config_gpu.items():
            p, rec = item["problem"], item["rec"]
            w = synth.weights(p)
            x = np.ascontiguousarray(synth.inputs(p))
            if p.fmt == "iq3":
                grid = synth.iq3_grid()
                yr, sr = oracle.gemv_iq3(w, grid, x, p.n_in, p.n_out)
                dq = oracle.dequant_iq3(w, grid, p.n_out * p.n_in)
            elif p.batch > 1:
                yr, sr = oracle.gemm_q4k(w, x, p.n_in, p.n_out)
                dq = None
            else:
                yr, sr = oracle.gemv_q4k(w, x, p.n_in, p.n_out)
                dq = oracle.dequant_q4k(w, p.n_out * p.n_in)
            d = np.abs(item["y"].astype(np.float64).reshape(yr.shape) - yr)
            ratio = float(np.max(np.where(np.isnan(d), np.inf, d) / np.maximum(sr, 1e-300)))
            if not ratio <= 2e-6:
                raise SystemExit(f"{key}: a GPU output row is outside the 2e-6 bound ({ratio:.3g})")
            rec = dict(rec, parity_max_ratio=ratio)
            if dq is not None:
                rec["dequant_bit_mismatches"] = int(np.count_nonzero(
                    dq.reshape(-1).view(np.uint32) != item["deq_bits"]))
            per_config[key] = rec
    if configs_only:
        return per_config
    step_bytes = sum(p.algorithmic_bytes for p in probs)

    def run_for(seconds):
        runs, t = 0, 0.0
        while runs == 0 or t < seconds:
            t0 = time.perf_counter()
            for p, w, x in zip(probs, host_w, host_x):
                oracle.gemv_q4k(w, x, p.n_in, p.n_out)
            t += time.perf_counter() - t0
            runs += 1
        return runs, t

    info = cpu_info()
    cores = len(os.sched_getaffinity(0))
    oracle.set_threads(cores)
    runs_all, t_all = run_for(budget_s)
    # one core: this process pinned to one CPU, one OpenMP thread
    aff = os.sched_getaffinity(0)
    try:
        os.sched_setaffinity(0, {min(aff)})
        oracle.set_threads(1)
        runs_one, t_one = run_for(budget_s)
    finally:
        os.sched_setaffinity(0, aff)
        oracle.set_threads(threads0)
    cpu = {
        "value": round(step_bytes * runs_all / t_all / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{runs_all} full per-token streams (155 GEMVs, {step_bytes / 1e6:.0f} MB of "
                  f"algorithmic bytes each) in {t_all:.1f} s on {cores} threads",
        "one_core": {"value": round(step_bytes * runs_one / t_one / 1e9, 4), "unit": "GB/s",
                     "cores": 1, "sample": f"{runs_one} full streams in {t_one:.1f} s, pinned to one "
                                          "CPU with one thread"},
        "tokens_per_s_all_cores": round(runs_all / t_all, 2),
        **info,
    }
    return cpu, parity, per_config


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


def bench_dequant(args):
    """dequant_q4k, dequant_iq3, dequant_iq3s and dequant_iq4xs (whole blocks to
    fp32, row-major) over the 32000 x 2048 LM-head matrix: write-bound (1,024
    bytes written per 144-, 98-, 110- or 136-byte block). The outputs of one call into NaN-filled buffers are checked
    bit for bit against the oracle's decode before anything is timed."""
    import numpy as np
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth
    import oracle

    oracle.build(force=False)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    p = synth.config(3)[0]
    n = p.n_out * p.n_in
    grid_np = synth.iq3_grid()
    grid = torch.from_numpy(grid_np).to(dev)
    grid_s_np, table_np = synth.iq3s_grid(), synth.iq4nl_table()
    grid_s, table = torch.from_numpy(grid_s_np).to(dev), torch.from_numpy(table_np).to(dev)
    cases = {"q4k": (synth.weights(p), 144, lambda w, o: qwg.dequant_q4k(w, out=o),
                     lambda w: oracle.dequant_q4k(w, n)),
             "iq3": (synth.iq3_weights(p.n_out, p.n_in, p.cfg, p.tensor), 98,
                     lambda w, o: qwg.dequant_iq3(w, grid, out=o),
                     lambda w: oracle.dequant_iq3(w, grid_np, n)),
             "iq3s": (synth.iq3s_weights(p.n_out, p.n_in, p.cfg, p.tensor), 110,
                      lambda w, o: qwg.dequant_iq3s(w, grid_s, out=o),
                      lambda w: oracle.dequant_iq3s(w, grid_s_np, n)),
             "iq4xs": (synth.iq4xs_weights(p.n_out, p.n_in, p.cfg, p.tensor), 136,
                       lambda w, o: qwg.dequant_iq4xs(w, table, out=o),
                       lambda w: oracle.dequant_iq4xs(w, table_np, n))}
    res = {}
    for name, (w, block, call, ref) in cases.items():
        wd = torch.from_numpy(w).to(dev)
        out = torch.full((n,), float("nan"), device=dev)
        call(wd, out)
        torch.cuda.synchronize()
        bad = int(np.count_nonzero(host_bits(out) != ref(w).reshape(-1).view(np.uint32)))
        if bad:
            raise SystemExit(f"dequant_{name}: {bad} values differ from the oracle's decode")
        us = _event_us(lambda: call(wd, out), stream, args.steps, args.warmup)
        nbytes = (n // 256) * (block + 1024)
        res[name] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                     "frac_of_hbm_peak": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                     "bytes_per_call": nbytes, "bit_mismatches": bad}
        del wd, out
    print(json.dumps({
        "metric": "dequant to fp32, effective HBM GB/s (bytes read + written)",
        "value": res["q4k"]["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "qwg_dequant_q4k / _iq3 / _iq3s / _iq4xs of the 32000 x 2048 LM-head "
                               "matrix (256,000 blocks -> 65,536,000 fp32 weights)", **res},
        "roofline": {"bound": "hbm", "achieved": res["q4k"]["GBps"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": res["q4k"]["frac_of_hbm_peak"],
                     "kernel": "q4k_dequant_kernel", "kernel_us": res["q4k"]["us"]}}), flush=True)


def host_bits(t):
    """fp32 device tensor -> its bit patterns (uint32 numpy array)."""
    return t.detach().cpu().numpy().reshape(-1).view("<u4")


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
                     qwg.gemv_iq3s_tiled, qwg.gemv_iq3s, qwg.Iq3sGroup),
            "iq4xs": (synth.iq4xs_weights, synth.iq4nl_table, 136, qwg.pack_iq4xs_tiles,
                      qwg.gemv_iq4xs_tiled, qwg.gemv_iq4xs, qwg.Iq4xsGroup)}
    out = {}
    for name, (weights, table, nbytes, pack, gemv, gemv_rows, Group) in fmts.items():
        tab = torch.from_numpy(table()).to(dev)
        probs = synth.config(6)
        X = [torch.from_numpy(synth.inputs(p)).to(dev) for p in probs]
        Y = [torch.empty(p.n_out, device=dev) for p in probs]
        step = sum(p.n_out * (p.n_in // 256) * nbytes + 4 * (p.n_in + p.n_out) for p in probs)
        res = {}
        for layout in ("tiled", "rows"):
            W = [torch.from_numpy(weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev) for p in probs]
            if layout == "tiled":
                W = [pack(w, p.n_in) for w, p in zip(W, probs)]
            group = Group(zip(W, X, Y), tab, tiled=layout == "tiled")
            us = _event_us(lambda: group.run(stream), stream, args.steps, args.warmup)
            group.close()
            del W
            res[layout] = us
        singles = {}
        copies = 64
        for p in synth.config(4):
            w = torch.from_numpy(weights(p.n_out, p.n_in, p.cfg, p.tensor)).to(dev)
            x = torch.from_numpy(synth.inputs(p)).to(dev)
            y = torch.empty(p.n_out, device=dev)
            b = p.n_out * (p.n_in // 256) * nbytes + 4 * (p.n_in + p.n_out)
            for layout in ("tiled", "rows"):
                WT = torch.stack([pack(w, p.n_in) if layout == "tiled" else w] * copies)
                i = [0]

                def run():
                    if layout == "tiled":
                        gemv(WT[i[0] % copies], x, tab, p.n_out, out=y)
                    else:
                        gemv_rows(WT[i[0] % copies], x, tab, out=y)
                    i[0] += 1
                u = _event_us(run, stream, args.steps, args.warmup)
                singles[f"{p.name} {layout}"] = {"us": round(u, 2), "GBs": round(b / u / 1e3, 1)}
                del WT
        us = res["tiled"]
        out[name] = {"stream_us": round(us, 2), "stream_GBs": round(step / us / 1e3, 1),
                     "frac": round(step / us / 1e3 / HBM_PEAK_GBS, 4),
                     "stream_rows_us": round(res["rows"], 2),
                     "stream_rows_GBs": round(step / res["rows"] / 1e3, 1),
                     "algorithmic_bytes_per_step": step, "singles": singles}
    best = max(out.values(), key=lambda v: v["stream_GBs"])
    print(json.dumps({
        "metric": "effective HBM GB/s, IQ3_S / IQ4_XS GEMV stream, batch 1",
        "value": best["stream_GBs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "TinyLlama-1.1B-shaped per-token stream (155 GEMVs) in the IQ3_S and "
                               "IQ4_XS formats, one grouped launch each on the tile layout (value) "
                               "and on row-major blocks (stream_rows_*); single GEMVs of the IQ3 "
                               "configuration's shapes on both layouts, cold weights", **out},
    }), flush=True)


# Vector-ALU operations per weight of the IQ3 encoder's search (the rest is
# negligible): 16 codes x 256 grid rows per group of four weights, each row
# 4 multiplies + 3 adds (q.g), a doubling and a subtract (g2 - 2 q.g), a
# compare and two selects (the running minimum) = 12 operations.
ENCODE_OPS_PER_WEIGHT = 16 * 256 * 12 / 4
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz: a two-operand wave64 fp32 instruction
# issues in two cycles on MI355X (the vendor's 157.3 TFLOP/s fp32 vector figure
# is this rate counting an FMA as two; the encoder, whose search is multiplies,
# adds, compares and selects with no packed or fused forms, sustains 0.45
# wave64 instructions per SIMD-cycle). Three-operand forms (FMA, v_perm) take
# about four cycles, so this peak is the encoder's, not the GEMV dots'.
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


# Engines of qwg_gemm_q4k_ex by its `waves` argument (0: the automatic choice).
GEMM_ENGINES = {"auto": 0, "mfma_1col": 1, "mfma_2col": 2, "mfma_stream": 3, "valu_4w": 4,
                "valu_8w": 8, "valu_16w": 16}


def bench_gemm_ab(args):
    """Every batched-GEMM engine at batch 2..8 on the LM head and the layer
    shapes (qwg_gemm_q4k_ex with the engine forced and its own automatic
    splits), weights cycled over enough copies to stream from HBM."""
    import torch
    import quantized_weight_decode_gemv_amd as qwg
    from quantized_weight_decode_gemv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for n_out, n_in in ((32000, 2048), (2048, 2048), (5632, 2048), (2048, 5632)):
        w = torch.from_numpy(synth.q4k_weights(n_out, n_in, 1, 0)).to(dev)
        copies = max(2, (1 << 30) // w.numel())
        W = w.reshape(1, -1).repeat(copies, 1)
        nbytes = w.numel()
        for batch in range(2, 9):
            x = torch.from_numpy(synth.activations(n_in, 1, batch, batch=batch)).to(dev)
            y = torch.empty(batch, n_out, device=dev)
            row = {}
            # three rounds over the engines, the least time of each (clock and
            # ordering effects of one pass reach 1-2 us)
            for _ in range(3):
                for name, waves in GEMM_ENGINES.items():
                    i = [0]

                    def run():
                        qwg.gemm_q4k(W[i[0] % copies].view(n_out, -1), x, out=y, waves=waves)
                        i[0] += 1
                    t = round(_event_us(run, stream, args.steps, args.warmup), 2)
                    row[name] = min(row.get(name, t), t)
            best = min((k for k in row if k != "auto"), key=row.get)
            row["best"] = best
            row["best_GBs"] = round((nbytes + 4 * batch * (n_in + n_out)) / row[best] / 1e3, 1)
            out[f"{n_out}x{n_in}_b{batch}"] = row
            print(f"# {n_out}x{n_in} b{batch} {row}", file=sys.stderr, flush=True)
    lm8 = out["32000x2048_b8"]
    print(json.dumps({
        "metric": "batched Q4_K GEMM time per call by engine (us), batch 2..8", "value": lm8["auto"],
        "unit": "us (LM head, batch 8, automatic engine)", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "Q4_K GEMM (row-major weights, cold), LM head 32000x2048 and layer "
                               "shapes 2048x2048, 5632x2048, 2048x5632, batch 2..8, every engine",
                   **out},
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


if __name__ == "__main__":
    main()
