#!/usr/bin/env python3
"""Benchmark of the LiLiCorr reranking path on one MI355X.

One step = one lilicorr_rerank call over a batch of synthetic draft blocks:
fused log-partition + top-K, node build, two encoder layers, in/out heads,
pair scores and the greedy walk (every row of the hot path). The default
workload is the largest batch of the lattice head that the pages' shapes give:
256 independent blocks, B = 16, V = 151,936 bf16 logits with three spikes per
slot, K = 16, encoder width 1024, 8 heads, FFN 4096, d_e 128 (1.245 GB of
logits per step, the top-K stage's bandwidth case). --workload picks another
(c1_qwen3_8b is the concurrency-1 block).

Logits are resident in HBM before timing; consecutive steps rotate over
enough logits buffers (>= 768 MiB in total) that each step reads its logits
cold, not from the 256 MiB Infinity Cache. Prints one JSON line.

Per-stage times come from the library's stage-timing events (two events
recorded on the library's stream around one stage of a lilicorr_rerank
call). The dominant stage is found in untimed steps; in the timed steps it is
bracketed by its own event pair every step, and `roofline` divides that
stage's algorithmic bytes or flops by the mean bracketed duration. `traffic`
is the HBM bytes per launch from a committed rocprofv3 counter summary
(profiles/traffic_<workload>_<stage>.md), reported only while the kernel
sources still hash to the value recorded there.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "draft blocks/sec reranked at 1 MI355X; % peak HBM GB/s (top-K); MFMA util"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c256_k16")
    ap.add_argument("--tier", type=int, default=0)
    ap.add_argument("--rotate-mib", type=float, default=768.0)
    ap.add_argument("--stage-reps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU-baseline budget: half for the one-core figure, half for the all-core pool")
    ap.add_argument("--cpu-workers", type=int, default=16,
                    help="most worker processes of the all-core oracle pool (the host's CPU share)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step from a captured HIP graph")
    ap.add_argument("--rule", default="greedy", choices=["greedy", "exact", "sample"],
                    help="commit rule: greedy walk (default), exact best path, or sampled commit "
                         "(seeded per-block temperatures and per-slot uniforms)")
    ap.add_argument("--topk-shards", type=int, default=0,
                    help="also time the vocabulary-sharded top-K at G shards: one shard's kernel on its "
                         "[rows, V/G] slice (cold, rotating copies) and the merge of G shard outputs")
    ap.add_argument("--copy-probe-mib", type=float, default=0.0,
                    help="after the run, stream this many MiB through a plain copy kernel three "
                         "times (the known-size reference for HBM byte counters)")
    ap.add_argument("--no-clock-probe", dest="clock_probe", action="store_false",
                    help="skip the shader-clock readings taken after the run (untimed): the "
                         "library's diagnostic probe on a second stream, with the GPU idle, beside "
                         "full steps, and beside the dominant linear's kernel run on its own")
    ap.add_argument("--summarize-kernels", metavar="KT_DIR",
                    help="no GPU: turn a rocprofv3 --kernel-trace --stats run of this script into a "
                         "markdown table of kernel durations")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR",
                    help="no GPU: turn a rocprofv3 --kernel-trace --pmc MfmaUtil MfmaFlopsBF16 run of this "
                         "script into MFMA utilisation and counted bf16 MFMA flops per stage launch")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="PMC_DIR",
                    help="no GPU: turn rocprofv3 --pmc runs of this script (any counters, one or "
                         "more runs) into per-stage means of every counter, summed over a stage's "
                         "kernels, with the wave-time fractions of the SQ wait/active counters")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then "
                         "WRITE_SIZE, both with --copy-probe-mib) into HBM bytes per stage launch")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_kernels:
        summarize_kernels(args.summarize_kernels)
        summarize_stage_kernels(args.summarize_kernels)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path here "
              "(draft blocks are independent; the path would shard by blocks)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import synth

    w = synth.WORKLOADS[args.workload]
    host = synth.make_logits(w, args.tier)
    # The CPU baseline runs first, before this process touches the GPU: its
    # all-core figure forks worker processes, and a fork of a process holding
    # GPU state is best avoided.
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, host, args.cpu_seconds, args.rule,
                                                         args.cpu_workers)

    import torch

    import draft_block_candidate_amd as L

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    esize = 2 if w.dtype == "bf16" else 4
    logit_bytes = host.nbytes
    nbuf = max(1, math.ceil(args.rotate_mib * 2 ** 20 / logit_bytes))
    first = torch.from_numpy(host.view(np.int16) if w.dtype == "bf16" else host).to(dev)
    if w.dtype == "bf16":
        first = first.view(torch.bfloat16)
    bufs = [first] + [first.clone() for _ in range(nbuf - 1)]
    dims = L.EncoderDims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden,
                         drafter_hidden=w.drafter_hidden)
    weights = L.Weights(dims, w.vocab, synth.WEIGHTS_SEED, device=dev)
    head_kw = {}
    if w.target_hidden > 0:     # the paper's head: drafter hidden states and target states
        hid_bits, tgt_bits = synth.make_head_inputs(w)
        head_kw = {"hidden": torch.from_numpy(hid_bits.view(np.int16)).to(dev),
                   "target": torch.from_numpy(tgt_bits.view(np.int16)).to(dev)}
    ws = L.Workspace(w.num_blocks, w.slots, w.vocab, w.topk, dims, device=dev)
    out = torch.empty((w.num_blocks, w.slots), dtype=torch.int32, device=dev)
    N, B, V, K = w.num_blocks, w.slots, w.vocab, w.topk
    H, F, de = w.hidden, w.ffn, w.d_e
    ldt = L.BF16 if w.dtype == "bf16" else L.F32
    rule_kw = {}
    if args.rule == "sample":
        rule_kw = {"temperature": torch.from_numpy(synth.make_temperatures(N, seed=1)).to(dev),
                   "uniforms": torch.from_numpy(synth.make_uniforms(N, B, seed=2)).to(dev),
                   "proposal": torch.empty((N, B, K), dtype=torch.float32, device=dev)}
    params = [L.make_params(N, ldt, weights, ws, w.alpha, w.use_logp, rule=args.rule, **rule_kw, **head_kw)
              for _ in range(1)]
    lib = L.lib()
    state = {"i": 0}

    def step():
        b = bufs[state["i"] % nbuf]
        state["i"] += 1
        rc = lib.lilicorr_rerank(ctypes.c_void_p(b.data_ptr()), B, V, K, ctypes.byref(params[0]),
                                 ctypes.c_void_p(out.data_ptr()))
        if rc != 0:
            raise L.LilicorrError(rc, "rerank")

    run = step
    if args.graph:
        # one graph per logits buffer would be needed for rotation; replay a
        # graph over the rotating set instead
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for _ in range(3):
                step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        params[0].stream = ctypes.c_void_p(0)
        for k in range(nbuf):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                params[0].stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                state["i"] = k
                step()
            graphs.append(g)
        params[0].stream = ctypes.c_void_p(stream.cuda_stream)
        gstate = {"i": 0}

        def run():
            graphs[gstate["i"] % nbuf].replay()
            gstate["i"] += 1

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # ---- per-stage durations, measured in the pipeline with the library's
    # stage events (a few untimed steps per stage)
    stage_names = stage_table(w)
    stage_ms = {}

    def new_event():
        # torch creates the HIP event on its first record; the library then
        # re-records the same handle
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    # each stage is bracketed in stage_reps consecutive steps with no host
    # synchronisation between them, as in the timed region
    cal = [(new_event(), new_event()) for _ in range(args.stage_reps)]
    for sid in stage_names:
        for i in range(args.stage_reps):
            set_timing(params[0], sid, cal[i][0], cal[i][1])
            step()
        cal[-1][1].synchronize()
        stage_ms[sid] = sum(a.elapsed_time(b) for a, b in cal) / args.stage_reps
    set_timing(params[0], None)
    dom_sid = max(stage_ms, key=lambda k: stage_ms[k])

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    # ---- timed region: K steps; the dominant stage is bracketed by its own
    # event pair in every step (not in graph mode, where the step is replayed)
    pairs = [(new_event(), new_event()) for _ in range(args.steps)] if not args.graph else []
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        if pairs:
            set_timing(params[0], dom_sid, pairs[i][0], pairs[i][1])
        run()
    stop.record(stream)
    stop.synchronize()
    wall = time.perf_counter() - t_wall
    set_timing(params[0], None)
    ms = start.elapsed_time(stop) / args.steps
    value = N / (ms * 1e-3)
    if pairs:
        dom_ms = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
        dom_src = "live: stage events in every timed step"
    else:
        dom_ms = stage_ms[dom_sid]
        dom_src = "stage events in untimed eager steps (graph mode)"

    dom = stage_names[dom_sid]
    work = stage_work(w, dom_sid)
    intensity = work["flops"] / max(work["bytes"], 1)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if work["flops"] and intensity >= ridge:
        achieved = work["flops"] / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = work["bytes"] / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = counter_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["us_per_launch"] = dom_ms * 1e3
    roof["duration_source"] = dom_src
    roof["algorithmic"] = {"bytes": work["bytes"], "flops": work["flops"]}

    stages = {}
    enc_flops = enc_ms = 0.0
    for sid, name in stage_names.items():
        wk = stage_work(w, sid)
        t = stage_ms[sid]
        stages[name] = {"us": round(t * 1e3, 2), "GB_s": round(wk["bytes"] / (t * 1e-3) / 1e9, 1),
                        "TFLOP_s": round(wk["flops"] / (t * 1e-3) / 1e12, 2)}
        if sid not in (0, 14):
            enc_flops += wk["flops"]
            enc_ms += t
    topk_w = stage_work(w, 0)
    topk_gbs = topk_w["bytes"] / (stage_ms[0] * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "blocks/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_blocks": N, "slots": B, "vocab": V, "topk": K,
                   "hidden": H, "heads": w.heads, "ffn": F, "d_e": de, "alpha": w.alpha,
                   "use_logp": bool(w.use_logp), "head": "paper" if w.target_hidden else "lattice",
                   "target_hidden": w.target_hidden, "drafter_hidden": w.drafter_hidden,
                   "logits": f"{w.dtype} {w.recipe}", "weights": "seeded random (SplitMix64)",
                   "graph": bool(args.graph), "rotating_logits_buffers": nbuf, "rule": args.rule},
        "roofline": roof,
        "topk_hbm": {"achieved_GB_s": topk_gbs, "frac": topk_gbs / PEAK_HBM_GBS},
        "encoder_mfma": {"achieved_TFLOP_s": enc_flops / (enc_ms * 1e-3) / 1e12,
                         "frac": enc_flops / (enc_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                         "counters": counter_mfma(w.name)},
        "stages": stages,
        "wall_s_timed": wall,
    }

    # step-time spread: a separate untimed pass, each step between its own
    # event pair (the timed region above carries no per-step events, so its
    # mean is not inflated by them)
    n_spread = min(args.steps, 100)
    spread_ev = [(new_event(), new_event()) for _ in range(n_spread)]
    torch.cuda.synchronize()
    for i in range(n_spread):
        spread_ev[i][0].record(stream)
        run()
        spread_ev[i][1].record(stream)
    spread_ev[-1][1].synchronize()
    st_ms = np.sort(np.array([a.elapsed_time(b) for a, b in spread_ev]))
    result["step_ms"] = {"median": float(np.median(st_ms)), "p10": float(np.percentile(st_ms, 10)),
                         "p90": float(np.percentile(st_ms, 90)), "steps": n_spread,
                         "blocks_per_s_at_median": N / (float(np.median(st_ms)) * 1e-3),
                         "source": "per-step event pairs in a separate untimed pass after the timed steps"}
    props = torch.cuda.get_device_properties(dev)
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count,
                        "memory_GiB": round(props.total_memory / 2**30, 1)}

    if args.topk_shards > 0:
        result["topk_sharded"] = bench_topk_shards(L, w, bufs[0].view(N * B, V), args.topk_shards,
                                                   args.rotate_mib, max(args.steps, 20), stream)

    if args.clock_probe:
        try:
            result["clock"] = clock_probe(L, w, run, ms, roof, stream)
        except Exception as e:   # a diagnostic: its failure must not cost the bench line
            result["clock"] = {"error": f"{type(e).__name__}: {e}"}

    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)
    if args.copy_probe_mib > 0:
        n = int(args.copy_probe_mib * 2 ** 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)    # reads and writes n * 4 bytes once each
        torch.cuda.synchronize()


# gfx950's dense bf16 MFMA peak is quoted at its 2.4 GHz peak shader clock
PEAK_CLOCK_GHZ = 2.4


def clock_probe(L, w, run, ms_step, roof, stream):
    """Shader clock (GHz) read by the library's probe (one wave on a second
    stream comparing the shader-clock counter with the 100 MHz constant
    counter over a window) with the GPU idle, beside full steps on the main
    stream, and beside repeated calls of the dominant linear (random operands
    of its shape). `concurrent` says whether the probe's window ended before
    the work beside it did, i.e. whether the reading is of that work."""
    import torch
    side = torch.cuda.Stream()
    out = torch.zeros(2, dtype=torch.int64, device=stream.device)

    def read():
        v = out.cpu().tolist()
        return 0.1 * v[1] / max(v[0], 1)

    def beside(work, total_ms):
        # the probe covers the middle of the work's span
        window_us = max(1, int(total_ms * 1e3 * 0.6))
        e0 = torch.cuda.Event(enable_timing=True)
        e_probe = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            torch.cuda._sleep(int(total_ms * 1e3 * 0.2 * 1000))   # start inside the work
            L.clock_probe(out, window_us, side)
            e_probe.record(side)
        work()
        e1.record(stream)
        torch.cuda.synchronize()
        return read(), e0.elapsed_time(e_probe) < e0.elapsed_time(e1)

    torch.cuda.synchronize()
    L.clock_probe(out, 2000, stream)
    torch.cuda.synchronize()
    res = {"idle_GHz": round(read(), 3)}
    n_steps = max(4, int(math.ceil(20.0 / max(ms_step, 1e-3))))
    def steps():
        for _ in range(n_steps):
            run()

    ghz, ok = beside(steps, n_steps * ms_step)
    res["steps_GHz"] = round(ghz, 3)
    res["steps_concurrent"] = ok
    dom = roof["kernel"]
    shapes = {"linear_ffn1": (w.hidden, w.ffn, L.EPI_SILU_BF16), "linear_ffn2": (w.ffn, w.hidden, L.EPI_RESID_F32),
              "linear_qkv": (w.hidden, 3 * w.hidden, L.EPI_BF16), "linear_o": (w.hidden, w.hidden, L.EPI_RESID_F32)}
    key = dom.split(".")[0]
    if key in shapes and roof["unit"] == "TFLOP/s":
        kd, n, epi = shapes[key]
        m = w.num_blocks * w.slots * w.topk
        g = torch.Generator(device=stream.device).manual_seed(5)
        A = (torch.randn((m, kd), device=stream.device, generator=g) * 0.5).to(torch.bfloat16)
        Wt = (torch.randn((n, kd), device=stream.device, generator=g) * 0.03).to(torch.bfloat16)
        b = torch.zeros(n, dtype=torch.float32, device=stream.device)
        r = torch.zeros((m, n), dtype=torch.float32, device=stream.device) if epi == L.EPI_RESID_F32 else None
        wsz = L.lib().lilicorr_linear_workspace_bytes(m, kd, n)
        wsp = torch.empty(max(wsz, 256), dtype=torch.uint8, device=stream.device)
        L.linear(A, Wt, b, epi, r, wsp)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        L.linear(A, Wt, b, epi, r, wsp)
        t1.record(stream)
        torch.cuda.synchronize()
        call_ms = t0.elapsed_time(t1)
        calls = max(4, int(math.ceil(20.0 / max(call_ms, 1e-3))))
        def linears():
            for _ in range(calls):
                L.linear(A, Wt, b, epi, r, wsp)

        ghz, ok = beside(linears, calls * call_ms)
        peak = PEAK_BF16_TFLOPS * ghz / PEAK_CLOCK_GHZ
        res.update({"dominant_kernel": dom, "dominant_kernel_GHz": round(ghz, 3),
                    "dominant_concurrent": ok,
                    "mfma_peak_at_that_clock_TFLOP_s": round(peak, 1),
                    "roofline_frac_at_that_clock": round(roof["achieved"] / peak, 4)})
    res["method"] = ("lilicorr_clock_probe: shader-clock cycles (s_memtime) per 100 MHz constant-counter "
                     "tick (s_memrealtime) over a window inside the work; peaks scale with clock from "
                     f"{PEAK_BF16_TFLOPS:.0f} TFLOP/s at {PEAK_CLOCK_GHZ} GHz")
    return res


def bench_topk_shards(L, w, logits2d, G, rotate_mib, reps, stream):
    """Time the split-vocabulary top-K: the shard kernel on one shard's slice
    (the work one GPU of a G-way tensor-parallel head does) and the merge of the
    G shard outputs, each bracketed by events on the library's stream."""
    import math
    import torch
    rows, V = logits2d.shape
    K = w.topk
    dev = logits2d.device
    # contiguous split of the vocabulary, the first V % G shards one longer
    base, extra = divmod(V, G)
    edges = [0]
    for g in range(G):
        edges.append(edges[-1] + base + (1 if g < extra else 0))
    bounds = list(zip(edges[:-1], edges[1:]))
    val = torch.empty((G, rows, K), dtype=torch.float32, device=dev)
    idx = torch.empty((G, rows, K), dtype=torch.int32, device=dev)
    ms = torch.empty((G, rows, 2), dtype=torch.float32, device=dev)
    for g, (lo, hi) in enumerate(bounds):
        L.topk_shard(logits2d[:, lo:hi].contiguous(), K, lo, out=(val[g], idx[g], ms[g]))
    lo, hi = bounds[0]
    sl = logits2d[:, lo:hi].contiguous()
    nrot = max(1, math.ceil(rotate_mib * 2 ** 20 / (sl.numel() * sl.element_size())))
    slices = [sl] + [sl.clone() for _ in range(nrot - 1)]
    nbytes = int(L.lib().lilicorr_topk_shard_workspace_bytes(rows, hi - lo, K))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    outs = (torch.empty((rows, K), dtype=torch.float32, device=dev),
            torch.empty((rows, K), dtype=torch.int32, device=dev),
            torch.empty((rows, 2), dtype=torch.float32, device=dev))

    def timed(fn):
        for i in range(3):
            fn(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(reps):
            fn(i)
        b.record(stream)
        b.synchronize()
        return a.elapsed_time(b) / reps * 1e3

    shard_us = timed(lambda i: L.topk_shard(slices[i % nrot], K, lo, out=outs, workspace=ws))
    merge_us = timed(lambda i: L.topk_merge(val, idx, ms))
    by = rows * (hi - lo) * logits2d.element_size()
    return {"shards": G, "shard_shape": [rows, hi - lo], "shard_us": shard_us,
            "shard_GB_s": by / (shard_us * 1e-6) / 1e9, "shard_frac": by / (shard_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "merge_us": merge_us, "note": "one shard's kernel (cold input) and the merge of G shard "
                                          "outputs; the all-gather between GPUs is not run (one GPU)"}


def set_timing(params, sid, begin=None, end=None):
    """Point the library's stage-timing events at (begin, end) for stage sid."""
    import ctypes
    if sid is None:
        params.timing_begin = None
        params.timing_end = None
        params.timing_stage = 0
        return
    params.timing_stage = sid
    params.timing_begin = ctypes.c_void_p(begin.cuda_event)
    params.timing_end = ctypes.c_void_p(end.cuda_event)


def stage_table(w):
    """lilicorr_stage id -> name (layer stages of layer l at base + 5 l)."""
    names = {0: "topk_lse", 1: "node_build", 2: "linear_conf_w2"}
    for l in range(2):
        for j, n in enumerate(["linear_qkv", "lattice_attention", "linear_o", "linear_ffn1", "linear_ffn2"]):
            names[3 + j + 5 * l] = f"{n}.l{l}"
    names[13] = "linear_heads"
    names[14] = "scores_walk"
    return names


def stage_work(w, sid):
    """Algorithmic bytes and flops of one stage for one call over the workload."""
    N, B, V, K = w.num_blocks, w.slots, w.vocab, w.topk
    H, F, de, h = w.hidden, w.ffn, w.d_e, w.heads
    Ht, Hd = w.target_hidden, w.drafter_hidden
    paper = Ht > 0
    rows = N * B
    Bl = B - 1 if paper else B           # slots in the lattice
    T = Bl * K
    M = N * T                            # lattice rows
    es = 2 if w.dtype == "bf16" else 4

    def lin(kd, n, a_b, out_b, resid=False, norm_out=False, m=None):
        m = M if m is None else m
        by = m * kd * a_b + n * kd * 2 + n * 4 + m * n * out_b
        if resid:
            by += m * n * 4          # residual read (the write is out_b)
        if norm_out:
            by += m * n * 2          # bf16 RMSNorm output
        return {"bytes": by, "flops": 2 * m * n * kd}

    def add(*parts):
        return {"bytes": sum(p["bytes"] for p in parts), "flops": sum(p["flops"] for p in parts)}

    layer = sid - 3
    if sid == 0:
        return {"bytes": rows * V * es + rows * (8 * K + 4), "flops": 0}
    if sid == 1:
        # first confidence layer: reads the ids and log-probabilities, writes hid (bf16)
        node = {"bytes": H * (5 * 2 + 4) + M * 8 + M * H * 2, "flops": 2 * M * H * 5}
        if not paper:
            # the lattice head's table sum is formed in the next stage
            return node
        # slot/rank tables, projected drafter states (read per node), the
        # gathered E_t rows; writes x (f32)
        node["bytes"] += 2 * 64 * H * 2 + M * H * 4 + 2 * M * Ht * 2 + M * H * 4
        node["flops"] += 4 * M * H
        return add(lin(Hd, H, 2, 4, m=rows), node)
    if sid == 2:
        if not paper:
            # the residual is rebuilt from the tables: E rows by id, slot and rank rows
            tables = {"bytes": M * 4 + M * H * 2 + 2 * 64 * H * 2, "flops": 2 * M * H}
            return add(lin(H, H, 2, 4, norm_out=True), tables)
        return add(lin(H, H, 2, 4, resid=True), lin(Ht, H, 2, 4, resid=True, norm_out=True))
    # few rows with d_h = 128 and 65..128 tokens: the attention launch also
    # multiplies by W_o (the library's attention_o_fusable), and the O stage is
    # the residual + RMSNorm reduce
    fused_o = (H == h * 128 and 64 < T <= 128 and M < 2048 and h in (2, 3, 4, 6, 8, 12, 16))
    if 3 <= sid <= 12:
        j = layer % 5
        if j == 0:
            return lin(H, 3 * H, 2, 2)
        if j == 1:
            att = {"bytes": M * 3 * H * 2 + M * H * 2 + h * 128 * 4,
                   "flops": 4 * N * h * T * T * (H // h)}
            if fused_o:
                # W_o read and the product instead of the bf16 output write
                att = {"bytes": M * 3 * H * 2 + H * H * 2 + h * 128 * 4,
                       "flops": att["flops"] + 2 * M * H * H}
            return att
        if j == 2:
            if fused_o:
                return {"bytes": H * 4 + M * H * 4 + M * H * 4 + M * H * 2, "flops": 0}
            return lin(H, H, 2, 4, resid=True, norm_out=True)
        if j == 3:
            return lin(H, F, 2, 2)
        return lin(F, H, 2, 4, resid=True, norm_out=True)
    if sid == 13:
        if not paper:
            return lin(H, 2 * de, 2, 2)
        tnorm = {"bytes": N * Ht * 4 + Ht * 4, "flops": 3 * N * Ht}
        concat = {"bytes": M * H * 2 + N * H * 2 + M * 3 * H * 2, "flops": M * H}
        anchor = {"bytes": N * de * 4 + 2 * N * K * de * 2, "flops": 3 * N * de}
        return add(tnorm, lin(Ht, H, 2, 2, m=N), lin(H, de, 2, 4, m=N), concat,
                   lin(3 * H, H, 2, 2), lin(H, 2 * de, 2, 2), anchor)
    return {"bytes": 2 * rows * K * de * 2 + rows * K * 8 + rows * 4,
            "flops": 2 * N * (B - 1) * K * K * de}


def counter_traffic(workload, stage):
    """HBM bytes per launch of a stage from the committed rocprofv3 counter
    summary of this workload, if the kernel sources are unchanged since the
    counters were taken; else None."""
    import re
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"^csrc_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m_h or m_h.group(1) != csrc_sha256():
        return None
    m = re.search(r"^\|\s*" + re.escape(stage) + r"\s*\|\s*(\d+)\s*\|", text, re.M)
    return int(m.group(1)) if m else None


# Kernel roles, by name, for splitting a step's dispatch sequence into stages.
_GEMM_MAIN = ("gemm_kernel", "gemm_part_kernel", "gemm_dma_kernel", "gemm_fullk_kernel", "gemm_skinny_kernel",
              "gemm_skinny2_kernel")


def _fused_attention_o(name):
    """The attention launch that also forms the output projection's per-head
    K slices (few rows): its O linear is then only the split-K reduce."""
    import re
    return re.search(r"attention_res_kernel<[^>]*true>", name) is not None
_GEMM_TAIL = ("splitk_", "rmsnorm")
_LINEAR_ORDER = ["linear_conf_w2"] + [f"{n}.l{l}" for l in range(2)
                                      for n in ("linear_qkv", "linear_o", "linear_ffn1", "linear_ffn2")] \
    + ["linear_heads"]


def split_step_stages(names):
    """Stage name for each kernel of one step's dispatch sequence."""
    import re
    out, lin, att = [], 0, 0
    for n in names:
        if "topk_" in n:
            out.append("topk_lse")
        elif "node_build" in n:
            out.append("node_build")
        elif re.search(r"attention_\w*kernel", n):
            out.append(f"lattice_attention.l{att}")
            att += 1
            if _fused_attention_o(n):
                lin += 1   # the launch is also the O linear's product; its reduce follows
        elif any(k in n for k in _GEMM_MAIN):
            out.append(_LINEAR_ORDER[lin])
            lin += 1
        elif any(k in n for k in _GEMM_TAIL):
            out.append(_LINEAR_ORDER[lin - 1])
        elif "scores_walk" in n or "pair_scores" in n or "pair_slices" in n or "greedy_walk" in n:
            out.append("scores_walk")
        else:
            out.append(None)
    return out


def read_counter_csv(d, counter):
    """(dispatch id, kernel name, value) rows of one counter from a rocprofv3 CSV directory."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
            prev = rows.get(key)
            val = float(r["Counter_Value"]) + (prev[2] if prev else 0.0)
            rows[key] = (key, r["Kernel_Name"], val)
    return [rows[k] for k in sorted(rows)]


def summarize_counters(args):
    """Per-stage HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs."""
    scale = {}
    per_stage = {}
    for counter, d in zip(("FETCH_SIZE", "WRITE_SIZE"), args.summarize_counters):
        rows = read_counter_csv(d, counter)
        copy = [v for _, n, v in rows if "neg_kernel" in n or "neg" in n.split("<")[0]]
        ref_kib = args.copy_probe_mib * 1024
        if not copy or ref_kib <= 0:
            raise SystemExit("the counter runs need --copy-probe-mib and its copy kernel")
        scale[counter] = ref_kib / (sum(copy[-3:]) / len(copy[-3:]))
        # steps: from each top-K dispatch to the next scores/walk dispatch
        names = [n for _, n, _ in rows]
        i = 0
        while i < len(rows):
            if "topk_partial" not in names[i]:
                i += 1
                continue
            j = i
            while j < len(rows) and not ("scores_walk" in names[j] or "greedy_walk" in names[j]):
                j += 1
            if j >= len(rows):
                break
            seq = rows[i:j + 1]
            step_sum = {}
            for (_, n, v), st in zip(seq, split_step_stages([n for _, n, _ in seq])):
                if st is not None:
                    step_sum[st] = step_sum.get(st, 0.0) + v
            for st, v in step_sum.items():
                per_stage.setdefault(st, {}).setdefault(counter, []).append(v)
            i = j + 1
    w = args.workload
    print(f"# HBM traffic per stage launch: {w}\n")
    print("Counters: rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE (KiB per dispatch), one run each,")
    print("scaled by what the same counter reads for a plain copy kernel of known size")
    print(f"({args.copy_probe_mib:g} MiB read and written by torch.neg):")
    print(f"FETCH_SIZE scale {scale['FETCH_SIZE']:.4f}, WRITE_SIZE scale {scale['WRITE_SIZE']:.4f}.\n")
    print(f"csrc_sha256: {csrc_sha256()}\n")
    print("| stage | HBM bytes per launch (fetch + write) | fetch bytes | write bytes | steps |")
    print("|---|---|---|---|---|")
    for st, c in per_stage.items():
        f = c.get("FETCH_SIZE", [])
        wr = c.get("WRITE_SIZE", [])
        f_b = sum(f) / max(1, len(f)) * 1024 * scale["FETCH_SIZE"]
        w_b = sum(wr) / max(1, len(wr)) * 1024 * scale["WRITE_SIZE"]
        print(f"| {st} | {int(round(f_b + w_b))} | {int(round(f_b))} | {int(round(w_b))} | {len(f)} |")


def read_kernel_durations(d):
    """dispatch id -> duration (ns) from a rocprofv3 kernel-trace CSV, if present."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return {}
    out = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            try:
                out[int(r["Dispatch_Id"])] = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            except (KeyError, ValueError):
                continue
    return out


def summarize_mfma(args):
    """Per-stage MFMA counters of one workload: bf16 MFMA flops counted by the
    hardware (MfmaFlopsBF16 = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512) against the
    stage's algorithmic flops, and MFMA utilisation (MfmaUtil = MFMA-busy cycles
    over GRBM_GUI_ACTIVE cycles of all SIMDs), weighted by kernel duration over
    the stage's kernels."""
    d = args.summarize_mfma
    util = {k: (n, v) for k, n, v in read_counter_csv(d, "MfmaUtil")}
    flops = {k: (n, v) for k, n, v in read_counter_csv(d, "MfmaFlopsBF16")}
    dur = read_kernel_durations(d)
    ids = sorted(util)
    names = [util[k][0] for k in ids]
    import synth
    w = synth.WORKLOADS[args.workload]
    stage_ids = {v: k for k, v in stage_table(w).items()}
    per = {}
    i = 0
    while i < len(ids):
        if "topk_partial" not in names[i]:
            i += 1
            continue
        j = i
        while j < len(ids) and not ("scores_walk" in names[j] or "greedy_walk" in names[j]):
            j += 1
        if j >= len(ids):
            break
        seq = ids[i:j + 1]
        acc = {}
        for k, st in zip(seq, split_step_stages([util[k][0] for k in seq])):
            if st is None:
                continue
            a = acc.setdefault(st, [0.0, 0.0, 0.0])
            t = dur.get(k, 1.0)
            a[0] += flops.get(k, (None, 0.0))[1]
            a[1] += util[k][1] * t
            a[2] += t
        for st, a in acc.items():
            per.setdefault(st, []).append(a)
        i = j + 1
    print(f"# MFMA counters per stage launch: {w.name}\n")
    print("rocprofv3 --kernel-trace --pmc MfmaUtil MfmaFlopsBF16 (derived counters of")
    print("SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16), one run.")
    print("`util` = MFMA-busy cycles / (GRBM_GUI_ACTIVE x SIMDs), weighted by kernel duration over the")
    print("stage's kernels; `counted` = bf16 MFMA flops the hardware issued per launch;")
    print("`algorithmic` = the stage's flops from the method (bench.py stage_work).\n")
    print(f"csrc_sha256: {csrc_sha256()}\n")
    print("| stage | MFMA util % | counted bf16 MFMA flops | algorithmic flops | counted / algorithmic | us (trace) | steps |")
    print("|---|---|---|---|---|---|---|")
    tot_busy = tot_t = 0.0
    for st, lst in per.items():
        fl = sum(a[0] for a in lst) / len(lst)
        t = sum(a[2] for a in lst) / len(lst)
        u = sum(a[1] for a in lst) / max(sum(a[2] for a in lst), 1e-30)
        alg = stage_work(w, stage_ids[st])["flops"] if st in stage_ids else 0
        ratio = f"{fl / alg:.3f}" if alg else "-"
        if st not in ("topk_lse", "scores_walk"):
            tot_busy += u * t
            tot_t += t
        print(f"| {st} | {u:.1f} | {fl:.4g} | {alg:.4g} | {ratio} | {t / 1e3:.1f} | {len(lst)} |")
    if tot_t:
        print(f"\nencoder MFMA util (duration-weighted over node build .. heads): {tot_busy / tot_t:.1f} %")


def summarize_pmc(args):
    """Per-stage means of every counter in one or more rocprofv3 --pmc runs,
    each summed over the stage's kernels in a step. SQ_WAVE_CYCLES, the
    SQ_WAIT_* and the SQ_ACTIVE_INST_* counters share a unit (wave-cycles), so
    their ratios are the fractions of the waves' resident time spent waiting
    or issuing each instruction class."""
    import csv
    import glob
    import synth
    w = synth.WORKLOADS[args.workload]
    per = {}
    names_all = []
    for d in args.summarize_pmc:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no *counter_collection.csv under {d}")
        rows = {}
        with open(files[0]) as f:
            for r in csv.DictReader(f):
                key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
                ent = rows.setdefault(key, [r["Kernel_Name"], {}])
                c = r["Counter_Name"]
                ent[1][c] = ent[1].get(c, 0.0) + float(r["Counter_Value"])
        ids = sorted(rows)
        names = [rows[k][0] for k in ids]
        for c in (rows[ids[0]][1] if ids else {}):
            if c not in names_all:
                names_all.append(c)
        i = 0
        while i < len(ids):
            if "topk_partial" not in names[i]:
                i += 1
                continue
            j = i
            while j < len(ids) and not ("scores_walk" in names[j] or "greedy_walk" in names[j]):
                j += 1
            if j >= len(ids):
                break
            seq = ids[i:j + 1]
            acc = {}
            for k, st in zip(seq, split_step_stages([rows[k][0] for k in seq])):
                if st is None:
                    continue
                a = acc.setdefault(st, {})
                for c, v in rows[k][1].items():
                    a[c] = a.get(c, 0.0) + v
            for st, a in acc.items():
                for c, v in a.items():
                    per.setdefault(st, {}).setdefault(c, []).append(v)
            i = j + 1
    print(f"# SQ counters per stage launch: {w.name}\n")
    print("Means over the run's steps of each counter summed over a stage's kernels "
          "(rocprofv3 --pmc, one run per counter group).\n")
    print(f"csrc_sha256: {csrc_sha256()}\n")
    print("| stage | " + " | ".join(names_all) + " |")
    print("|---" * (len(names_all) + 1) + "|")
    for st, d in per.items():
        print(f"| {st} | " + " | ".join(f"{sum(d[c]) / len(d[c]):.4g}" if c in d else "-" for c in names_all) + " |")
    frac = [c for c in names_all if c.startswith(("SQ_WAIT_", "SQ_ACTIVE_INST_"))]
    if "SQ_WAVE_CYCLES" in names_all and frac:
        print("\nFractions of wave-resident time (counter / SQ_WAVE_CYCLES):\n")
        print("| stage | " + " | ".join(frac) + " |")
        print("|---" * (len(frac) + 1) + "|")
        for st, d in per.items():
            wc = sum(d["SQ_WAVE_CYCLES"]) / len(d["SQ_WAVE_CYCLES"]) if "SQ_WAVE_CYCLES" in d else 0.0
            print(f"| {st} | " + " | ".join(
                f"{sum(d[c]) / len(d[c]) / wc:.3f}" if c in d and wc else "-" for c in frac) + " |")


def counter_mfma(workload):
    """Encoder MFMA utilisation from the committed MfmaUtil summary of this
    workload, while the kernel sources hash the same; else None."""
    import re
    path = os.path.join(ROOT, "profiles", f"mfma_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_h = re.search(r"^csrc_sha256:\s*([0-9a-f]+)", text, re.M)
    if not m_h or m_h.group(1) != csrc_sha256():
        return None
    m = re.search(r"encoder MFMA util \(duration-weighted[^)]*\): ([0-9.]+) %", text)
    stages = {mm.group(1): float(mm.group(2)) for mm in
              re.finditer(r"^\|\s*([\w.]+)\s*\|\s*([0-9.]+)\s*\|", text, re.M)}
    return {"util_frac": float(m.group(1)) / 100 if m else None,
            "stage_util_frac": {k: v / 100 for k, v in stages.items()},
            "source": f"profiles/mfma_{workload}.md (rocprofv3 MfmaUtil)"}


def summarize_kernels(d):
    """Markdown table of a rocprofv3 run_kernel_stats.csv (durations in microseconds)."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    print("| kernel | calls | avg us | min us | max us | % of kernel time |")
    print("|---|---|---|---|---|---|")
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            name = r["Name"]
            m = re.search(r"(\w+(?:<[^()]*>)?)\(", name)
            short = m.group(1) if m else name[:60]
            print(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.2f} |")


def summarize_stage_kernels(d):
    """Per-stage kernel time per step from a rocprofv3 kernel trace (lattice head).

    Each step's dispatches (top-K through the walk) are split into stages by
    kernel role; a stage's duration is the sum of its kernels' durations in
    that step, averaged over every step of the run. Steps whose linear launches
    do not match the lattice head's sequence are left out."""
    import csv
    import glob
    import re
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        return
    with open(files[0]) as f:
        rows = sorted(((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                       for r in csv.DictReader(f)), key=lambda t: t[0])
    names = [n for _, n, _ in rows]
    per, kern, steps = {}, {}, 0
    i = 0
    while i < len(rows):
        if "topk_partial" not in names[i]:
            i += 1
            continue
        j = i
        while j < len(rows) and not ("scores_walk" in names[j] or "greedy_walk" in names[j]):
            j += 1
        if j >= len(rows):
            break
        seq = rows[i:j + 1]
        if sum(any(k in n for k in _GEMM_MAIN) or _fused_attention_o(n) for _, n, _ in seq) != len(_LINEAR_ORDER):
            i = j + 1
            continue
        step = {}
        for (_, n, ns), st in zip(seq, split_step_stages([n for _, n, _ in seq])):
            if st is None:
                continue
            step[st] = step.get(st, 0) + ns
            m = re.search(r"(\w+)(?:<|\()", n)
            kern.setdefault(st, [])
            short = m.group(1) if m else n[:40]
            if short not in kern[st]:
                kern[st].append(short)
        for st, ns in step.items():
            per.setdefault(st, []).append(ns)
        steps += 1
        i = j + 1
    if not steps:
        return
    print(f"\nPer stage, from the kernel trace ({steps} steps of the run): the sum of the stage's kernel")
    print("durations in a step, averaged over the steps.\n")
    print("| stage | kernels | mean us per step | min us |")
    print("|---|---|---|---|")
    for st in sorted(per, key=lambda k: -sum(per[k]) / len(per[k])):
        v = per[st]
        print(f"| {st} | {' + '.join(kern[st])} | {sum(v) / len(v) / 1e3:.2f} | {min(v) / 1e3:.2f} |")


def csrc_sha256():
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "draft_block_candidate_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


_CPU = {}


def _cpu_block(b):
    """One oracle pass over block b (the state is set up before the pool forks)."""
    st = _CPU
    import oracle
    w = st["w"]
    return oracle.rerank_block(st["host"][b], w.topk, st["ow"], w.alpha, w.use_logp, rule=st["rule"],
                               temperature=float(st["temps"][b]), uniforms=st["unif"][b],
                               hidden=None if st["hidden"] is None else st["hidden"][b],
                               target=None if st["target"] is None else st["target"][b])


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _BLAS_LIMIT
    _BLAS_LIMIT = threadpool_limits(1)     # held for the worker's life


def _cpu_chunk(blocks):
    for b in blocks:
        _cpu_block(b)
    return len(blocks)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, host, seconds, rule="greedy", max_workers=16):
    """The oracle, untuned, on this host, with the same commit rule (and, for
    sampling, the same temperatures and draws) as the GPU run. Two figures:
      * one core: BLAS limited to one thread, passes over the workload's
        blocks in order for about seconds / 2;
      * all cores: a fork-started process pool with one worker per core of this
        process's affinity mask (at most max_workers), BLAS limited to one
        thread in each, over about seconds / 2 worth of blocks.
    The dense weights are generated before timing (each pass generates its
    block's embedding rows, as the oracle does). `value` is the all-core figure."""
    import multiprocessing as mp
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    ow = oracle.OracleWeights(oracle.Dims(w.hidden, w.heads, w.ffn, w.d_e, target_hidden=w.target_hidden,
                                          drafter_hidden=w.drafter_hidden), w.vocab, synth.WEIGHTS_SEED)
    hidden = target = None
    if w.target_hidden > 0:
        hb, tb = synth.make_head_inputs(w)
        hidden = synth.bf16_bits_to_f32(hb).astype(np.float64)
        target = synth.bf16_bits_to_f32(tb).astype(np.float64)
    _CPU.update(w=w, host=host, ow=ow, rule=rule, temps=synth.make_temperatures(w.num_blocks, seed=1),
                unif=synth.make_uniforms(w.num_blocks, w.slots, seed=2), hidden=hidden, target=target)
    N = host.shape[0]
    with threadpool_limits(1):
        _cpu_block(0)                      # generates the dense weights: excluded
        n1 = 0
        t0 = time.perf_counter()
        while True:
            _cpu_block(n1 % N)
            n1 += 1
            el1 = time.perf_counter() - t0
            if el1 >= seconds / 2 or n1 >= 100000:
                break
    one_core = n1 / el1
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, max_workers))
    per_worker = max(1, int(round(one_core * seconds / 2)))
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        pool.map(_cpu_chunk, [[b % N] for b in range(workers)])          # warm the workers
        chunks = [[(k * workers + i) % N for k in range(per_worker)] for i in range(workers)]
        t0 = time.perf_counter()
        done = sum(pool.map(_cpu_chunk, chunks, chunksize=1))
        el = time.perf_counter() - t0
    all_core = done / el
    _CPU.clear()
    return {"value": all_core, "unit": "blocks/s", "cores": workers, "kind": "oracle",
            "sample": f"{done} oracle passes over the {w.name} blocks ({el:.1f} s) in a pool of {workers} "
                      f"processes, BLAS one thread each; float64 numpy; dense weight generation excluded",
            "one_core": {"value": one_core, "unit": "blocks/s", "cores": 1,
                         "sample": f"{n1} passes over the first blocks in order ({el1:.1f} s), BLAS one thread"},
            "affinity_cores": cores, "cpu_model": _cpu_model()}


if __name__ == "__main__":
    main()
