#!/usr/bin/env python3
"""Benchmark of the LiLiCorr reranking path on one MI355X.

One step = one lilicorr_rerank call over a batch of synthetic draft blocks:
fused log-partition + top-K, node build, two encoder layers, in/out heads,
pair scores and the greedy walk (every row of the hot path). The default
workload is the concurrency-1, Qwen3-8B-like block (1 block, B = 16,
V = 151,936 bf16 logits with three spikes per slot, K = 8, encoder width 1024,
8 heads, FFN 4096, d_e 128).

Logits are resident in HBM before timing; consecutive steps rotate over
enough logits buffers (>= 768 MiB in total) that each step reads its logits
cold, not from the 256 MiB Infinity Cache. Prints one JSON line.
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
    ap.add_argument("--workload", default="c1_qwen3_8b")
    ap.add_argument("--tier", type=int, default=0)
    ap.add_argument("--rotate-mib", type=float, default=768.0)
    ap.add_argument("--probe-reps", type=int, default=50)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step from a captured HIP graph")
    return ap.parse_args()


def event_time_ms(fn, reps, stream):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    stop.record(stream)
    stop.synchronize()
    return start.elapsed_time(stop) / reps


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(blocks are independent; see DESIGN.md for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_block_candidate_amd as L
    import synth

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    host = synth.make_logits(w, args.tier)
    esize = 2 if w.dtype == "bf16" else 4
    logit_bytes = host.nbytes
    nbuf = max(1, math.ceil(args.rotate_mib * 2 ** 20 / logit_bytes))
    first = torch.from_numpy(host.view(np.int16) if w.dtype == "bf16" else host).to(dev)
    if w.dtype == "bf16":
        first = first.view(torch.bfloat16)
    bufs = [first] + [first.clone() for _ in range(nbuf - 1)]
    dims = L.EncoderDims(w.hidden, w.heads, w.ffn, w.d_e)
    weights = L.Weights(dims, w.vocab, synth.WEIGHTS_SEED, device=dev)
    ws = L.Workspace(w.num_blocks, w.slots, w.vocab, w.topk, dims, device=dev)
    out = torch.empty((w.num_blocks, w.slots), dtype=torch.int32, device=dev)
    N, B, V, K = w.num_blocks, w.slots, w.vocab, w.topk
    ldt = L.BF16 if w.dtype == "bf16" else L.F32
    params = [L.make_params(N, ldt, weights, ws, w.alpha, True) for _ in range(1)]
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
    t_wall = time.perf_counter()
    ms = event_time_ms(run, args.steps, stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    value = N / (ms * 1e-3)

    # ---- live per-kernel probes (same kernels through the component entry points)
    M = N * B * K
    H, F, de = w.hidden, w.ffn, w.d_e
    probes = {}
    tk = {"i": 0}
    nb = len(bufs)
    rows = N * B

    def topk_probe():
        b = bufs[tk["i"] % nb]
        tk["i"] += 1
        L.topk_lse(b.view(rows, V), K)

    # allocation inside topk_lse happens through torch's caching allocator; warm it
    topk_probe()
    torch.cuda.synchronize()
    t_topk = event_time_ms(topk_probe, args.probe_reps, stream)
    topk_bytes = rows * V * esize + rows * (8 * K + 4)
    probes["topk_lse"] = {"ms": t_topk, "launches_per_step": 1, "bytes": topk_bytes, "flops": 0}

    g = torch.Generator(device="cpu").manual_seed(0)
    def rnd(shape, scale=1.0):
        return (torch.randn(shape, generator=g) * scale).to(torch.bfloat16).to(dev)
    shapes = {
        "linear_conf_w2": (M, H, H, L.EPI_RESID_F32, 1),
        "linear_qkv": (M, H, 3 * H, L.EPI_BF16, 2),
        "linear_o": (M, H, H, L.EPI_RESID_F32, 2),
        "linear_ffn1": (M, H, F, L.EPI_SILU_BF16, 2),
        "linear_ffn2": (M, F, H, L.EPI_RESID_F32, 2),
        "linear_heads": (M, H, 2 * de, L.EPI_F32, 1),
    }
    for name, (m, kd, n, epi, cnt) in shapes.items():
        A = rnd((m, kd))
        Wt = rnd((n, kd), 1 / math.sqrt(kd))
        bias = torch.zeros(n, dtype=torch.float32, device=dev)
        resid = torch.zeros((m, n), dtype=torch.float32, device=dev)
        lws = torch.empty(max(256, int(lib.lilicorr_linear_workspace_bytes(m, kd, n))), dtype=torch.uint8,
                          device=dev)
        fn = lambda: L.linear(A, Wt, bias, epi, resid if epi == L.EPI_RESID_F32 else None, lws)
        fn()
        torch.cuda.synchronize()
        t = event_time_ms(fn, args.probe_reps, stream)
        out_b = 4 if epi in (L.EPI_F32, L.EPI_RESID_F32) else 2
        nbytes = m * kd * 2 + n * kd * 2 + n * 4 + m * n * out_b + (m * n * 4 if epi == L.EPI_RESID_F32 else 0)
        probes[name] = {"ms": t, "launches_per_step": cnt, "bytes": nbytes, "flops": 2 * m * n * kd}
    qkv = rnd((M, 3 * H))
    dist = torch.zeros((w.heads, 127), dtype=torch.float32, device=dev)
    same = torch.zeros((w.heads,), dtype=torch.float32, device=dev)
    fn = lambda: L.lattice_attention(qkv, N, B, K, H, w.heads, dist, same)
    fn()
    torch.cuda.synchronize()
    T = B * K
    probes["lattice_attention"] = {"ms": event_time_ms(fn, args.probe_reps, stream), "launches_per_step": 2,
                                   "bytes": M * 3 * H * 2 + M * H * 2,
                                   "flops": 4 * N * w.heads * T * T * (H // w.heads)}

    for p in probes.values():
        p["ms_per_step"] = p["ms"] * p["launches_per_step"]
    dom_name = max(probes, key=lambda k: probes[k]["ms_per_step"])
    dom = probes[dom_name]
    intensity = dom["flops"] / max(dom["bytes"], 1)
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if dom["flops"] and intensity >= ridge:
        achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = dom_name

    enc_flops = sum(p["flops"] * p["launches_per_step"] for k, p in probes.items() if k != "topk_lse")
    enc_ms = sum(p["ms_per_step"] for k, p in probes.items() if k != "topk_lse")
    stages = {k: {"us": round(p["ms"] * 1e3, 3), "per_step": p["launches_per_step"],
                  "GB_s": round(p["bytes"] / (p["ms"] * 1e-3) / 1e9, 1),
                  "TFLOP_s": round(p["flops"] / (p["ms"] * 1e-3) / 1e12, 2)} for k, p in probes.items()}
    topk_gbs = topk_bytes / (t_topk * 1e-3) / 1e9

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
                   "logits": f"{w.dtype} {w.recipe}", "weights": "seeded random (SplitMix64)",
                   "graph": bool(args.graph), "rotating_logits_buffers": nbuf},
        "roofline": roof,
        "topk_hbm": {"achieved_GB_s": topk_gbs, "frac": topk_gbs / PEAK_HBM_GBS},
        "encoder_mfma": {"achieved_TFLOP_s": enc_flops / (enc_ms * 1e-3) / 1e12 if enc_ms else None,
                         "frac": (enc_flops / (enc_ms * 1e-3) / 1e12) / PEAK_BF16_TFLOPS if enc_ms else None},
        "stages": stages,
        "wall_s_timed": wall,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(w, host, seconds):
    """The oracle, untuned, on this host: repeated passes over the workload's blocks."""
    import oracle
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    ow = oracle.OracleWeights(oracle.Dims(w.hidden, w.heads, w.ffn, w.d_e), w.vocab, synth.WEIGHTS_SEED)
    oracle.rerank_block(host[0], w.topk, ow, w.alpha)   # generates the weights: excluded
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.rerank_block(host[n % host.shape[0]], w.topk, ow, w.alpha)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= 100000:
            break
    return {"value": n / el, "unit": "blocks/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} oracle passes over the {w.name} block(s) ({el:.1f} s; float64 numpy; "
                      f"weight generation excluded)"}


if __name__ == "__main__":
    main()
