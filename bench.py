#!/usr/bin/env python3
"""Benchmark of the routed-expert MoE layer with a GPU slot cache on one MI355X.

Headline workload (printed as the one JSON line on stdout): decode, 48 MoE
layers, d=2048, E=128 experts, top-8, f=768, bf16, one token per step; the
host bank holds all 6,144 layer-expert records (58 GB pinned), the slot cache
1,024 of them and starts cold; B_P/B_H = 20/60 GB/s; hidden states follow a
per-layer AR(1) stream.  A step is one token through all 48 layers: routing,
the control kernel, fills, GPU experts, host experts and the combine.
`value` is tokens/s over the K timed steps that follow W warm-up steps
(W + K = 256 by default).

Also reported: the live roofline of the dominant kernel (the decode gate/up
GEMV, HIP events on the stream it runs on), the oracle timed on the host
cores on a bounded sample, p50/p99 latency of each call of the decode path
(route, classify, forward), and a prefill section (8,192-token chunk: MFMA
utilisation of the grouped GEMMs with all experts resident, and 24 layers
streamed through the double buffer over PCIe).

    python bench.py [--gpus 1] [--steps 240] [--warmup 16]
"""
import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp4": 10100.0}
FP64_PEAK_TFLOPS = 78.6          # MI355X fp64 (vector and matrix)
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_sha():
    """Hash of the sources that define the one-token decode kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_wg.h", "wfmt.h"):
        with open(os.path.join(ROOT, "moe_expert_execution_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """The committed rocprofv3 counter summary of the decode kernel (HBM bytes
    per launch, and their ratio to the algorithmic bytes of the same run), if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        with open(path) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None
    if d.get("source_sha") != kernel_source_sha() or d.get("kernel") != kernel_key:
        return None
    return d


def time_route(M, shp, x, wr, T, ids, w, stream, reps=10):
    """Average time of one ft_moe_route call (torch events on the stream it runs on)."""
    import torch
    M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), T, ids.data_ptr(), w.data_ptr(), stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), T, ids.data_ptr(), w.data_ptr(), stream)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def decode_bench(args):
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["decode"]
    L, E, k, d, f, S = cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.S
    steps = args.warmup + args.steps
    t = time.time()
    bank = PinnedBank(L * E * S)
    synth.bank(cfg, out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
    log(f"decode bank {L * E * S / 1e9:.1f} GB pinned+generated in {time.time() - t:.1f}s")
    wr = torch.stack([torch.from_numpy(synth.router(cfg, l).view(np.int16)) for l in range(L)]).cuda()
    xs = torch.stack([torch.from_numpy(synth.ar1_tokens(cfg, l, steps).view(np.int16)) for l in range(L)]).cuda()
    ids = torch.empty((L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, k), dtype=torch.float32, device="cuda")
    y = torch.empty((L, d), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def new_cache():
        return SlotCache(L, E, k, d, f, "bf16", bank.ptr, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps)

    def step(h, shp, s):
        for l in range(L):
            xp = xs[l, s].data_ptr()
            M.ft_moe_route(shp, xp, wr[l].data_ptr(), 1, ids[l].data_ptr(), w[l].data_ptr(), stream)
            M.ft_cache_classify(h, l, ids[l].data_ptr(), 1, None, stream)
            M.ft_moe_forward(h, l, M.FT_MODE_CACHED, xp, ids[l].data_ptr(), w[l].data_ptr(), 1, y[l].data_ptr(),
                             stream)

    def run(sc, timed_kernels):
        """Cold cache: warm-up steps, then the timed steps; returns (seconds, stats before, stats after)."""
        h, shp = sc.handle, sc.shape
        for s in range(args.warmup):
            step(h, shp, s)
        torch.cuda.synchronize()
        a = M.ft_cache_stats(h).as_dict()
        M.ft_cache_set_timing(h, timed_kernels)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(args.warmup, steps):
            step(h, shp, s)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        b = M.ft_cache_stats(h).as_dict()
        return el, a, b

    # (1) the headline: tokens/s of the whole layer stack, nothing instrumented
    sc = new_cache()
    elapsed, s0, s1 = run(sc, False)
    assert s1["error_flags"] == 0, s1
    sc.close()
    # (2) the same run from a cold cache with every expert kernel timed by HIP
    # events (the per-launch event packets slow the whole step, so tokens/s
    # comes from (1)); cache counts and branch rates come from this run too
    sc = new_cache()
    h = sc.handle
    el2, s0, s1 = run(sc, True)
    tm = M.ft_cache_timing(h)
    assert s1["error_flags"] == 0, s1
    delta = {key: s1[key] - s0[key] for key in ("calls", "unique", "hits", "misses", "fills", "cpu_experts",
                                                "evictions", "bytes_filled", "host_experts", "host_bytes",
                                                "host_seconds")}
    # algorithmic bytes: each GPU-executed expert's gate and up banks are read
    # once by the gate/up GEMV, its down bank once by the down GEMV
    gu_bytes = 2 * f * d * 2
    dn_bytes = d * f * 2
    n_gu, n_dn = tm.launches[M.FT_K_GEMV_GU], tm.launches[M.FT_K_GEMV_DOWN]
    ms_gu, ms_dn = tm.ms[M.FT_K_GEMV_GU], tm.ms[M.FT_K_GEMV_DOWN]
    experts = tm.gemv_experts
    fused = n_dn == 0          # one launch per call: gate/up, SwiGLU and down together
    both_gbs = experts * (gu_bytes + dn_bytes) / ((ms_gu + ms_dn) / 1e3) / 1e9
    gu_gbs = experts * gu_bytes / (ms_gu / 1e3) / 1e9
    dn_gbs = experts * dn_bytes / (ms_dn / 1e3) / 1e9 if n_dn else None
    kernel_key = "decode_kernel<bf16,all>" if fused else "gemv_gateup_kernel<bf16,1>+gemv_down_kernel<bf16,1>"
    traffic = measured_traffic(kernel_key)
    res = {
        "value": args.steps / elapsed,
        "ms_per_step": elapsed / args.steps * 1e3,
        "ms_per_step_kernel_timed_run": el2 / args.steps * 1e3,
        # the decode expert GEMV of one layer call: gate/up with SwiGLU, then
        # down; the unit is the GPU-executed experts' records (G x S bytes),
        # so achieved = their bytes / the time of the call's expert launch(es)
        "roofline": {
            "bound": "hbm", "kernel": kernel_key, "achieved": both_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": both_gbs / HBM_PEAK_GBS, "traffic": traffic["traffic_bytes_per_launch"] if traffic else None,
            # the counters' run has its own experts per launch: their ratio to that run's algorithmic bytes
            "traffic_over_algorithmic": traffic["traffic_over_algorithmic"] if traffic else None,
            "bytes_per_launch": experts * (gu_bytes + dn_bytes) / max(n_gu, 1),
            "avg_launch_us": (ms_gu + ms_dn) / max(n_gu, 1) * 1e3, "launches": n_gu,
            "timing": "HIP events stamped by each launch on the caller's stream (kernel-timed run)",
        },
        "decode_kernels": {
            "gpu_experts_per_layer_step": experts / max(n_gu, 1),
        },
        "cache": {**delta, "layer_calls": delta["calls"],
                  "miss_rate": delta["misses"] / max(delta["unique"], 1)},
        "branches": {
            # achieved B_P: record bytes over the fill kernels' event time
            "fill_gbs": delta["bytes_filled"] / max(tm.ms[M.FT_K_FILL] / 1e3, 1e-12) / 1e9,
            "fill_ms_total": tm.ms[M.FT_K_FILL],
            # achieved B_H: record bytes the host workers read over their busy time
            "host_gbs": delta["host_bytes"] / max(delta["host_seconds"], 1e-12) / 1e9,
            "host_seconds_total": delta["host_seconds"],
            "host_threads_env": os.environ.get("FTMOE_HOST_THREADS", "default"),
        },
    }
    if not fused:
        res["roofline"]["gateup"] = {"achieved": gu_gbs, "frac": gu_gbs / HBM_PEAK_GBS,
                                     "bytes_per_launch": experts * gu_bytes / max(n_gu, 1),
                                     "avg_launch_us": ms_gu / max(n_gu, 1) * 1e3}
        res["roofline"]["down"] = {"achieved": dn_gbs, "frac": dn_gbs / HBM_PEAK_GBS,
                                   "bytes_per_launch": experts * dn_bytes / max(n_gu, 1),
                                   "avg_launch_us": ms_dn / max(n_gu, 1) * 1e3}
    log(f"decode: {res['value']:.1f} tok/s, {res['ms_per_step']:.2f} ms/step, expert kernels {both_gbs:.0f} GB/s "
        f"({both_gbs / HBM_PEAK_GBS:.1%}, {res['roofline']['avg_launch_us']:.2f} us per call), miss rate {res['cache']['miss_rate']:.2f}, "
        f"fill {res['branches']['fill_gbs']:.1f} GB/s, host {res['branches']['host_gbs']:.1f} GB/s "
        f"({delta['host_seconds']:.2f}s busy of {el2:.2f}s in the kernel-timed run)")
    # (3) hits only: the last step replayed on the warm cache with fills off
    # (max_fetch 0), so every GPU-executed expert is a resident record and each
    # is read again only after the other 47 layers (~2.7 GB of reads), far more
    # than the 256 MB Infinity Cache; a record that a fill has just written is
    # never among them.  Same experts per launch as the run above.
    M.ft_cache_set_timing(h, False)
    M.ft_cache_set_profile(h, M.profile(cfg.bp_mbps, cfg.bh_mbps, 0))
    step(h, sc.shape, steps - 1)
    torch.cuda.synchronize()
    q0 = M.ft_cache_stats(h).as_dict()
    M.ft_cache_set_timing(h, True)
    for _ in range(args.hits_only_reps):
        step(h, sc.shape, steps - 1)
    torch.cuda.synchronize()
    th = M.ft_cache_timing(h)
    q1 = M.ft_cache_stats(h).as_dict()
    assert q1["error_flags"] == 0 and q1["fills"] == q0["fills"], q1
    # back to the configured profile (ft_cache_profile keeps the cache's max_fetch)
    M.ft_cache_set_profile(h, M.profile(cfg.bp_mbps, cfg.bh_mbps, cfg.max_fetch))
    hx = th.gemv_experts
    ms_h = th.ms[M.FT_K_GEMV_GU] + th.ms[M.FT_K_GEMV_DOWN]
    res["decode_kernels"]["hits_only"] = {
        "expert_kernels_gbs": hx * (gu_bytes + dn_bytes) / (ms_h / 1e3) / 1e9,
        "frac": hx * (gu_bytes + dn_bytes) / (ms_h / 1e3) / 1e9 / HBM_PEAK_GBS,
        "avg_us_per_call": ms_h / max(th.launches[M.FT_K_GEMV_GU], 1) * 1e3,
        "gpu_experts_per_layer_step": hx / max(th.launches[M.FT_K_GEMV_GU], 1),
        "launches": th.launches[M.FT_K_GEMV_GU], "fills": q1["fills"] - q0["fills"],
        "workload": f"decode step {steps - 1} replayed {args.hits_only_reps} times on the warm cache, max_fetch 0",
    }
    log(f"decode hits only: expert kernels {res['decode_kernels']['hits_only']['expert_kernels_gbs']:.0f} GB/s, "
        f"{res['decode_kernels']['hits_only']['gpu_experts_per_layer_step']:.2f} experts per launch")
    if not args.no_measured_profile:
        # the same decode run again from a cold cache, with q* fed by this machine's measured B_P / B_H
        M.ft_cache_set_timing(h, False)
        prof = M.ft_cache_profile(h, 16)          # leaves the cache empty (cold)
        assert prof.max_fetch == cfg.max_fetch, prof.max_fetch
        try:
            from moe_expert_execution_amd import bwprofile
            bwprofile.save("bf16", bwprofile.gpu_key(), prof.bp_mbps, prof.bh_mbps,
                           directory=os.environ.get("FTMOE_PROFILE_DIR", bwprofile.DEFAULT_DIR))
        except Exception as exc:          # the store is a convenience; the measurement stands
            log(f"profile not stored: {exc}")
        M.ft_cache_set_profile(h, prof)
        for s_ in range(args.warmup):
            step(h, sc.shape, s_)
        torch.cuda.synchronize()
        p0 = M.ft_cache_stats(h).as_dict()
        t0 = time.perf_counter()
        for s_ in range(args.warmup, steps):
            step(h, sc.shape, s_)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        p1 = M.ft_cache_stats(h).as_dict()
        calls = max(p1["calls"] - p0["calls"], 1)
        res["measured_profile"] = {
            "bp_mbps": prof.bp_mbps, "bh_mbps": prof.bh_mbps,
            "tokens_per_s": args.steps / el, "ms_per_step": el / args.steps * 1e3,
            "fills_per_call": (p1["fills"] - p0["fills"]) / calls,
            "host_experts_per_call": (p1["cpu_experts"] - p0["cpu_experts"]) / calls,
            "miss_rate": (p1["misses"] - p0["misses"]) / max(p1["unique"] - p0["unique"], 1),
        }
        log(f"decode with the measured profile B_P/B_H {prof.bp_mbps / 1e3:.1f}/{prof.bh_mbps / 1e3:.1f} GB/s: "
            f"{args.steps / el:.1f} tok/s, fills {res['measured_profile']['fills_per_call']:.2f} and host experts "
            f"{res['measured_profile']['host_experts_per_call']:.2f} per layer call")
    sc.close()
    if not args.no_graph:
        # (4) the same steps from a cold cache, each one a replay of a HIP graph
        # that holds one whole decode step (48 x route + classify + forward;
        # the host experts run in captured host functions); the step's hidden
        # states are copied into the graph's input buffer first
        sc = new_cache()
        h = sc.handle
        xg = torch.empty((L, d), dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gst = torch.cuda.current_stream().cuda_stream
            for l in range(L):
                M.ft_moe_route(sc.shape, xg[l].data_ptr(), wr[l].data_ptr(), 1, ids[l].data_ptr(), w[l].data_ptr(),
                               gst)
                M.ft_cache_classify(h, l, ids[l].data_ptr(), 1, None, gst)
                M.ft_moe_forward(h, l, M.FT_MODE_CACHED, xg[l].data_ptr(), ids[l].data_ptr(), w[l].data_ptr(), 1,
                                 y[l].data_ptr(), gst)
        torch.cuda.synchronize()
        for s_ in range(args.warmup):
            xg.copy_(xs[:, s_])
            g.replay()
        torch.cuda.synchronize()
        g0 = M.ft_cache_stats(h).as_dict()
        t0 = time.perf_counter()
        for s_ in range(args.warmup, steps):
            xg.copy_(xs[:, s_])
            g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        g1 = M.ft_cache_stats(h).as_dict()
        assert g1["error_flags"] == 0, g1
        res["graph"] = {"tokens_per_s": args.steps / el, "ms_per_step": el / args.steps * 1e3,
                        "miss_rate": (g1["misses"] - g0["misses"]) / max(g1["unique"] - g0["unique"], 1),
                        "same_decisions_as_headline": all(g1[k_] - g0[k_] == s1[k_] - s0[k_]
                                                          for k_ in ("hits", "misses", "fills", "cpu_experts"))}
        log(f"decode replayed from a HIP graph of one step: {args.steps / el:.1f} tok/s ({el / args.steps * 1e3:.2f} "
            f"ms/step), same decisions as the eager runs: {res['graph']['same_decisions_as_headline']}")
        del g
        sc.close()
    if not args.no_latency:
        # (5) latency of each call on the path: HIP events on the calls' stream
        # around every route, classify and forward of 2 steps x 48 layers
        # (after the warm-up, cold start); forward holds the planner + the
        # PCIe pull of the call's fills, the GPU experts and the combine
        sc = new_cache()
        h, shp = sc.handle, sc.shape
        for s_ in range(args.warmup):
            step(h, shp, s_)
        torch.cuda.synchronize()
        evs = []
        for s_ in range(args.warmup, args.warmup + min(2, args.steps)):
            for l in range(L):
                xp = xs[l, s_].data_ptr()
                e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
                e[0].record()
                M.ft_moe_route(shp, xp, wr[l].data_ptr(), 1, ids[l].data_ptr(), w[l].data_ptr(), stream)
                e[1].record()
                M.ft_cache_classify(h, l, ids[l].data_ptr(), 1, None, stream)
                e[2].record()
                M.ft_moe_forward(h, l, M.FT_MODE_CACHED, xp, ids[l].data_ptr(), w[l].data_ptr(), 1,
                                 y[l].data_ptr(), stream)
                e[3].record()
                evs.append(e)
        torch.cuda.synchronize()
        lat = {}
        for name, a_, b_ in (("route", 0, 1), ("classify", 1, 2), ("forward", 2, 3)):
            v = sorted(e[a_].elapsed_time(e[b_]) * 1e3 for e in evs)
            lat[name] = {"p50": v[len(v) // 2], "p99": v[min(len(v) - 1, int(0.99 * len(v)))], "calls": len(v)}
        res["latency_us"] = lat
        log("per-call latency (us, p50/p99): " +
            ", ".join(f"{n} {v['p50']:.1f}/{v['p99']:.1f}" for n, v in lat.items()))
        assert M.ft_cache_stats(h).error_flags == 0
        sc.close()
    return res, bank, cfg


def cpu_baseline(bank, cfg, sample_steps):
    """The oracle (route + slot-cache simulator + fp64 layer) on the host cores,
    on decode steps 0..sample_steps-1 of the same workload, all 48 layers."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import cache as OC, formats as OF, moe as OM, route as OR
    L, E, k = cfg.layers, cfg.E, cfg.k
    recs = bank.records(cfg.S)
    xs = [synth.ar1_tokens(cfg, l, sample_steps) for l in range(L)]
    wrs = [synth.router(cfg, l) for l in range(L)]
    sim = OC.SlotCacheSim(L, E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    part = {"route": 0.0, "simulator": 0.0, "layer": 0.0}
    clk = time.perf_counter
    t0 = clk()
    for s in range(sample_steps):
        for l in range(L):
            x = xs[l][s:s + 1]
            ta = clk()
            ids, w, _ = OR.route(x, wrs[l], k)
            tb = clk()
            sim.classify(l, ids)
            tc = clk()
            OM.moe_layer(x, ids, w, lambda e: OF.decode_record(recs[l * E + e], cfg.fmt, cfg.d, cfg.f))
            td = clk()
            part["route"] += tb - ta
            part["simulator"] += tc - tb
            part["layer"] += td - tc
    el = clk() - t0
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    cores = len(os.sched_getaffinity(0))
    calls = sample_steps * L
    return {"value": sample_steps / el, "unit": "tokens/s", "cores": cores,
            "blas_threads": blas[0].get("num_threads") if blas else 1,
            "blas_library": blas[0].get("internal_api") if blas else None,
            "kind": "oracle", "seconds": el,
            "us_per_layer_call": {key: v / calls * 1e6 for key, v in part.items()},
            "sample": f"decode steps 0..{sample_steps - 1} x {L} layers (route + LRU simulator + fp64 layer)"}


def prefill_bench(args):
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["prefill"]
    L, E, k, d, f, S, T = cfg.stream_layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.S, cfg.tokens[0]
    t = time.time()
    bank = PinnedBank(L * E * S)
    synth.bank(cfg.with_(layers=L), out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
    log(f"prefill bank {L * E * S / 1e9:.1f} GB in {time.time() - t:.1f}s")
    sc = SlotCache(L, E, k, d, f, "bf16", bank.ptr, 2 * E, T, cfg.bp_mbps, cfg.bh_mbps)
    h, shp = sc.handle, sc.shape
    stream = torch.cuda.current_stream().cuda_stream
    x = torch.from_numpy(synth.tokens(cfg, T, 7).view(np.int16)).cuda()
    wr = torch.stack([torch.from_numpy(synth.router(cfg, l).view(np.int16)) for l in range(L)]).cuda()
    ids = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        M.ft_moe_route(shp, x.data_ptr(), wr[l].data_ptr(), T, ids[l].data_ptr(), w[l].data_ptr(), stream)
    torch.cuda.synchronize()
    route_ms = time_route(M, shp, x, wr[0], T, ids[0], w[0], stream)

    def fwd(l, flags=M.FT_PREFETCH_NEXT):
        M.ft_moe_forward(h, l, M.FT_MODE_STREAMED | flags, x.data_ptr(), ids[l].data_ptr(), w[l].data_ptr(), T,
                         y.data_ptr(), stream)

    # (1) grouped GEMMs with layer 0 resident in buffer 0 (loaded by the first
    # call; no transfer in the timed loop)
    fwd(0, 0)
    torch.cuda.synchronize()
    M.ft_cache_set_timing(h, True)
    reps = 10
    t0 = time.perf_counter()
    for _ in range(reps):
        fwd(0, 0)
    torch.cuda.synchronize()
    t_layer = (time.perf_counter() - t0) / reps
    tm = M.ft_cache_timing(h)
    rows = tm.gemm_rows / reps
    fl_gu, fl_dn = 2.0 * rows * d * 2 * f, 2.0 * rows * f * d
    ms_gu = tm.ms[M.FT_K_GEMM_GU] / reps
    ms_dn = tm.ms[M.FT_K_GEMM_DOWN] / reps
    tf_gu = fl_gu / (ms_gu / 1e3) / 1e12
    tf_dn = fl_dn / (ms_dn / 1e3) / 1e12
    tf_pair = (fl_gu + fl_dn) / ((ms_gu + ms_dn) / 1e3) / 1e12
    M.ft_cache_set_timing(h, False)
    # (2) all layers streamed through the double buffer, prefetching layer
    # l+1; an untimed pass first leaves layers L-2 and L-1 in the buffers, so
    # the timed pass loads every layer (the bytes moved come from the
    # library's own layer-load counter)
    for l in range(L):
        fwd(l)
    torch.cuda.synchronize()
    loads0 = M.ft_cache_stats(h).layers_streamed
    t0 = time.perf_counter()
    for l in range(L):
        fwd(l)
    torch.cuda.synchronize()
    t_stream = time.perf_counter() - t0
    st = M.ft_cache_stats(h)
    assert st.error_flags == 0
    loads = st.layers_streamed - loads0
    bytes_stream = loads * E * S
    # (2b) the stream once more with kernel timing on: the GEMMs as they run
    # inside it, each pair after ~20 ms of layer transfer (the back-to-back
    # repetitions of (1) heat the chip, and its clock drops as they go)
    M.ft_cache_set_timing(h, True)
    for l in range(L):
        fwd(l)
    torch.cuda.synchronize()
    tms = M.ft_cache_timing(h)
    M.ft_cache_set_timing(h, False)
    rows_s = tms.gemm_rows / L
    fs_gu, fs_dn = 2.0 * rows_s * d * 2 * f, 2.0 * rows_s * f * d
    ms_gu_s, ms_dn_s = tms.ms[M.FT_K_GEMM_GU] / L, tms.ms[M.FT_K_GEMM_DOWN] / L
    tf_pair_s = (fs_gu + fs_dn) / ((ms_gu_s + ms_dn_s) / 1e3) / 1e12
    # (3) the same layer transfers alone, no compute: one host-to-device copy of
    # the layer's E records per layer, the copy the double buffer issues
    dst = torch.empty(E * S, dtype=torch.uint8, device="cuda")
    src = torch.from_numpy(bank.array)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for l in range(L - loads, L):
        dst.copy_(src[l * E * S:(l + 1) * E * S], non_blocking=True)
    torch.cuda.synchronize()
    t_pcie = time.perf_counter() - t0
    del dst, src
    res = {
        "workload": f"prefill chunk T={T}, d={d}, E={E}, top-{k}, f={f}, bf16",
        "route": {"ms": route_ms, "gflop_fp64": 2.0 * T * d * E / 1e9,
                  "tflops_fp64": 2.0 * T * d * E / (route_ms / 1e3) / 1e12,
                  "frac_fp64_peak": 2.0 * T * d * E / (route_ms / 1e3) / 1e12 / FP64_PEAK_TFLOPS},
        # back to back: layer 0 resident, 10 repetitions in a row (sustained clock)
        "gemm": {"dtype": "bf16", "peak_tflops": MFMA_PEAK_TFLOPS["bf16"],
                 "gateup_tflops": tf_gu, "down_tflops": tf_dn, "pair_tflops": tf_pair,
                 "frac": tf_pair / MFMA_PEAK_TFLOPS["bf16"], "gateup_ms": ms_gu, "down_ms": ms_dn,
                 "layer_ms_resident": t_layer * 1e3, "rows": rows},
        # inside the 24-layer stream, one pair per layer
        "gemm_in_stream": {"gateup_tflops": fs_gu / (ms_gu_s / 1e3) / 1e12,
                           "down_tflops": fs_dn / (ms_dn_s / 1e3) / 1e12, "pair_tflops": tf_pair_s,
                           "frac": tf_pair_s / MFMA_PEAK_TFLOPS["bf16"], "gateup_ms": ms_gu_s,
                           "down_ms": ms_dn_s, "rows": rows_s},
        "stream": {"layers": L, "layer_loads": loads, "bytes": bytes_stream, "seconds": t_stream,
                   "pcie_gbs": bytes_stream / t_stream / 1e9, "tokens_per_s": T / t_stream,
                   "compute_only_s": L * t_layer, "gpu_busy_frac": L * t_layer / t_stream,
                   "pcie_only_s": t_pcie, "pcie_only_gbs": bytes_stream / t_pcie / 1e9,
                   # 1.0 = the stream takes no longer than the slower of its two parts alone
                   "overlap": max(t_pcie, L * t_layer) / t_stream},
    }
    log(f"prefill: route {route_ms * 1e3:.0f} us ({res['route']['tflops_fp64']:.1f} TFLOP/s fp64); "
        f"GEMM pair {tf_pair:.0f} TFLOP/s back to back ({res['gemm']['frac']:.1%} of bf16 peak), "
        f"{tf_pair_s:.0f} inside the stream ({tf_pair_s / MFMA_PEAK_TFLOPS['bf16']:.1%}), layer "
        f"{t_layer * 1e3:.2f} ms; stream {res['stream']['pcie_gbs']:.1f} GB/s over {L} layers in {t_stream:.2f}s "
        f"(copies alone {t_pcie:.2f}s, overlap {res['stream']['overlap']:.3f})")
    sc.close()
    bank.close()
    return res

def expert_bytes(fmt, d, f):
    """Algorithmic bytes of one expert's gate+up banks and of its down bank (codes and scales)."""
    if fmt == "bf16":
        return 2 * f * d * 2, d * f * 2
    if fmt == "fp8":
        sc = (f // 128) * (d // 128) * 4
        return 2 * f * d + 2 * sc, d * f + sc
    return 2 * f * d // 2 + 2 * f * d // 32, d * f // 2 + d * f // 32


def formats_bench(args):
    """Block-FP8 and MXFP4 layers with one layer resident (STREAMED buffer 0, 2E slots): the decode GEMV at
    T = 1 over fresh tokens (each call routes to other experts, so successive calls read different records
    and the working set is the whole layer, far above the Infinity Cache), and the grouped GEMM at the
    prefill token counts of each configuration."""
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    out = {}
    stream = torch.cuda.current_stream().cuda_stream
    for name, Ts in (("fp8", (64, 2048)), ("mxfp4", (4096,))):
        cfg = synth.CONFIGS[name].with_(layers=1, layer_alias=0)
        E, k, d, f, S = cfg.E, cfg.k, cfg.d, cfg.f, cfg.S
        t = time.time()
        bank = PinnedBank(E * S)
        synth.bank(cfg, out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
        log(f"{name} bank {E * S / 1e9:.1f} GB in {time.time() - t:.1f}s")
        Tmax = max(Ts)
        sc = SlotCache(1, E, k, d, f, name, bank.ptr, 2 * E, Tmax, cfg.bp_mbps, cfg.bh_mbps)
        h, shp = sc.handle, sc.shape
        wr = torch.from_numpy(synth.router(cfg, 0).view(np.int16)).cuda()
        y = torch.empty((Tmax, d), dtype=torch.int16, device="cuda")
        gu_b, dn_b = expert_bytes(name, d, f)
        res = {"workload": f"one {name} layer resident: d={d}, E={E}, top-{k}, f={f}"}

        def routed(T, tag):
            x = torch.from_numpy(synth.tokens(cfg, T, tag).view(np.int16)).cuda()
            ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
            w = torch.empty((T, k), dtype=torch.float32, device="cuda")
            M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), T, ids.data_ptr(), w.data_ptr(), stream)
            return x, ids, w

        def fwd(x, ids, w, T):
            M.ft_moe_forward(h, 0, M.FT_MODE_STREAMED, x.data_ptr(), ids.data_ptr(), w.data_ptr(), T, y.data_ptr(),
                             stream)

        # decode GEMV: 96 single tokens, each routed afresh
        x1, ids1, w1 = routed(96, 11)
        fwd(x1[:1], ids1[:1], w1[:1], 1)          # loads the layer into buffer 0
        torch.cuda.synchronize()
        M.ft_cache_set_timing(h, True)
        for i in range(96):
            fwd(x1[i:i + 1], ids1[i:i + 1], w1[i:i + 1], 1)
        torch.cuda.synchronize()
        tm = M.ft_cache_timing(h)
        n = max(tm.launches[M.FT_K_GEMV_GU], 1)
        ex = tm.gemv_experts / n
        gu_us = tm.ms[M.FT_K_GEMV_GU] / n * 1e3
        dn_us = tm.ms[M.FT_K_GEMV_DOWN] / n * 1e3
        # one launch per call (gate/up, SwiGLU and down) unless down launches too
        fused = tm.launches[M.FT_K_GEMV_DOWN] == 0
        pair_gbs = ex * (gu_b + dn_b) / (gu_us + dn_us) / 1e3
        res["gemv_T1"] = {"experts_per_launch": ex,
                          "kernel": "decode_kernel (gate/up, SwiGLU, down in one launch)" if fused else
                                    "gate/up GEMV + down GEMV",
                          "us_per_call": gu_us + dn_us, "pair_gbs": pair_gbs, "pair_frac": pair_gbs / HBM_PEAK_GBS}
        M.ft_cache_set_timing(h, False)
        # grouped GEMM
        for T in Ts:
            x, ids, w = routed(T, 12)
            r_ms = time_route(M, shp, x, wr, T, ids, w, stream)
            fwd(x, ids, w, T)
            torch.cuda.synchronize()
            reps = 10
            M.ft_cache_set_timing(h, True)
            for _ in range(reps):
                fwd(x, ids, w, T)
            torch.cuda.synchronize()
            tm = M.ft_cache_timing(h)
            rows = tm.gemm_rows / reps
            act = tm.gemm_experts / reps
            ms_gu = tm.ms[M.FT_K_GEMM_GU] / reps
            ms_dn = tm.ms[M.FT_K_GEMM_DOWN] / reps
            fl = 2.0 * rows * 3 * d * f
            by = act * (gu_b + dn_b)
            ms = ms_gu + ms_dn
            tf = fl / (ms / 1e3) / 1e12
            gbs = by / (ms / 1e3) / 1e9
            t_roof = max(fl / (MFMA_PEAK_TFLOPS["bf16"] * 1e12), by / (HBM_PEAK_GBS * 1e9)) * 1e3
            res[f"gemm_T{T}"] = {"route_ms": r_ms,
                                 "route_frac_fp64_peak": 2.0 * T * d * E / (r_ms / 1e3) / 1e12 / FP64_PEAK_TFLOPS,
                                 "rows": rows, "active_experts": act, "gateup_ms": ms_gu, "down_ms": ms_dn,
                                 "tflops": tf, "mfma_frac_bf16": tf / MFMA_PEAK_TFLOPS["bf16"],
                                 "weight_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                                 "t_roofline_ms": t_roof, "roofline_frac": t_roof / ms}
            M.ft_cache_set_timing(h, False)
        st = M.ft_cache_stats(h)
        assert st.error_flags == 0
        log(f"{name}: T=1 expert kernel(s) {res['gemv_T1']['pair_gbs']:.0f} GB/s "
            f"({res['gemv_T1']['pair_frac']:.1%}, {res['gemv_T1']['us_per_call']:.1f} us per call), " +
            ", ".join(f"GEMM T={T} {res[f'gemm_T{T}']['tflops']:.0f} TFLOP/s / {res[f'gemm_T{T}']['weight_gbs']:.0f}"
                      f" GB/s ({res[f'gemm_T{T}']['roofline_frac']:.1%} of roofline time)" for T in Ts))
        out[name] = res
        sc.close()
        bank.close()
    return out


def buffer_ablation_bench(Ts=(4096, 8192, 16384)):
    """The prefill stream (24 layers of the prefill configuration from pinned
    host banks) with the full-layer double buffer and with one buffer, at
    several chunk lengths: tokens/s of each and the one-buffer slowdown."""
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["prefill"]
    L, E, k, d, f, S = cfg.stream_layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.S
    Tm = max(Ts)
    bank = PinnedBank(L * E * S)
    synth.bank(cfg.with_(layers=L), out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
    sc = SlotCache(L, E, k, d, f, "bf16", bank.ptr, 2 * E, Tm, cfg.bp_mbps, cfg.bh_mbps)
    h, shp = sc.handle, sc.shape
    stream = torch.cuda.current_stream().cuda_stream
    x = torch.from_numpy(synth.tokens(cfg, Tm, 7).view(np.int16)).cuda()
    ids = torch.empty((L, Tm, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, Tm, k), dtype=torch.float32, device="cuda")
    y = torch.empty((Tm, d), dtype=torch.int16, device="cuda")
    for l in range(L):     # routing is per token: the first T rows are the routes of a T-token chunk
        wr = torch.from_numpy(synth.router(cfg, l).view(np.int16)).cuda()
        M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), Tm, ids[l].data_ptr(), w[l].data_ptr(), stream)
    torch.cuda.synchronize()

    def stream_pass(T, flags):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            M.ft_moe_forward(h, l, M.FT_MODE_STREAMED | M.FT_PREFETCH_NEXT | flags, x.data_ptr(), ids[l].data_ptr(),
                             w[l].data_ptr(), T, y.data_ptr(), stream)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    stream_pass(Ts[0], 0)      # warm-up
    rows = []
    for T in Ts:
        t2 = stream_pass(T, 0)
        t1 = stream_pass(T, M.FT_SINGLE_BUFFER)
        rows.append({"T": T, "two_buffers_s": t2, "one_buffer_s": t1, "two_buffers_tokens_per_s": T / t2,
                     "one_buffer_tokens_per_s": T / t1, "one_buffer_slowdown": 1.0 - t2 / t1,
                     "pcie_gbs_two_buffers": L * E * S / t2 / 1e9})
        log(f"buffer ablation T={T}: two buffers {T / t2:.0f} tok/s ({t2:.3f}s), one buffer {T / t1:.0f} tok/s "
            f"({t1:.3f}s): {1.0 - t2 / t1:.1%} slower")
    # prefill-warms-decode variant: after a streamed chunk, decode control over
    # the same layers' AR(1) routing, with the streamed layers left volatile
    # (the default) or registered as residents (FT_WARM_DECODE)
    from moe_expert_execution_amd import replay as R
    _, trace = R.record_decode_trace(cfg.with_(layers=L), 0, 32)
    dev_trace = torch.from_numpy(trace).cuda()
    warm = {}
    for name, flag in (("volatile", 0), ("warm", M.FT_WARM_DECODE)):
        for l in range(L):
            M.ft_moe_forward(h, l, M.FT_MODE_STREAMED | M.FT_PREFETCH_NEXT | flag, x.data_ptr(), ids[l].data_ptr(),
                             w[l].data_ptr(), Ts[0], y.data_ptr(), stream)
        s0 = M.ft_cache_stats(h)
        work = dev_trace.clone()
        for st_ in range(trace.shape[0]):
            for l in range(L):
                M.ft_cache_classify(h, l, work[st_, l].data_ptr(), 1, None, stream)
        s1 = M.ft_cache_stats(h)
        warm[name] = {"misses": s1.misses - s0.misses, "unique": s1.unique - s0.unique,
                      "miss_rate": (s1.misses - s0.misses) / (s1.unique - s0.unique)}
    log(f"decode after a streamed prefill ({trace.shape[0]} steps x {L} layers, {2 * E} slots): miss rate "
        f"{warm['volatile']['miss_rate']:.3f} with volatile buffers, {warm['warm']['miss_rate']:.3f} with the last "
        f"two layers registered")
    assert M.ft_cache_stats(h).error_flags == 0
    sc.close()
    bank.close()
    return {"workload": f"prefill stream, {L} layers of d={d}, E={E}, top-{k}, f={f}, bf16 from pinned host banks",
            "rows": rows, "decode_after_prefill": warm}


def miss_replay_bench():
    """Decode-time miss rate vs cache capacity for four placement policies on
    identical traces: the decode workload's AR(1) routing (64 prompt steps,
    then 256 decode steps over 48 layers) and a Zipf(1.1) popularity (one
    layer of 256 experts; a 512-token prompt, then 2048 decode steps)."""
    import synth
    from moe_expert_execution_amd import replay as R
    out = {}
    t0 = time.perf_counter()
    cfg = synth.CONFIGS["decode"]
    prompt, trace = R.record_decode_trace(cfg, 64, 256)
    out["ar1"] = {"workload": f"decode AR(1) routing, L={cfg.layers}, E={cfg.E}, top-{cfg.k}, 256 steps after a "
                              f"64-step prompt; profile {cfg.bp_mbps // 1000}/{cfg.bh_mbps // 1000} GB/s",
                  "rows": R.miss_table(prompt, trace, cfg.E, cfg.k, cfg.bp_mbps, cfg.bh_mbps, extra_slots=(cfg.slots,))}
    cfg = synth.CONFIGS["fp8"]
    prompt, trace = R.record_zipf_trace(cfg, 512, 2048)
    out["zipf"] = {"workload": f"Zipf(1.1) popularity, L=1, E={cfg.E}, top-{cfg.k}, 2048 steps after a 512-token "
                               f"prompt; profile {cfg.bp_mbps // 1000}/{cfg.bh_mbps // 1000} GB/s",
                   "rows": R.miss_table(prompt, trace, cfg.E, cfg.k, cfg.bp_mbps, cfg.bh_mbps, extra_slots=(cfg.slots,))}
    for name, v in out.items():
        log(f"miss replay {name}: " + "; ".join(
            f"{r['capacity']:.0%} ft {r['freetoken']:.2f} lru {r['lru']:.2f} prefill {r['prefill']:.2f} "
            f"load {r['load']:.2f}" for r in v["rows"]))
    log(f"miss replay took {time.perf_counter() - t0:.1f}s")
    return out


def _stats_delta(a, b, keys=("calls", "unique", "hits", "misses", "fills", "cpu_experts", "evictions",
                               "bytes_filled", "host_experts", "host_bytes", "host_seconds")):
    return {key: b[key] - a[key] for key in keys}


def _kernel_figures(M, tm, fmt, d, f, calls):
    """Expert-kernel rooflines of a kernel-timed run: GEMV (HBM) and grouped
    GEMM (bf16 MFMA, HBM) over the algorithmic bytes and flops of the
    GPU-executed experts."""
    gu_b, dn_b = expert_bytes(fmt, d, f)
    out = {}
    n_gu = tm.launches[M.FT_K_GEMV_GU]
    if n_gu:
        ms = tm.ms[M.FT_K_GEMV_GU] + tm.ms[M.FT_K_GEMV_DOWN]
        by = tm.gemv_experts * (gu_b + dn_b)
        out["gemv"] = {"experts_per_call": tm.gemv_experts / n_gu,
                       "pair_gbs": by / (ms / 1e3) / 1e9, "pair_frac_hbm": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "pair_us_per_call": ms / n_gu * 1e3,
                       "launches_per_call": 1 if tm.launches[M.FT_K_GEMV_DOWN] == 0 else 2}
        if tm.launches[M.FT_K_GEMV_DOWN]:
            out["gemv"]["gateup_gbs"] = tm.gemv_experts * gu_b / (tm.ms[M.FT_K_GEMV_GU] / 1e3) / 1e9
    n_gm = tm.launches[M.FT_K_GEMM_GU]
    if n_gm:
        ms = tm.ms[M.FT_K_GEMM_GU] + tm.ms[M.FT_K_GEMM_DOWN]
        fl = 2.0 * tm.gemm_rows * 3 * d * f
        by = tm.gemm_experts * (gu_b + dn_b)
        t_roof = max(fl / (MFMA_PEAK_TFLOPS["bf16"] * 1e12), by / (HBM_PEAK_GBS * 1e9))
        out["gemm"] = {"mfma_dtype": "bf16", "tflops": fl / (ms / 1e3) / 1e12,
                       "frac_bf16_mfma": fl / (ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"],
                       "weight_gbs": by / (ms / 1e3) / 1e9, "frac_hbm": by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                       "roofline_frac": t_roof / (ms / 1e3), "rows_per_call": tm.gemm_rows / n_gm,
                       "experts_per_call": tm.gemm_experts / n_gm, "ms_per_call": ms / n_gm}
    if tm.launches[M.FT_K_FILL]:
        out["fill_ms_total"] = tm.ms[M.FT_K_FILL]
    return out


def fp8_config_bench(args):
    """The block-FP8 configuration as configured: one layer (d=4096, E=256,
    top-8, f=2048, e4m3 + 128x128 fp32 scales) through the CACHED path, a
    64-slot cache that starts cold for each token count, Zipf(1.1) routes
    (routing bypassed: ids and weights are inputs), B_P/B_H 20/60 GB/s;
    T = 1, 64, 2048 for 256, 256, 16 steps.  Per T: tokens/s of the whole
    run (no instrumentation), then the same calls from cold with the expert
    kernels event-timed (identical decisions) for their rooflines; at T = 2048
    the one run is event-timed (its steps take seconds, the events microseconds)."""
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["fp8"]
    E, k, d, f, S = cfg.E, cfg.k, cfg.d, cfg.f, cfg.S
    t = time.time()
    bank = PinnedBank(E * S)
    synth.bank(cfg, out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
    log(f"fp8 bank {E * S / 1e9:.1f} GB in {time.time() - t:.1f}s")
    stream = torch.cuda.current_stream().cuda_stream
    res = {"workload": f"block-FP8 layer d={d}, E={E}, top-{k}, f={f}, CACHED, {cfg.slots} slots cold per T, "
                       f"Zipf(1.1) routes, B_P/B_H {cfg.bp_mbps // 1000}/{cfg.bh_mbps // 1000} GB/s", "runs": {}}
    for T, steps in zip(cfg.tokens, cfg.steps):
        xs = torch.stack([torch.from_numpy(synth.tokens(cfg, T, 300 + s, T).view(np.int16))
                          for s in range(steps)]).cuda()
        zr = [synth.zipf_routes(cfg, T, s) for s in range(steps)]
        ids_all = torch.from_numpy(np.stack([z[0] for z in zr]).astype(np.int32)).cuda()
        w_all = torch.from_numpy(np.stack([z[1] for z in zr])).cuda()
        work = torch.empty((T, k), dtype=torch.int32, device="cuda")
        y = torch.empty((T, d), dtype=torch.int16, device="cuda")

        def run(timed):
            sc = SlotCache(1, E, k, d, f, "fp8", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
            M.ft_cache_set_timing(sc.handle, timed)
            torch.cuda.synchronize()
            a = M.ft_cache_stats(sc.handle).as_dict()
            t0 = time.perf_counter()
            for s in range(steps):
                work.copy_(ids_all[s])
                M.ft_cache_classify(sc.handle, 0, work.data_ptr(), T, None, stream)
                M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xs[s].data_ptr(), work.data_ptr(),
                                 w_all[s].data_ptr(), T, y.data_ptr(), stream)
                if T >= 2048:
                    torch.cuda.synchronize()
                    log(f"fp8 T={T}: step {s + 1} of {steps} ({time.perf_counter() - t0:.1f}s)")
            torch.cuda.synchronize()
            el = time.perf_counter() - t0
            b = M.ft_cache_stats(sc.handle).as_dict()
            assert b["error_flags"] == 0, b
            tm = M.ft_cache_timing(sc.handle) if timed else None
            sc.close()
            return el, _stats_delta(a, b), tm

        if T >= 2048:
            el, dl, tm = run(True)
        else:
            el, dl, _ = run(False)
            _, _, tm = run(True)
        r = {"T": T, "steps": steps, "tokens_per_s": T * steps / el, "seconds": el,
             "miss_rate": dl["misses"] / max(dl["unique"], 1), "per_call": {key: v / steps for key, v in dl.items()},
             "host_gbs": dl["host_bytes"] / max(dl["host_seconds"], 1e-12) / 1e9,
             "event_timed_run": T >= 2048, **_kernel_figures(M, tm, "fp8", d, f, steps)}
        if dl["bytes_filled"] and tm.ms[M.FT_K_FILL]:
            r["fill_gbs"] = dl["bytes_filled"] / (tm.ms[M.FT_K_FILL] / 1e3) / 1e9
        res["runs"][f"T{T}"] = r
        log(f"fp8 T={T}: {r['tokens_per_s']:.1f} tok/s over {steps} steps ({el:.2f}s), miss rate "
            f"{r['miss_rate']:.2f}, host experts {r['per_call']['cpu_experts']:.1f}/call at {r['host_gbs']:.1f} GB/s" +
            (f", GEMV pair {r['gemv']['pair_gbs']:.0f} GB/s" if "gemv" in r else "") +
            (f", GEMM {r['gemm']['tflops']:.0f} TFLOP/s" if "gemm" in r else ""))
        del xs, ids_all, w_all
    bank.close()
    return res


def mxfp4_config_bench(args, phys_layers=8):
    """The MXFP4 configuration as configured: 61 layers (d=7168, E=256, top-8,
    f=2048, e2m1 + e8m0 per 32).  The 365 GB host bank cannot be pinned, so the
    layer banks alias: layer l reads physical layer l mod `phys_layers`
    (ft_cache_create_layers; flat ids, and every control decision, stay per
    layer).  Decode: 128 steps x 61 layers, one token per step, from a cold
    cache of 7,385 slots (60% of 288e9 bytes), B_P/B_H 20/60 GB/s, AR(1)
    hidden states, routing on the GPU; then the same steps from cold with the
    expert kernels event-timed.  Prefill: a 4,096-token chunk streamed through
    all 61 layers with the double buffer (2E slots), the grouped GEMM's MFMA
    utilisation measured with one layer resident."""
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["mxfp4"]
    L, E, k, d, f, S = cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.S
    LP = phys_layers
    t = time.time()
    bank = PinnedBank(LP * E * S)
    synth.bank(cfg.with_(layers=LP), out=bank.records(S), nthreads=min(16, len(os.sched_getaffinity(0))))
    ptrs = [bank.ptr + (l % LP) * E * S for l in range(L)]
    log(f"mxfp4 bank: {LP} physical layers, {LP * E * S / 1e9:.1f} GB pinned in {time.time() - t:.1f}s")
    stream = torch.cuda.current_stream().cuda_stream
    res = {"workload": f"MXFP4, {L} layers (banks of {LP} physical layers, aliased l mod {LP}), d={d}, E={E}, "
                       f"top-{k}, f={f}"}
    # ---- decode
    steps = cfg.steps[cfg.tokens.index(1)]
    xs = torch.stack([torch.from_numpy(synth.ar1_tokens(cfg, l, steps).view(np.int16)) for l in range(L)]).cuda()
    wr = torch.stack([torch.from_numpy(synth.router(cfg, l).view(np.int16)) for l in range(L)]).cuda()
    ids = torch.empty((L, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, k), dtype=torch.float32, device="cuda")
    y = torch.empty((L, d), dtype=torch.int16, device="cuda")

    def decode_run(timed):
        sc = SlotCache(L, E, k, d, f, "mxfp4", ptrs, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps)
        h, shp = sc.handle, sc.shape
        M.ft_cache_set_timing(h, timed)
        torch.cuda.synchronize()
        a = M.ft_cache_stats(h).as_dict()
        t0 = time.perf_counter()
        marks = []
        for s in range(steps):
            for l in range(L):
                xp = xs[l, s].data_ptr()
                M.ft_moe_route(shp, xp, wr[l].data_ptr(), 1, ids[l].data_ptr(), w[l].data_ptr(), stream)
                M.ft_cache_classify(h, l, ids[l].data_ptr(), 1, None, stream)
                M.ft_moe_forward(h, l, M.FT_MODE_CACHED, xp, ids[l].data_ptr(), w[l].data_ptr(), 1, y[l].data_ptr(),
                                 stream)
            if s + 1 in (steps // 2, steps):
                torch.cuda.synchronize()
                marks.append(time.perf_counter() - t0)
        b = M.ft_cache_stats(h).as_dict()
        assert b["error_flags"] == 0, b
        tm = M.ft_cache_timing(h) if timed else None
        sc.close()
        return marks, _stats_delta(a, b), tm

    marks, dl, _ = decode_run(False)
    _, _, tm = decode_run(True)
    calls = steps * L
    dec = {"steps": steps, "slots": cfg.slots, "tokens_per_s": steps / marks[-1], "seconds": marks[-1],
           "tokens_per_s_second_half": (steps - steps // 2) / (marks[1] - marks[0]),
           "miss_rate": dl["misses"] / max(dl["unique"], 1), "per_call": {key: v / calls for key, v in dl.items()},
           "host_gbs": dl["host_bytes"] / max(dl["host_seconds"], 1e-12) / 1e9,
           **_kernel_figures(M, tm, "mxfp4", d, f, calls)}
    if tm.ms[M.FT_K_FILL]:
        dec["fill_gbs"] = dl["bytes_filled"] / (tm.ms[M.FT_K_FILL] / 1e3) / 1e9
    res["decode"] = dec
    log(f"mxfp4 decode: {dec['tokens_per_s']:.1f} tok/s over {steps} steps from cold "
        f"({dec['tokens_per_s_second_half']:.1f} in the second half), miss rate {dec['miss_rate']:.2f}, GEMV pair "
        f"{dec['gemv']['pair_gbs']:.0f} GB/s ({dec['gemv']['pair_frac_hbm']:.1%})")
    del xs, wr
    # ---- prefill
    T = cfg.tokens[0]
    sc = SlotCache(L, E, k, d, f, "mxfp4", ptrs, 2 * E, T, cfg.bp_mbps, cfg.bh_mbps)
    h, shp = sc.handle, sc.shape
    x = torch.from_numpy(synth.tokens(cfg, T, 7).view(np.int16)).cuda()
    pids = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
    pw = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
    py = torch.empty((T, d), dtype=torch.int16, device="cuda")
    for l in range(L):
        wl = torch.from_numpy(synth.router(cfg, l).view(np.int16)).cuda()
        M.ft_moe_route(shp, x.data_ptr(), wl.data_ptr(), T, pids[l].data_ptr(), pw[l].data_ptr(), stream)
    torch.cuda.synchronize()

    def fwd(l, flags=M.FT_PREFETCH_NEXT):
        M.ft_moe_forward(h, l, M.FT_MODE_STREAMED | flags, x.data_ptr(), pids[l].data_ptr(), pw[l].data_ptr(), T,
                         py.data_ptr(), stream)

    fwd(0, 0)
    torch.cuda.synchronize()
    M.ft_cache_set_timing(h, True)
    reps = 5
    t0 = time.perf_counter()
    for _ in range(reps):
        fwd(0, 0)
    torch.cuda.synchronize()
    t_layer = (time.perf_counter() - t0) / reps
    tm = M.ft_cache_timing(h)
    M.ft_cache_set_timing(h, False)
    gem = _kernel_figures(M, tm, "mxfp4", d, f, reps)["gemm"]
    for l in range(L):          # untimed pass: the timed one then loads every layer
        fwd(l)
    torch.cuda.synchronize()
    loads0 = M.ft_cache_stats(h).layers_streamed
    t0 = time.perf_counter()
    for l in range(L):
        fwd(l)
        if l % 20 == 19:
            log(f"mxfp4 prefill stream: layer {l + 1} of {L} enqueued ({time.perf_counter() - t0:.1f}s)")
    torch.cuda.synchronize()
    t_stream = time.perf_counter() - t0
    stt = M.ft_cache_stats(h)
    assert stt.error_flags == 0
    loads = stt.layers_streamed - loads0
    res["prefill"] = {"T": T, "gemm": gem, "layer_ms_resident": t_layer * 1e3,
                      "stream": {"layers": L, "layer_loads": loads, "bytes": loads * E * S, "seconds": t_stream,
                                 "pcie_gbs": loads * E * S / t_stream / 1e9, "tokens_per_s": T / t_stream,
                                 "compute_only_s": L * t_layer, "gpu_busy_frac": L * t_layer / t_stream}}
    log(f"mxfp4 prefill: GEMM {gem['tflops']:.0f} TFLOP/s ({gem['frac_bf16_mfma']:.1%} of bf16 MFMA), stream "
        f"{res['prefill']['stream']['pcie_gbs']:.1f} GB/s over {L} layers, {T / t_stream:.0f} tok/s")
    sc.close()
    bank.close()
    return res


def tiny_config_bench(args, calls=8):
    """The tiny configuration: one layer (d=256, E=8, top-2, f=128, bf16), a
    4-slot cache from cold, B_P/B_H 25/50 GB/s; `calls` calls of 16 fresh
    tokens (route, classify, CACHED forward), timed after the same calls ran
    once untimed on a cache of their own: the median of five passes, each on
    a new cold cache."""
    import numpy as np
    import torch

    import moe_expert_execution_amd as M
    import synth
    from moe_expert_execution_amd.tensors import PinnedBank, SlotCache

    cfg = synth.CONFIGS["tiny"]
    T = cfg.tokens[0]
    bank = PinnedBank(cfg.E * cfg.S)
    synth.bank(cfg, out=bank.records(cfg.S))
    stream = torch.cuda.current_stream().cuda_stream
    xs = torch.stack([torch.from_numpy(synth.tokens(cfg, T, 0 if c == 0 else 100 + c).view(np.int16))
                      for c in range(calls)]).cuda()
    wr = torch.from_numpy(synth.router(cfg, 0).view(np.int16)).cuda()
    ids = torch.empty((T, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    y = torch.empty((T, cfg.d), dtype=torch.int16, device="cuda")

    def run(n):
        sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for c in range(n):
            M.ft_moe_route(sc.shape, xs[c].data_ptr(), wr.data_ptr(), T, ids.data_ptr(), w.data_ptr(), stream)
            M.ft_cache_classify(sc.handle, 0, ids.data_ptr(), T, None, stream)
            M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xs[c].data_ptr(), ids.data_ptr(), w.data_ptr(), T,
                             y.data_ptr(), stream)
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        st = M.ft_cache_stats(sc.handle)
        assert st.error_flags == 0
        sc.close()
        return el, st

    # untimed: the same calls on a cache of their own (the first launches of
    # this shape's kernels in the process cost several hundred microseconds);
    # then five timed passes, each on a new cold cache (the same decisions),
    # reported by their median: a pass is about half a millisecond of host
    # and GPU work, which a host core busy elsewhere for a moment stretches
    run(calls)
    passes = [run(calls) for _ in range(5)]
    els = sorted(p_[0] for p_ in passes)
    el, st = els[len(els) // 2], passes[0][1]
    bank.close()
    return {"workload": f"tiny layer d={cfg.d}, E={cfg.E}, top-{cfg.k}, f={cfg.f}, bf16, {cfg.slots} slots from "
                        f"cold, {calls} calls of {T} tokens (median of 5 passes)", "tokens_per_s": calls * T / el,
            "us_per_call": el / calls * 1e6, "us_per_call_passes": [e / calls * 1e6 for e in els],
            "fills": st.fills, "host_experts": st.cpu_experts, "hits": st.hits}


def oracle_subsets():
    """The oracle as it stands (route + slot-cache simulator + fp64 layer),
    timed on the host cores on a bounded subset of every configuration.  The
    record decodes of the oracle dominate its float layer (about 0.07 s per
    bf16 decode record, 0.5 s per block-FP8 record and 1 s per MXFP4 record
    on one core), so the float subsets are small; the control subsets are
    whole traces.  Each entry: what ran, seconds, tokens/s on exactly that."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import cache as OC, formats as OF, moe as OM, route as OR
    clk = time.perf_counter
    out = {"cores": len(os.sched_getaffinity(0)),
           "blas": [{key: p_.get(key) for key in ("internal_api", "num_threads")} for p_ in threadpool_info()
                    if p_.get("user_api") == "blas"]}

    def rec(name, what, tokens, seconds, **kw):
        out[name] = {"sample": what, "tokens": tokens, "seconds": seconds, "tokens_per_s": tokens / seconds, **kw}
        log(f"oracle {name}: {tokens / seconds:.4g} tok/s ({what}, {seconds:.1f}s)")

    def decoder(recs, cfg, layer, phys=None):
        lp = layer if phys is None else layer % phys
        return lambda e: OF.decode_record(recs[lp * cfg.E + e], cfg.fmt, cfg.d, cfg.f)

    # tiny: all 8 calls
    cfg = synth.CONFIGS["tiny"]
    recs = synth.bank(cfg)
    wr = synth.router(cfg, 0)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    t0 = clk()
    for c in range(8):
        x = synth.tokens(cfg, 16, 0 if c == 0 else 100 + c)
        ids, w, _ = OR.route(x, wr, cfg.k)
        sim.classify(0, ids)
        OM.moe_layer(x, ids, w, decoder(recs, cfg, 0))
    rec("tiny", "8 calls of 16 tokens (route + simulator + layer)", 128, clk() - t0)
    # decode: control over the whole trace; the float layer on 2 steps x 48 layers
    cfg = synth.CONFIGS["decode"]
    L, steps = cfg.layers, cfg.steps[0]
    xs = [synth.ar1_tokens(cfg, l, steps) for l in range(L)]
    wrs = [synth.router(cfg, l) for l in range(L)]
    sim = OC.SlotCacheSim(L, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    t0 = clk()
    for s in range(steps):
        for l in range(L):
            ids, w, _ = OR.route(xs[l][s:s + 1], wrs[l], cfg.k)
            sim.classify(l, ids)
    el = clk() - t0
    rec("decode_control", f"route + simulator, all {steps} steps x {L} layers", steps, el,
        us_per_call=el / (steps * L) * 1e6)
    recs = synth.bank(cfg, 0, 2 * cfg.E).reshape(2, cfg.E, -1)
    t0 = clk()
    for s in range(2):
        for l in range(L):
            ids, w, _ = OR.route(xs[l][s:s + 1], wrs[l], cfg.k)
            r_ = synth.bank(cfg, l * cfg.E, (l + 1) * cfg.E) if l >= 2 else recs[l]
            OM.moe_layer(xs[l][s:s + 1], ids, w, lambda e: OF.decode_record(r_[e], cfg.fmt, cfg.d, cfg.f))
    rec("decode_layer", f"route + fp64 layer, steps 0-1 x {L} layers (bank generation included)", 2, clk() - t0)
    # prefill: one layer of the 8,192-token chunk
    cfg = synth.CONFIGS["prefill"]
    T = cfg.tokens[0]
    x = synth.tokens(cfg, T, 7)
    recs = synth.bank(cfg, 0, cfg.E)
    t0 = clk()
    ids, w, _ = OR.route(x, synth.router(cfg, 0), cfg.k)
    OM.moe_layer(x, ids, w, decoder(recs, cfg, 0))
    rec("prefill_layer", f"one layer, T={T} (route + fp64 layer)", T, clk() - t0)
    # fp8: control over all three traces; the float layer on T=1 x 4 steps and T=64 x 1 step
    cfg = synth.CONFIGS["fp8"]
    t0 = clk()
    ntok = 0
    for T, steps in zip(cfg.tokens, cfg.steps):
        sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
        for s in range(steps):
            ids, _ = synth.zipf_routes(cfg, T, s)
            sim.classify(0, ids)
        ntok += T * steps
    rec("fp8_control", "simulator over the T=1/64/2048 traces (256/256/16 steps; Zipf draws included)", ntok,
        clk() - t0)
    recs = synth.bank(cfg)
    for T, n in ((1, 4), (64, 1)):
        t0 = clk()
        for s in range(n):
            x = synth.tokens(cfg, T, 300 + s, T)
            ids, w = synth.zipf_routes(cfg, T, s)
            OM.moe_layer(x, ids, w, decoder(recs, cfg, 0))
        rec(f"fp8_layer_T{T}", f"fp64 layer, T={T} x {n} step(s)", T * n, clk() - t0)
    del recs
    # mxfp4: control over the 128-step decode trace (7,385 slots); the float
    # layer on one decode step x 4 layers
    cfg = synth.CONFIGS["mxfp4"]
    L, steps = cfg.layers, cfg.steps[1]
    xs = [synth.ar1_tokens(cfg, l, steps) for l in range(L)]
    wrs = [synth.router(cfg, l) for l in range(L)]
    sim = OC.SlotCacheSim(L, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    t0 = clk()
    for s in range(steps):
        for l in range(L):
            ids, w, _ = OR.route(xs[l][s:s + 1], wrs[l], cfg.k)
            sim.classify(l, ids)
    el = clk() - t0
    rec("mxfp4_decode_control", f"route + simulator ({cfg.slots} slots), all {steps} steps x {L} layers", steps, el,
        us_per_call=el / (steps * L) * 1e6)
    recs = synth.bank(cfg, 0, 4 * cfg.E)
    t0 = clk()
    for l in range(4):
        ids, w, _ = OR.route(xs[l][:1], wrs[l], cfg.k)
        OM.moe_layer(xs[l][:1], ids, w, decoder(recs, cfg, l))
    el = clk() - t0
    rec("mxfp4_decode_layer", "route + fp64 layer, step 0 x layers 0-3", 4 / L, el, s_per_layer_call=el / 4)
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--cpu-sample-steps", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the decode run replayed from a HIP graph")
    ap.add_argument("--no-latency", action="store_true", help="skip the per-call latency run of the decode path")
    ap.add_argument("--hits-only-reps", type=int, default=32,
                    help="replays of the last decode step with fills off (hit-only GEMV bandwidth)")
    ap.add_argument("--no-measured-profile", action="store_true",
                    help="skip the second decode run with the measured B_P / B_H")
    ap.add_argument("--prefill-only", action="store_true", help="skip the decode part (kernel work)")
    ap.add_argument("--formats", action="store_true",
                    help="only run the block-FP8 and MXFP4 kernel measurements (one resident layer each)")
    ap.add_argument("--buffer-ablation", action="store_true",
                    help="only stream the prefill layers with two buffers and with one, at T = 4k, 8k, 16k")
    ap.add_argument("--miss-replay", action="store_true",
                    help="only replay routing traces through the placement policies (miss rate vs capacity)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (HBM counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the tiny, block-FP8 and MXFP4 configuration runs")
    ap.add_argument("--configs-only", action="store_true",
                    help="only the tiny, block-FP8 and MXFP4 configuration runs (one JSON line)")
    ap.add_argument("--oracle-subsets", action="store_true",
                    help="only time the oracle on bounded subsets of every configuration (host cores)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer and its slot cache run on a single device and this build has "
              f"no multi-GPU path, so --gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_expert_execution_amd as M
    M.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.oracle_subsets:
        print(json.dumps({"oracle_subsets": oracle_subsets()}), flush=True)
        return

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n}))
        return

    if args.formats:
        print(json.dumps({"formats": formats_bench(args)}), flush=True)
        return
    if args.miss_replay:
        print(json.dumps({"miss_replay": miss_replay_bench()}), flush=True)
        return
    if args.buffer_ablation:
        print(json.dumps({"buffer_ablation": buffer_ablation_bench()}), flush=True)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_bench(args)}), flush=True)
        return
    if args.configs_only:
        print(json.dumps({"configs": {"tiny": tiny_config_bench(args), "fp8": fp8_config_bench(args),
                                      "mxfp4": mxfp4_config_bench(args)}}), flush=True)
        return
    dec, bank, cfg = decode_bench(args)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(bank, cfg, args.cpu_sample_steps)
        log(f"cpu oracle: {cpu['value']:.4f} tok/s over {cpu['seconds']:.1f}s on {cpu['cores']} cores")
    bank.close()
    pre = None if args.no_prefill else prefill_bench(args)
    configs = None
    if not args.no_configs:
        configs = {"tiny": tiny_config_bench(args), "fp8": fp8_config_bench(args), "mxfp4": mxfp4_config_bench(args)}

    line = {
        "metric": "MoE-layer tokens/s: decode HBM GB/s %peak; prefill MFMA %peak",
        "value": dec["value"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode: 48 MoE layers, d=2048, E=128, top-8, ffn=768, bf16, 1 token/step, "
                               "1024 of 6144 layer-experts cached (cold start), B_P/B_H 20/60 GB/s, AR(1) hidden "
                               "states", "global_batch": 1, "seq_len": args.warmup + args.steps,
                   "parallelism": "single GPU"},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "decode_kernels": dec["decode_kernels"],
        "cache": dec["cache"],
        "kernel_timed_run_ms_per_step": dec["ms_per_step_kernel_timed_run"],
        "branches": dec["branches"],
        "measured_profile": dec.get("measured_profile"),
        "graph": dec.get("graph"),
        "latency_us": dec.get("latency_us"),
        "prefill": pre,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
