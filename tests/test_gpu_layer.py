"""GPU parity of the float layer (routing -> control -> GPU experts + host
experts -> combine) against the oracle, on the shapes of the decode, prefill,
block-FP8 and MXFP4 configurations: every output row, at the full token
counts too (the oracle runs expert by expert, one record decode per expert).
Bar: max |y - y_ref| <= 2e-2 max |y_ref| (bf16 weights) and <= 5e-2
max |y_ref| (FP8, MXFP4), outputs accumulated in fp32."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import cache as OC, route as OR

from gpu_util import (assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, expert_fn, gpu, make_bank,
                      oracle_layer_all_rows, oracle_rows, record_decoder)

TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp4": 5e-2}


def run_cached(sc, layer, x, ids, w):
    T = x.shape[0]
    st = torch.cuda.current_stream().cuda_stream
    xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w.astype(np.float32))
    y = torch.zeros((T, x.shape[1]), dtype=torch.int16, device="cuda")
    M.ft_cache_classify(sc.handle, layer, idd.data_ptr(), T, None, st)
    M.ft_moe_forward(sc.handle, layer, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), T,
                     y.data_ptr(), st)
    torch.cuda.synchronize()
    return bf16_bits_to_f64(y), idd.cpu().numpy()


@gpu
def test_decode_gemv_bf16():
    """Decode shape (d=2048, E=128, top-8, f=768, bf16) over 2 layers with 64
    slots: T = 1..4 tokens (GEMV path), hits, fills and host experts mixed."""
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=2, slots=64)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 4, cfg.bp_mbps,
                   cfg.bh_mbps)
    sim = OC.SlotCacheSim(cfg.layers, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    try:
        exs = [expert_fn(recs, cfg, l, maxsize=40) for l in range(cfg.layers)]
        xs = [synth.ar1_tokens(cfg, l, 16) for l in range(cfg.layers)]
        classes = set()
        for step in range(6):
            for l in range(cfg.layers):
                T = 1 + (step % 4)
                x = xs[l][step:step + T] if T == 1 else synth.tokens(cfg, T, 50 + step, l)
                ids, w, _ = OR.route(x, synth.router(cfg, l), cfg.k)
                r = sim.classify(l, ids)
                classes |= set(r.cls)
                y, routes = run_cached(sc, l, x, ids, w)
                assert np.array_equal(routes, r.routes)
                assert_close_rel(y, oracle_rows(x, ids, w, exs[l], range(T)), TOL["bf16"], f"step {step} layer {l}")
        assert classes == {OC.HIT, OC.FILL, OC.CPU}
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
def test_prefill_streamed_bf16():
    """Prefill shape (d=2048, E=128, top-8, f=768): two layers through the
    full-layer double buffer with prefetch, T = 8192, then ragged T = 300 and
    T = 100; every row of every call against the oracle."""
    cuda()
    cfg = synth.CONFIGS["prefill"].with_(layers=2, slots=256)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 8192, cfg.bp_mbps,
                   cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        for T in (8192, 300, 100):
            x = synth.tokens(cfg, T, 7, T)
            xd = dev_u16(x)
            for l in range(cfg.layers):
                ids, w, _ = OR.route(x, synth.router(cfg, l), cfg.k)
                idd, wd = dev(ids.astype(np.int32)), dev(w)
                y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
                M.ft_moe_forward(sc.handle, l, M.FT_MODE_STREAMED | M.FT_PREFETCH_NEXT, xd.data_ptr(),
                                 idd.data_ptr(), wd.data_ptr(), T, y.data_ptr(), st)
                torch.cuda.synchronize()
                ref = oracle_layer_all_rows(x, ids, w, record_decoder(recs, cfg, l))
                assert_close_rel(bf16_bits_to_f64(y), ref, TOL["bf16"], f"T {T} layer {l}")
        s = M.ft_cache_stats(sc.handle)
        assert s.error_flags == 0 and s.layers_streamed >= 2
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_streamed_one_token(fmt):
    """One-token calls in STREAMED mode run the one-launch decode kernel over
    the full-layer buffer (slot = buffer base + expert id): three layers, so
    both buffers, with and without prefetch; every output against the oracle,
    and the last call's kernel timing shows one expert launch and no down
    launch."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=512, f=256, E=8, k=2, layers=3, slots=16, cfg_id=97)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 4, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        for l in range(cfg.layers):
            ex = expert_fn(recs, cfg, l, maxsize=cfg.E)
            wr = synth.router(cfg, l)
            for t in range(3):
                x = synth.tokens(cfg, 1, 900 + 10 * l + t)
                ids, w, _ = OR.route(x, wr, cfg.k)
                xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w.astype(np.float32))
                y = torch.zeros((1, cfg.d), dtype=torch.int16, device="cuda")
                last = l == cfg.layers - 1 and t == 2
                if last:
                    M.ft_cache_set_timing(sc.handle, True)
                flags = M.FT_PREFETCH_NEXT if t == 2 else 0
                M.ft_moe_forward(sc.handle, l, M.FT_MODE_STREAMED | flags, xd.data_ptr(), idd.data_ptr(),
                                 wd.data_ptr(), 1, y.data_ptr(), st)
                torch.cuda.synchronize()
                assert_close_rel(bf16_bits_to_f64(y), oracle_rows(x, ids, w, ex, np.arange(1)), TOL[fmt],
                                 f"{fmt} layer {l} token {t}")
        tm = M.ft_cache_timing(sc.handle)
        assert tm.launches[M.FT_K_GEMV_GU] == 1 and tm.launches[M.FT_K_GEMV_DOWN] == 0
        s = M.ft_cache_stats(sc.handle)
        assert s.error_flags == 0 and s.layers_streamed >= cfg.layers
    finally:
        sc.close()
        bank.close()


@gpu
def test_prefill_streamed_single_buffer():
    """The one-buffer ablation: three layers through buffer 0 alone on a cache
    of exactly E slots (T = 300, every row against the oracle); the double
    buffer is refused on that cache, and flags are refused in CACHED mode."""
    cuda()
    cfg = synth.CONFIGS["prefill"].with_(layers=3, slots=128)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.E, 300, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        T = 300
        x = synth.tokens(cfg, T, 9, T)
        xd = dev_u16(x)
        y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
        ids0, w0, _ = OR.route(x, synth.router(cfg, 0), cfg.k)
        i0, w0d = dev(ids0.astype(np.int32)), dev(w0)
        lib = M.lib()
        assert lib.ft_moe_forward(sc.handle, 0, M.FT_MODE_STREAMED, xd.data_ptr(), i0.data_ptr(), w0d.data_ptr(), T,
                                  y.data_ptr(), st) == M.FT_ERR_STATE
        assert lib.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED | M.FT_SINGLE_BUFFER, xd.data_ptr(), i0.data_ptr(),
                                  w0d.data_ptr(), T, y.data_ptr(), st) == M.FT_ERR_ARG
        for l in range(cfg.layers):
            ids, w, _ = OR.route(x, synth.router(cfg, l), cfg.k)
            idd, wd = dev(ids.astype(np.int32)), dev(w)
            M.ft_moe_forward(sc.handle, l, M.FT_MODE_STREAMED | M.FT_SINGLE_BUFFER | M.FT_PREFETCH_NEXT,
                             xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), T, y.data_ptr(), st)
            torch.cuda.synchronize()
            rows = np.arange(T)
            ref = oracle_rows(x, ids, w, expert_fn(recs, cfg, l, maxsize=130), rows)
            assert_close_rel(bf16_bits_to_f64(y), ref, TOL["bf16"], f"single buffer layer {l}")
        s = M.ft_cache_stats(sc.handle)
        assert s.error_flags == 0 and s.layers_streamed == cfg.layers
    finally:
        sc.close()
        bank.close()


@gpu
def test_mxfp4_prefill_streamed_T4096():
    """MXFP4 prefill at its full chunk (d=7168, E=256, top-8, f=2048, T=4096):
    the layer in a full-layer buffer, the grouped MFMA GEMM as bench.py times
    it, every row against the oracle."""
    cuda()
    cfg = synth.CONFIGS["mxfp4"].with_(layers=1)
    T = 4096
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "mxfp4", bank.ptr, 2 * cfg.E, T, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        x = synth.tokens(cfg, T, 7, T)
        ids, w, _ = OR.route(x, synth.router(cfg, 0), cfg.k)
        xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
        y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
        M.ft_moe_forward(sc.handle, 0, M.FT_MODE_STREAMED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), T,
                         y.data_ptr(), st)
        torch.cuda.synchronize()
        ref = oracle_layer_all_rows(x, ids, w, record_decoder(recs, cfg, 0))
        assert_close_rel(bf16_bits_to_f64(y), ref, TOL["mxfp4"], "mxfp4 T 4096")
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("T,steps", [(1, 4), (16, 2)])
def test_mxfp4_cached(T, steps):
    """MXFP4 shape (d=7168, E=256, top-8, f=2048, e2m1 + e8m0 per 32), one
    layer, 64 slots: GEMV (T=1) and MFMA (T=16) paths, every row."""
    cuda()
    cfg = synth.CONFIGS["mxfp4"].with_(layers=1, slots=64)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "mxfp4", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
    try:
        dec = record_decoder(recs, cfg, 0)
        wr = synth.router(cfg, 0)
        for step in range(steps):
            x = synth.tokens(cfg, T, 400 + step, T)
            ids, w, _ = OR.route(x, wr, cfg.k)
            y, _ = run_cached(sc, 0, x, ids, w)
            assert_close_rel(y, oracle_layer_all_rows(x, ids, w, dec), TOL["mxfp4"], f"T {T} step {step}")
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("d,f", [(32768, 128), (128, 8192)])
def test_layer_at_the_size_limits(fmt, d, f):
    """The largest d (32768) and f (8192) the library accepts, every format:
    T = 1 and 4 (GEMV: eight K-parts at d = 32768, 64 KiB of h in LDS at
    f = 8192) and T = 37 (MFMA GEMM with a ragged last tile); all rows
    against the oracle, every expert resident after its fill."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(d=d, f=f, E=4, k=2, fmt=fmt, slots=4, bp_mbps=60000, bh_mbps=60000,
                                      cfg_id=95)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 37, cfg.bp_mbps, cfg.bh_mbps)
    try:
        ex = expert_fn(recs, cfg, 0, maxsize=4)
        wr = synth.router(cfg, 0)
        for T in (1, 4, 37):
            x = synth.tokens(cfg, T, 500 + T)
            ids, w, _ = OR.route(x, wr, cfg.k)
            y, _ = run_cached(sc, 0, x, ids, w)
            assert_close_rel(y, oracle_rows(x, ids, w, ex, np.arange(T)), TOL[fmt], f"{fmt} d {d} f {f} T {T}")
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
@pytest.mark.parametrize("d", [8192, 8320])
def test_one_token_width_boundary(fmt, d):
    """d = 8,192 is the widest token the one-launch decode kernel stages in
    LDS; d = 8,320 takes the two-launch GEMV.  CACHED one-token calls with
    hits, fills and host experts, every output against the oracle; the last
    call's kernel timing shows which path ran (one expert launch and no down
    launch, or a gate/up launch and the down side's)."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=d, f=256, E=8, k=2, slots=4, cfg_id=98)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    try:
        ex = expert_fn(recs, cfg, 0, maxsize=cfg.E)
        wr = synth.router(cfg, 0)
        classes = set()
        for t in range(8):
            x = synth.tokens(cfg, 1, 700 + t)
            ids, w, _ = OR.route(x, wr, cfg.k)
            r = sim.classify(0, ids)
            classes |= set(r.cls)
            if t == 7:
                M.ft_cache_set_timing(sc.handle, True)
            y, routes = run_cached(sc, 0, x, ids, w)
            assert np.array_equal(routes, r.routes)
            assert_close_rel(y, oracle_rows(x, ids, w, ex, np.arange(1)), TOL[fmt], f"{fmt} d {d} token {t}")
        assert classes == {OC.HIT, OC.FILL, OC.CPU}, classes
        tm = M.ft_cache_timing(sc.handle)
        if d <= 8192:
            assert tm.launches[M.FT_K_GEMV_GU] == 1 and tm.launches[M.FT_K_GEMV_DOWN] == 0
        else:   # with its K split in parts, the down side is a SwiGLU launch and the down launch
            assert tm.launches[M.FT_K_GEMV_GU] == 1 and tm.launches[M.FT_K_GEMV_DOWN] >= 1
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_host_token_counts(fmt):
    """One CACHED call whose eight experts all run on the host (max_fetch 0,
    cold cache) with 1, 2, 3, 4, 7, 8, 9 and 16 tokens each: the host
    branch's one-token, streaming and decode-once forms side by side in its
    pooled phases (the streaming form takes up to 8 tokens for bf16 and
    block-FP8, up to 3 for MXFP4), d = 2,304 so the many-token dots end in a
    ragged column slice.  Routes as classify rewrote them against the
    simulator, every output row against the oracle; then the same call again."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=2304, f=256, E=16, k=2, slots=4, cfg_id=100)
    counts = (1, 2, 3, 4, 7, 8, 9, 16)
    col = np.repeat(np.arange(len(counts)) * 2 + 1, counts)          # experts 1, 3, ..., 15
    T = col.size // 2
    ids = np.stack([col[:T], col[T:]], axis=1).astype(np.int32)      # 16 < T: a token's two experts differ
    assert np.all(ids[:, 0] != ids[:, 1])
    w = np.random.default_rng(100).uniform(0.2, 1.0, size=ids.shape).astype(np.float32)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps, 0)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps, 0)
    try:
        ex = expert_fn(recs, cfg, 0, maxsize=cfg.E)
        for call in range(2):
            x = synth.tokens(cfg, T, 800 + call)
            r = sim.classify(0, ids)
            assert set(r.cls) == {OC.CPU}, r.cls
            before = M.ft_cache_stats(sc.handle).as_dict()
            y, routes = run_cached(sc, 0, x, ids, w)
            after = M.ft_cache_stats(sc.handle).as_dict()
            assert np.array_equal(routes, r.routes)
            assert after["cpu_experts"] - before["cpu_experts"] == len(counts)
            assert_close_rel(y, oracle_rows(x, ids, w, ex, np.arange(T)), TOL[fmt], f"{fmt} call {call}")
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_top16_layer(fmt):
    """The largest top-k (16): E = 32 over 24 slots, so calls mix hits, fills
    and host experts; T = 1 (one-launch decode kernel and its combine),
    T = 3 (GEMV), T = 40 (grouped GEMM).  Routes as classify rewrote them
    against the simulator, every output row against the oracle."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(fmt=fmt, d=256, f=256, E=32, k=16, slots=24, cfg_id=99)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 40, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    try:
        ex = expert_fn(recs, cfg, 0, maxsize=cfg.E)
        wr = synth.router(cfg, 0)
        classes = set()
        for i, T in enumerate((1, 1, 3, 40, 1, 3, 40, 1)):
            x = synth.tokens(cfg, T, 600 + i)
            ids, w, _ = OR.route(x, wr, cfg.k)
            r = sim.classify(0, ids)
            classes |= set(r.cls)
            y, routes = run_cached(sc, 0, x, ids, w)
            assert np.array_equal(routes, r.routes)
            assert_close_rel(y, oracle_rows(x, ids, w, ex, np.arange(T)), TOL[fmt], f"{fmt} call {i} T {T}")
        assert classes == {OC.HIT, OC.FILL, OC.CPU}, classes
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("T,k", [(128, 8), (129, 8), (6, 1), (300, 1)])
def test_planner_boundary_and_top1(T, k):
    """T * k = 1,024 routes is the largest call of the one-workgroup planner
    (which rides in the fill's launch); 1,032 takes the chunked planner and
    a separate fill.  Top-1 routing on both sides of the GEMV/GEMM switch.
    Decode shape, 64 slots, every class mixed; all rows against the oracle."""
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=1, slots=64, k=k)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
    try:
        ex = expert_fn(recs, cfg, 0, maxsize=cfg.E)
        wr = synth.router(cfg, 0)
        for s in range(2):
            x = synth.tokens(cfg, T, 800 + s)
            ids, w, _ = OR.route(x, wr, cfg.k)
            y, routes = run_cached(sc, 0, x, ids, w)
            assert (routes < 0).any() or s > 0
            assert_close_rel(y, oracle_rows(x, ids, w, ex, np.arange(T)), TOL["bf16"], f"T {T} k {k} call {s}")
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()
