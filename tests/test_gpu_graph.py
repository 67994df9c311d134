"""Decode layer steps captured into a HIP graph: replaying the graph gives,
step for step, exactly the eager result (routes, layer outputs, cache maps,
stamps and counters), with eager work and synchronisations between replays,
and the layer outputs match the oracle.  A call that cannot be captured is
refused with the documented status."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import moe as OM

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, expert_fn, gpu, make_bank


def _setup(cfg, steps, T=1):
    """Per layer: `steps` calls of T tokens (T = 1: the AR(1) decode stream)."""
    L = cfg.layers
    if T == 1:
        xs = torch.stack([torch.from_numpy(synth.ar1_tokens(cfg, l, steps).view(np.int16)) for l in range(L)])
        xs = xs[:, :, None, :]
    else:
        xs = torch.stack([torch.stack([torch.from_numpy(synth.tokens(cfg, T, 60 + s, l).view(np.int16))
                                       for s in range(steps)]) for l in range(L)])
    wr = torch.stack([torch.from_numpy(synth.router(cfg, l).view(np.int16)) for l in range(L)]).cuda()
    return xs.cuda(), wr


class Step:
    """Fixed buffers of one step: T tokens through every layer."""

    def __init__(self, cfg, sc, wr, T=1):
        L, k, d = cfg.layers, cfg.k, cfg.d
        self.cfg, self.sc, self.wr, self.T = cfg, sc, wr, T
        self.x = torch.zeros((L, T, d), dtype=torch.int16, device="cuda")
        self.ids = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
        self.routes = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
        self.w = torch.zeros((L, T, k), dtype=torch.float32, device="cuda")
        self.y = torch.zeros((L, T, d), dtype=torch.int16, device="cuda")

    def enqueue(self):
        h, shp, T = self.sc.handle, self.sc.shape, self.T
        st = torch.cuda.current_stream().cuda_stream
        for l in range(self.cfg.layers):
            M.ft_moe_route(shp, self.x[l].data_ptr(), self.wr[l].data_ptr(), T, self.ids[l].data_ptr(),
                           self.w[l].data_ptr(), st)
            self.routes[l].copy_(self.ids[l])
            M.ft_cache_classify(h, l, self.routes[l].data_ptr(), T, None, st)
            M.ft_moe_forward(h, l, M.FT_MODE_CACHED, self.x[l].data_ptr(), self.routes[l].data_ptr(),
                             self.w[l].data_ptr(), T, self.y[l].data_ptr(), st)


@gpu
@pytest.mark.parametrize("signal,fmt,T", [("mailbox", "bf16", 1), ("callback", "bf16", 1), ("mailbox", "fp8", 1),
                                          ("mailbox", "mxfp4", 1), ("mailbox", "bf16", 3), ("mailbox", "bf16", 8)])
def test_graph_replay_equals_eager_step_for_step(signal, fmt, T, monkeypatch):
    """`mailbox`: the captured calls post to the polling host thread with
    device-drawn numbers; `callback`: stream host functions, captured as host
    nodes (FTMOE_HOST_SIGNAL is read when a cache is created).  Every weight
    format with the mailbox; calls of 3 tokens (the 4-row GEMV) and of 8
    (the grouped GEMM)."""
    cuda()
    if signal == "callback":
        monkeypatch.setenv("FTMOE_HOST_SIGNAL", "callback")
    # a small cache under pressure: hits, fills and host-run misses every step
    # (calls of several tokens touch most of a layer's experts: more slots)
    cfg = synth.CONFIGS["decode"].with_(layers=4, d=256, E=16, k=4, f=128, slots=12 if T == 1 else 40,
                                        bp_mbps=20000, bh_mbps=60000, fmt=fmt)
    steps = 12
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    xs, wr = _setup(cfg, steps, T)
    mk = lambda: SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, T, cfg.bp_mbps,
                           cfg.bh_mbps)
    a, b = mk(), mk()
    try:
        ea, gb = Step(cfg, a, wr, T), Step(cfg, b, wr, T)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            gb.enqueue()                  # captured, not run
        torch.cuda.synchronize()
        n_ids = cfg.layers * cfg.E
        for s in range(steps):
            ea.x.copy_(xs[:, s])
            ea.enqueue()                  # eager
            gb.x.copy_(xs[:, s])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ea.ids, gb.ids) and torch.equal(ea.routes, gb.routes), f"step {s}"
            assert torch.equal(ea.y, gb.y), f"layer outputs differ at step {s}"
            sa = M.ft_cache_snapshot(a.handle, n_ids, cfg.slots)
            sb = M.ft_cache_snapshot(b.handle, n_ids, cfg.slots)
            for u, v in zip(sa[:3], sb[:3]):
                assert np.array_equal(u, v), f"cache state differs at step {s}"
            assert sa[3] == sb[3]
            if s in (0, steps - 1):
                x = xs[:, s].cpu().numpy().view(np.uint16)
                ids = ea.ids.cpu().numpy()
                w = ea.w.cpu().numpy()
                for l in range(cfg.layers):
                    ref = OM.moe_layer(x[l], ids[l], w[l], expert_fn(recs, cfg, l))
                    assert_close_rel(bf16_bits_to_f64(gb.y[l]), ref, 2e-2 if fmt == "bf16" else 5e-2,
                                     f"graph step {s} layer {l}")
        ca, cb = M.ft_cache_stats(a.handle), M.ft_cache_stats(b.handle)
        for key in ("calls", "unique", "hits", "misses", "fills", "cpu_experts", "evictions", "host_experts"):
            assert getattr(ca, key) == getattr(cb, key), key
        assert cb.fills > 0 and cb.cpu_experts > 0 and cb.hits > 0 and cb.error_flags == 0
    finally:
        a.close()
        b.close()
        bank.close()


@gpu
def test_uncapturable_calls_are_refused():
    cuda()
    cfg = synth.CONFIGS["prefill"].with_(layers=2, d=256, E=8, k=2, f=128, slots=16)
    bank = make_bank(cfg)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 4, cfg.bp_mbps,
                   cfg.bh_mbps)
    try:
        x = torch.zeros((4, cfg.d), dtype=torch.int16, device="cuda")
        ids = torch.zeros((4, cfg.k), dtype=torch.int32, device="cuda")
        ids[:, 1] = 1
        w = torch.full((4, cfg.k), 0.5, dtype=torch.float32, device="cuda")
        y = torch.zeros((4, cfg.d), dtype=torch.int16, device="cuda")
        lib = M.lib()
        h = sc.handle

        def capture(mode):
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st = torch.cuda.current_stream().cuda_stream
                r = lib.ft_moe_forward(h, 0, mode, x.data_ptr(), ids.data_ptr(), w.data_ptr(), 4, y.data_ptr(), st)
                y.add_(0)
            torch.cuda.synchronize()
            return r

        assert capture(M.FT_MODE_STREAMED) == M.FT_ERR_UNSUPPORTED, M.ft_last_error()
        M.ft_cache_set_timing(h, True)
        assert capture(M.FT_MODE_CACHED) == M.FT_ERR_STATE, M.ft_last_error()
        M.ft_cache_set_timing(h, False)
    finally:
        torch.cuda.synchronize()
        sc.close()
        bank.close()


@gpu
def test_graph_sees_new_profile_and_recapture_after_resize():
    """A replay uses the cache's profile at replay time: after
    ft_cache_set_profile (max_fetch 0, every miss to the host) the graph
    captured before it makes the eager cache's decisions and fills nothing.
    After ft_cache_resize the graph is captured again (the old one is void and
    is not replayed) and again equals the eager cache step for step, with
    outputs matching the oracle."""
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=4, d=256, E=16, k=4, f=128, slots=12, bp_mbps=20000, bh_mbps=60000)
    steps, T = 12, 1
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    xs, wr = _setup(cfg, steps, T)
    mk = lambda: SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, T, cfg.bp_mbps,
                           cfg.bh_mbps)
    a, b = mk(), mk()
    n_ids = cfg.layers * cfg.E

    def capture(step):
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step.enqueue()
        torch.cuda.synchronize()
        return g

    try:
        ea, gb = Step(cfg, a, wr, T), Step(cfg, b, wr, T)
        g = capture(gb)
        slots = cfg.slots
        for s in range(steps):
            if s == 4:
                for c in (a, b):
                    M.ft_cache_set_profile(c.handle, M.profile(cfg.bp_mbps, cfg.bh_mbps, 0))
                fills_before = M.ft_cache_stats(b.handle).fills
            if s == 8:
                assert M.ft_cache_stats(b.handle).fills == fills_before, "max_fetch 0 did not reach the replays"
                slots = 7
                for c in (a, b):
                    M.ft_cache_resize(c.handle, slots)
                    M.ft_cache_set_profile(c.handle, M.profile(cfg.bp_mbps, cfg.bh_mbps, -1))
                del g
                g = capture(gb)
            ea.x.copy_(xs[:, s])
            ea.enqueue()
            gb.x.copy_(xs[:, s])
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(ea.routes, gb.routes) and torch.equal(ea.y, gb.y), f"step {s}"
            sa = M.ft_cache_snapshot(a.handle, n_ids, slots)
            sb = M.ft_cache_snapshot(b.handle, n_ids, slots)
            for u, v in zip(sa[:3], sb[:3]):
                assert np.array_equal(u, v), f"cache state differs at step {s}"
            assert sa[3] == sb[3]
            if s in (5, steps - 1):
                x = xs[:, s].cpu().numpy().view(np.uint16)
                ids, w = ea.ids.cpu().numpy(), ea.w.cpu().numpy()
                for l in range(cfg.layers):
                    ref = OM.moe_layer(x[l], ids[l], w[l], expert_fn(recs, cfg, l))
                    assert_close_rel(bf16_bits_to_f64(gb.y[l]), ref, 2e-2, f"graph step {s} layer {l}")
        cb = M.ft_cache_stats(b.handle)
        assert cb.fills > fills_before and cb.error_flags == 0 and cb.num_slots == slots
    finally:
        a.close()
        b.close()
        bank.close()
