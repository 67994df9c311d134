"""GPU parity of the per-layer control step against the oracle's simulator:
unique sets, hit/fill/host classes, q, evictions, rewritten routes and the
maps, bit-exact, over whole routing traces of the decode, block-FP8 and MXFP4
configurations, plus edge cases and the hostile invalidation sequence.

Control decisions do not depend on d or f, so these traces run on caches whose
records are small (d = f = 128); the routing ids come from the full-size
routers and hidden states of each configuration."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import ClassifyBuffers, SlotCache
from oracle import cache as OC, moe as OM, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, expert_fn, gpu, make_bank

HIT, FILL, CPU = OC.HIT, OC.FILL, OC.CPU


class TraceRunner:
    """Runs many classify calls into per-call slices of big device buffers,
    then compares every call with the oracle simulator after one sync."""

    def __init__(self, cfg, calls_T, small=True):
        self.cfg = cfg
        self.small = cfg.with_(d=128, f=128, fmt="bf16") if small else cfg
        self.bank = make_bank(self.small)
        maxT = max(calls_T)
        self.sc = SlotCache(cfg.layers, cfg.E, cfg.k, self.small.d, self.small.f, self.small.fmt, self.bank.ptr,
                            cfg.slots, maxT, cfg.bp_mbps, cfg.bh_mbps, cfg.max_fetch)
        self.sim = OC.SlotCacheSim(cfg.layers, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps, cfg.max_fetch)
        n = len(calls_T)
        self.cap = maxT * cfg.k
        kw = dict(device="cuda")
        self.counts = torch.zeros((n, 4), dtype=torch.int32, **kw)
        self.arr = {name: torch.full((n, self.cap), -7, dtype=torch.int32, **kw)
                    for name in ("uniq", "slot", "ev_slot", "ev_old", "ev_new", "cpu_ids")}
        self.cls = torch.full((n, self.cap), 255, dtype=torch.uint8, **kw)
        self.ids = torch.full((n, self.cap), -7, dtype=torch.int32, **kw)
        self.n = 0
        self.results = []

    def out_struct(self, i):
        a = self.arr
        return M.FtClassifyOut(self.counts[i].data_ptr(), a["uniq"][i].data_ptr(), self.cls[i].data_ptr(),
                               a["slot"][i].data_ptr(), a["ev_slot"][i].data_ptr(), a["ev_old"][i].data_ptr(),
                               a["ev_new"][i].data_ptr(), a["cpu_ids"][i].data_ptr(), self.cap)

    def call(self, layer, ids_np):
        i = self.n
        T = ids_np.shape[0]
        R = T * self.cfg.k
        self.ids[i, :R] = torch.from_numpy(ids_np.reshape(-1).astype(np.int32)).cuda()
        out = self.out_struct(i)
        M.ft_cache_classify(self.sc.handle, layer, self.ids[i].data_ptr(), T, out,
                            torch.cuda.current_stream().cuda_stream)
        self.results.append((layer, T, self.sim.classify(layer, ids_np)))
        self.n += 1

    def check(self):
        torch.cuda.synchronize()
        counts = self.counts.cpu().numpy()
        arr = {k: v.cpu().numpy() for k, v in self.arr.items()}
        cls = self.cls.cpu().numpy()
        ids = self.ids.cpu().numpy()
        k = self.cfg.k
        hits = fills = cpu = 0
        for i, (layer, T, r) in enumerate(self.results):
            nu = len(r.uniq)
            where = f"call {i} (layer {layer}, T {T})"
            assert list(counts[i]) == [nu, r.hits, r.m, r.q], where
            assert arr["uniq"][i, :nu].tolist() == r.uniq, where
            assert cls[i, :nu].tolist() == r.cls, where
            assert arr["slot"][i, :nu].tolist() == r.slot, where
            assert arr["ev_slot"][i, :r.q].tolist() == [v for v, _, _ in r.evictions], where
            assert arr["ev_old"][i, :r.q].tolist() == [o for _, o, _ in r.evictions], where
            assert arr["ev_new"][i, :r.q].tolist() == [u for _, _, u in r.evictions], where
            assert arr["cpu_ids"][i, :r.m - r.q].tolist() == r.cpu, where
            assert np.array_equal(ids[i, :T * k], r.routes.reshape(-1)), where
            hits += r.hits
            fills += r.q
            cpu += r.m - r.q
        sfi, ios, stamp, clock = M.ft_cache_snapshot(self.sc.handle, self.cfg.layers * self.cfg.E, self.cfg.slots)
        osfi, oios, ostamp, oclock = self.sim.arrays()
        assert np.array_equal(sfi, osfi) and np.array_equal(ios, oios)
        assert np.array_equal(stamp, ostamp) and clock == oclock
        s = M.ft_cache_stats(self.sc.handle)
        assert (s.hits, s.fills, s.cpu_experts, s.error_flags) == (hits, fills, cpu, 0)
        return hits, fills, cpu

    def close(self):
        self.sc.close()
        self.bank.close()


def decode_ids(cfg, steps):
    """Routing ids of the decode trace: per-layer AR(1) hidden states through
    each layer's router (oracle routing), in call order (step, layer)."""
    per_layer = []
    for l in range(cfg.layers):
        x = synth.ar1_tokens(cfg, l, steps)
        ids, _, _ = OR.route(x, synth.router(cfg, l), cfg.k)
        per_layer.append(ids)
    return per_layer


@gpu
def test_decode_trace_full():
    """48 layers x 256 steps, 1 token per step, 1024 of 6144 layer-experts."""
    cuda()
    cfg = synth.CONFIGS["decode"]
    steps = cfg.steps[0]
    ids = decode_ids(cfg, steps)
    tr = TraceRunner(cfg, [1] * (steps * cfg.layers))
    try:
        for s in range(steps):
            for l in range(cfg.layers):
                tr.call(l, ids[l][s:s + 1])
        hits, fills, cpu = tr.check()
        assert hits > 0 and fills > 0 and cpu > 0
    finally:
        tr.close()


@gpu
def test_fp8_zipf_trace_T64():
    """Block-FP8 configuration's control trace: 256 steps of 64 tokens with
    Zipf(1.1) expert popularity, 64 slots."""
    cuda()
    cfg = synth.CONFIGS["fp8"]
    tr = TraceRunner(cfg, [64] * 256)
    try:
        for s in range(256):
            ids, _ = synth.zipf_routes(cfg, 64, s)
            tr.call(0, ids)
        tr.check()
    finally:
        tr.close()


@gpu
def test_mxfp4_decode_trace_7385_slots():
    """61 layers x 48 decode steps with 7,385 slots (60% of 288e9 bytes of
    MXFP4 records): the victim scan covers every slot."""
    cuda()
    cfg = synth.CONFIGS["mxfp4"].with_(slots=7385)
    steps = 48
    ids = decode_ids(cfg, steps)
    tr = TraceRunner(cfg, [1] * (steps * cfg.layers))
    try:
        for s in range(steps):
            for l in range(cfg.layers):
                tr.call(l, ids[l][s:s + 1])
        tr.check()
    finally:
        tr.close()


@gpu
@pytest.mark.parametrize("slots,bp,bh,mf", [(1, 20000, 60000, -1), (3, 60000, 20000, -1), (16, 20000, 60000, 0),
                                            (16, 20000, 60000, 2), (40, 11800, 47500, -1)])
def test_edge_profiles(slots, bp, bh, mf):
    """Thrash (1 slot), fewer slots than the active set, fetch caps, B_P > B_H."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(layers=3, E=16, k=4, slots=slots, bp_mbps=bp, bh_mbps=bh, max_fetch=mf)
    rng = np.random.default_rng(slots * 7 + mf)
    Ts = [int(rng.integers(1, 9)) for _ in range(60)]
    tr = TraceRunner(cfg, Ts, small=False)
    try:
        for T in Ts:
            ids = np.stack([rng.choice(cfg.E, size=cfg.k, replace=False) for _ in range(T)])
            tr.call(int(rng.integers(0, cfg.layers)), ids)
        tr.check()
    finally:
        tr.close()


@gpu
def test_out_of_range_ids_flagged():
    cuda()
    cfg = synth.CONFIGS["tiny"]
    bank = make_bank(cfg)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 4, cfg.bp_mbps, cfg.bh_mbps)
    try:
        ids = torch.tensor([[0, 1], [2, 99]], dtype=torch.int32, device="cuda")
        buf = ClassifyBuffers(8)
        M.ft_cache_classify(sc.handle, 0, ids.data_ptr(), 2, buf.struct, torch.cuda.current_stream().cuda_stream)
        got = buf.host()
        s = M.ft_cache_stats(sc.handle)
        assert s.error_flags & 1
        assert got["uniq"] == [0, 1, 2]
        assert ids.cpu().numpy()[1, 1] == M.ROUTE_INVALID
        with pytest.raises(M.FtError):
            M.ft_cache_classify(sc.handle, 1, ids.data_ptr(), 2, None, 0)      # layer out of range
        with pytest.raises(M.FtError):
            M.ft_cache_classify(sc.handle, 0, ids.data_ptr(), 5, None, 0)      # T > max_tokens
    finally:
        sc.close()
        bank.close()


@gpu
def test_empty_calls():
    """T = 0: routing enqueues nothing and writes nothing; classify and forward
    refuse it with FT_ERR_ARG and leave the cache as it was, so the next call
    behaves as if the refused ones had not been made."""
    cuda()
    cfg = synth.CONFIGS["tiny"]
    bank = make_bank(cfg)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 4, cfg.bp_mbps, cfg.bh_mbps)
    try:
        st = torch.cuda.current_stream().cuda_stream
        x = torch.zeros((1, cfg.d), dtype=torch.int16, device="cuda")
        wr = torch.zeros((cfg.d, cfg.E), dtype=torch.int16, device="cuda")
        ids = torch.full((1, cfg.k), -7, dtype=torch.int32, device="cuda")
        w = torch.full((1, cfg.k), -7.0, dtype=torch.float32, device="cuda")
        M.ft_moe_route(sc.shape, x.data_ptr(), wr.data_ptr(), 0, ids.data_ptr(), w.data_ptr(), st)
        torch.cuda.synchronize()
        assert (ids.cpu() == -7).all() and (w.cpu() == -7.0).all()
        before = M.ft_cache_stats(sc.handle).as_dict()
        with pytest.raises(M.FtError) as ei:
            M.ft_cache_classify(sc.handle, 0, ids.data_ptr(), 0, None, st)
        assert ei.value.status == M.FT_ERR_ARG
        with pytest.raises(M.FtError) as ei:
            M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, x.data_ptr(), ids.data_ptr(), w.data_ptr(), 0,
                             x.data_ptr(), st)
        assert ei.value.status == M.FT_ERR_ARG
        torch.cuda.synchronize()
        assert M.ft_cache_stats(sc.handle).as_dict() == before
        # the next call is the first one the cache sees: every expert misses
        ids = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
        buf = ClassifyBuffers(8)
        M.ft_cache_classify(sc.handle, 0, ids.data_ptr(), 1, buf.struct, st)
        got = buf.host()
        r = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps).classify(0, np.array([[0, 1]], np.int32))
        assert got["uniq"] == list(r.uniq) and got["cls"] == list(r.cls) and got["q"] == r.q and got["hits"] == 0
        assert got["slot"] == list(r.slot)
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
def test_streamed_needs_two_buffers():
    cuda()
    cfg = synth.CONFIGS["tiny"]
    bank = make_bank(cfg)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 4, cfg.bp_mbps, cfg.bh_mbps)
    try:
        x = torch.zeros((1, cfg.d), dtype=torch.int16, device="cuda")
        ids = torch.zeros((1, cfg.k), dtype=torch.int32, device="cuda")
        w = torch.zeros((1, cfg.k), dtype=torch.float32, device="cuda")
        with pytest.raises(M.FtError) as ei:
            M.ft_moe_forward(sc.handle, 0, M.FT_MODE_STREAMED, x.data_ptr(), ids.data_ptr(), w.data_ptr(), 1,
                             x.data_ptr(), 0)
        assert ei.value.status == M.FT_ERR_STATE
    finally:
        sc.close()
        bank.close()


@gpu
def test_hostile_invalidation_sequence_gpu():
    """Request A uses layer-0 experts; request B streams layers 1 and 2 through
    both full-layer buffers (every slot); A routes back and must miss, re-fill
    from layer 0's bank and produce layer 0's output ("The Expert Cache That
    Follows the Router", hostile-sequence paragraph)."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(layers=3, E=4, k=2, slots=8, bp_mbps=60000, bh_mbps=60000)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 16, cfg.bp_mbps,
                   cfg.bh_mbps)
    sim = OC.SlotCacheSim(cfg.layers, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        x = synth.tokens(cfg, 2, 0)
        ids = np.array([[0, 1], [2, 3]], dtype=np.int32)
        w = np.array([[0.5, 0.5], [0.25, 0.75]], np.float32)
        xd, wd = dev_u16(x), dev(w)
        ref0 = OM.moe_layer(x, ids, w, expert_fn(recs, cfg, 0))

        def decode_call():
            idd = dev(ids)
            y = torch.zeros((2, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_cache_classify(sc.handle, 0, idd.data_ptr(), 2, None, st)
            M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), 2,
                             y.data_ptr(), st)
            r = sim.classify(0, ids)
            torch.cuda.synchronize()
            return r, bf16_bits_to_f64(y)

        r, y = decode_call()
        assert_close_rel(y, ref0, 2e-2, "first decode")
        for layer in (1, 2):
            idd = dev(ids)
            y2 = torch.zeros((2, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_moe_forward(sc.handle, layer, M.FT_MODE_STREAMED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), 2,
                             y2.data_ptr(), st)
            sim.stream_load(layer % 2)
            torch.cuda.synchronize()
            assert_close_rel(bf16_bits_to_f64(y2), OM.moe_layer(x, ids, w, expert_fn(recs, cfg, layer)), 2e-2,
                             f"streamed layer {layer}")
        sfi, ios, stamp, clock = M.ft_cache_snapshot(sc.handle, cfg.layers * cfg.E, cfg.slots)
        assert (sfi < 0).all() and (ios < 0).all() and (stamp == 0).all()
        r, y = decode_call()
        assert r.hits == 0 and r.q == 4
        assert_close_rel(y, ref0, 2e-2, "decode after streaming")
        for v, u in r.fills:
            assert np.array_equal(M.ft_cache_read_slot(sc.handle, v, cfg.S), recs[u])
        assert M.ft_cache_stats(sc.handle).layers_streamed == 2
    finally:
        sc.close()
        bank.close()


@gpu
def test_warm_decode_variant_gpu():
    """Prefill-warms-decode variant: layers streamed with FT_WARM_DECODE become
    residents exactly as the oracle's register_buffer says (maps, stamps and
    clock bit-exact), decode then hits them and computes the right layer, and
    a later miss takes the empty slots first."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(layers=3, E=4, k=2, slots=10, bp_mbps=60000, bh_mbps=60000)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 16, cfg.bp_mbps,
                   cfg.bh_mbps)
    sim = OC.SlotCacheSim(cfg.layers, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    n_ids = cfg.layers * cfg.E

    def same_state(what):
        sfi, ios, stamp, clock = M.ft_cache_snapshot(sc.handle, n_ids, cfg.slots)
        o_sfi, o_ios, o_stamp, o_clock = sim.arrays()
        assert np.array_equal(sfi, o_sfi) and np.array_equal(ios, o_ios), what
        assert np.array_equal(stamp, o_stamp) and clock == o_clock, what

    try:
        x = synth.tokens(cfg, 2, 3)
        ids = np.array([[0, 1], [3, 1]], dtype=np.int32)
        w = np.array([[0.5, 0.5], [0.25, 0.75]], np.float32)
        xd, wd = dev_u16(x), dev(w)

        def decode_call(layer):
            idd = dev(ids)
            y = torch.zeros((2, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_cache_classify(sc.handle, layer, idd.data_ptr(), 2, None, st)
            M.ft_moe_forward(sc.handle, layer, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), 2,
                             y.data_ptr(), st)
            r = sim.classify(layer, ids)
            torch.cuda.synchronize()
            assert np.array_equal(idd.cpu().numpy(), r.routes), f"routes of layer {layer}"
            assert_close_rel(bf16_bits_to_f64(y), OM.moe_layer(x, ids, w, expert_fn(recs, cfg, layer)), 2e-2,
                             f"decode layer {layer}")
            return r

        decode_call(0)
        same_state("after the first decode call")
        for layer in (1, 2):
            idd = dev(ids)
            y2 = torch.zeros((2, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_moe_forward(sc.handle, layer, M.FT_MODE_STREAMED | M.FT_WARM_DECODE, xd.data_ptr(), idd.data_ptr(),
                             wd.data_ptr(), 2, y2.data_ptr(), st)
            sim.stream_load(layer % 2)
            sim.register_buffer(layer % 2, layer)
            torch.cuda.synchronize()
            same_state(f"after streaming layer {layer}")
        r = decode_call(1)
        assert r.hits == 3 and r.m == 0
        r = decode_call(0)
        assert r.hits == 0 and r.q == 3 and [v for v, _ in r.fills] == [8, 9, 6]   # empties, then the oldest stamp
        same_state("after decode on the warmed cache")
        for v, u in r.fills:
            assert np.array_equal(M.ft_cache_read_slot(sc.handle, v, cfg.S), recs[u])
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("slots", [12000, 32768])
def test_control_at_the_maxima(slots):
    """E = 4,096 experts (the largest accepted), 512-token calls (4,096 routes)
    and up to N = 32,768 slots (the largest accepted; 12,000 and 32,768 take
    the victim scan's 16- and 32-keys-per-thread kernels), with more
    layer-experts (40,960) than slots, so the pool fills and then evicts;
    every output and the maps bit-exact against the simulator.  Records are
    the smallest the library accepts (MXFP4, d = f = 128)."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(layers=10, E=4096, k=8, d=128, f=128, fmt="mxfp4", slots=slots,
                                      bp_mbps=60000, bh_mbps=60000)
    rng = np.random.default_rng(slots)
    calls = 40
    tr = TraceRunner(cfg, [512] * calls, small=False)
    try:
        for i in range(calls):
            ids = np.stack([rng.choice(cfg.E, size=cfg.k, replace=False) for _ in range(512)])
            tr.call(int(rng.integers(0, cfg.layers)), ids)
        hits, fills, cpu = tr.check()
        s = M.ft_cache_stats(tr.sc.handle)
        assert fills > slots and s.evictions > 0 and hits > 0
    finally:
        tr.close()


@gpu
def test_many_route_call_refused_past_planner_key_space():
    """A CACHED forward of more than 1,024 routes on a cache of more than
    8,192 slots is refused (FT_ERR_UNSUPPORTED) before it takes any state:
    the next call (1,024 routes) still matches the simulator and the oracle,
    and no error flag is raised."""
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(E=16, k=8, slots=8193, cfg_id=94)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, 129, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    lib = M.lib()
    wr = synth.router(cfg, 0)
    try:
        for T, refused in ((129, True), (128, False)):
            x = synth.tokens(cfg, T, 900 + T)
            ids, w, _ = OR.route(x, wr, cfg.k)
            r = sim.classify(0, ids)
            xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
            y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_cache_classify(sc.handle, 0, idd.data_ptr(), T, None, st)
            status = lib.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(),
                                        T, y.data_ptr(), st)
            torch.cuda.synchronize()
            assert np.array_equal(idd.cpu().numpy(), r.routes), f"T {T}"
            if refused:
                assert status == M.FT_ERR_UNSUPPORTED and "8192" in M.ft_last_error(), M.ft_last_error()
                continue
            assert status == M.FT_OK, M.ft_last_error()
            ref = OM.moe_layer(x, ids, w, expert_fn(recs, cfg, 0, maxsize=cfg.E))
            assert_close_rel(bf16_bits_to_f64(y), ref, 2e-2, f"T {T}")
        s = M.ft_cache_stats(sc.handle)
        assert s.error_flags == 0 and s.calls == 2
    finally:
        sc.close()
        bank.close()
