"""GPU parity on the one-layer tiny configuration (16 tokens, d=256, E=8, top-2,
f=128, 4 slots, B_P/B_H 25/50 GB/s): routing, control and the float layer."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import ClassifyBuffers, SlotCache
from oracle import cache as OC, moe as OM, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, expert_fn, gpu, make_bank

C1 = synth.CONFIGS["tiny"]


def _route_gpu(cfg, x, wr, T):
    shp = M.shape(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.fmt)
    xd, wd = dev_u16(x), dev_u16(wr)
    ids = torch.full((T, cfg.k), -1, dtype=torch.int32, device="cuda")
    w = torch.zeros((T, cfg.k), dtype=torch.float32, device="cuda")
    M.ft_moe_route(shp, xd.data_ptr(), wd.data_ptr(), T, ids.data_ptr(), w.data_ptr(),
                   torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@gpu
def test_route_tiny_bit_exact():
    cuda()
    x = synth.tokens(C1, 16, 0)
    wr = synth.router(C1, 0)
    ids, w = _route_gpu(C1, x, wr, 16)
    rid, rw, gap = OR.route(x, wr, C1.k)
    assert np.array_equal(ids, rid), (ids, rid)
    np.testing.assert_allclose(w, rw, rtol=1e-6, atol=0)


@gpu
@pytest.mark.parametrize("cfgname,T,E,k,d", [
    ("decode", 1, None, None, None), ("decode", 300, None, None, None), ("mxfp4", 37, None, None, None),
    ("tiny", 5, None, None, None), ("decode", 1531, None, None, None), ("fp8", 1000, None, None, None),
    ("decode", 77, 64, None, None), ("decode", 40, 96, None, None),
    # one token with E % 8 != 0; 2..16 tokens with odd E; one and 16 tokens at E = 256; the
    # general kernel at E = 200; d off a multiple of 128; a single expert
    ("tiny", 1, 5, 2, None), ("tiny", 7, 12, 3, None), ("fp8", 1, None, None, None),
    ("mxfp4", 16, None, None, None), ("decode", 17, 200, 6, None), ("tiny", 3, 24, 4, 200),
    ("tiny", 33, 60, 5, 72), ("tiny", 4, 1, 1, None),
    # the largest top-k (16): one token, the small-T path, the matrix cores
    ("decode", 1, None, 16, None), ("tiny", 9, 32, 16, None), ("decode", 40, None, 16, None)])
def test_route_shapes_bit_exact(cfgname, T, E, k, d):
    """Routing ids bit-exact and weights to fp32 rounding against the oracle, for
    the small-T paths (one token, 16-byte router rows when E % 8 == 0; up to 16
    tokens), the matrix-core path (E in {64, 128, 256}, d % 128 == 0; ragged
    last workgroup) and the general path."""
    cuda()
    cfg = synth.CONFIGS[cfgname]
    if E is not None:
        cfg = cfg.with_(E=E)
    if k is not None:
        cfg = cfg.with_(k=k)
    if d is not None:
        cfg = cfg.with_(d=d)
    x = synth.tokens(cfg, T, 11)
    wr = synth.router(cfg, 3)
    ids, w = _route_gpu(cfg, x, wr, T)
    rid, rw, gap = OR.route(x, wr, cfg.k)
    bad = np.nonzero((ids != rid).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} tokens differ; min top-(k+1) gap {gap:.2e}"
    np.testing.assert_allclose(w, rw, rtol=1e-6, atol=0)


def _compare_classify(r, got, layer):
    assert got["n_uniq"] == len(r.uniq) and got["hits"] == r.hits and got["m"] == r.m and got["q"] == r.q
    assert got["uniq"] == r.uniq
    assert got["cls"] == r.cls
    assert got["slot"] == r.slot
    assert got["ev_slot"] == [v for v, _, _ in r.evictions]
    assert got["ev_old"] == [o for _, o, _ in r.evictions]
    assert got["ev_new"] == [n for _, _, n in r.evictions]
    assert got["cpu_ids"] == r.cpu


@gpu
def test_tiny_layer_steps():
    """Eight calls of 16 fresh tokens: route, classify and forward against the
    oracle at every step (ids, classes, q, evictions, maps bit-exact; y within
    2e-2 of max |y|), and the filled slots hold the bank's bytes."""
    cuda()
    bank = make_bank(C1)
    recs = bank.records(C1.S)
    sc = SlotCache(1, C1.E, C1.k, C1.d, C1.f, "bf16", bank.ptr, C1.slots, 16, C1.bp_mbps, C1.bh_mbps)
    sim = OC.SlotCacheSim(1, C1.E, C1.slots, C1.bp_mbps, C1.bh_mbps)
    wr = synth.router(C1, 0)
    st = torch.cuda.current_stream().cuda_stream
    buf = ClassifyBuffers(16 * C1.k)
    ex = expert_fn(recs, C1, 0)
    saw = set()
    for step in range(8):
        x = synth.tokens(C1, 16, 100 + step)
        ids, w, _ = OR.route(x, wr, C1.k)
        r = sim.classify(0, ids)
        xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
        y = torch.zeros((16, C1.d), dtype=torch.int16, device="cuda")
        M.ft_cache_classify(sc.handle, 0, idd.data_ptr(), 16, buf.struct, st)
        M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), 16,
                         y.data_ptr(), st)
        torch.cuda.synchronize()
        _compare_classify(r, buf.host(), 0)
        assert np.array_equal(idd.cpu().numpy(), r.routes)
        sfi, ios, stamp, clock = M.ft_cache_snapshot(sc.handle, C1.E, C1.slots)
        osfi, oios, ostamp, oclock = sim.arrays()
        assert np.array_equal(sfi, osfi) and np.array_equal(ios, oios)
        assert np.array_equal(stamp, ostamp) and clock == oclock
        for v, u in r.fills:
            assert np.array_equal(M.ft_cache_read_slot(sc.handle, v, C1.S), recs[u])
        ref = OM.moe_layer(x, ids, w, ex)
        assert_close_rel(bf16_bits_to_f64(y), ref, 2e-2, f"step {step}")
        saw |= set(r.cls)
    assert saw == {OC.HIT, OC.FILL, OC.CPU}
    s = M.ft_cache_stats(sc.handle)
    assert s.error_flags == 0 and s.calls == 8
    sc.close()
    bank.close()


@gpu
@pytest.mark.parametrize("bp,bh,mf", [(60000, 60000, -1), (25000, 50000, 0), (11800, 47500, -1)])
def test_tiny_partition_identity(bp, bh, mf):
    """All-fill, all-host and mixed splits give the same layer output."""
    cuda()
    bank = make_bank(C1)
    recs = bank.records(C1.S)
    sc = SlotCache(1, C1.E, C1.k, C1.d, C1.f, "bf16", bank.ptr, C1.slots, 16, bp, bh, mf)
    wr = synth.router(C1, 0)
    st = torch.cuda.current_stream().cuda_stream
    ex = expert_fn(recs, C1, 0)
    sim = OC.SlotCacheSim(1, C1.E, C1.slots, bp, bh, mf)
    fills = cpu = 0
    for step in range(4):
        x = synth.tokens(C1, 16, 200 + step)
        ids, w, _ = OR.route(x, wr, C1.k)
        r = sim.classify(0, ids)
        fills += r.q
        cpu += r.m - r.q
        xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
        y = torch.zeros((16, C1.d), dtype=torch.int16, device="cuda")
        M.ft_cache_classify(sc.handle, 0, idd.data_ptr(), 16, None, st)
        M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), 16,
                         y.data_ptr(), st)
        torch.cuda.synchronize()
        assert_close_rel(bf16_bits_to_f64(y), OM.moe_layer(x, ids, w, ex), 2e-2, f"step {step}")
    s = M.ft_cache_stats(sc.handle)
    assert s.fills == fills and s.cpu_experts == cpu
    if mf == 0:
        assert s.fills == 0 and s.cpu_experts == s.misses
    sc.close()
    bank.close()
