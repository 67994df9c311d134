"""Records on their way into slots.  Every path that puts a record into a
slot copies the bank's record byte for byte: the decode fill, the full-layer
load of STREAMED mode and ft_cache_resize.  That includes block-FP8 records
whose size is not a multiple of 16 bytes (d = 256 with f = 128 or 384: 24 or
72 bytes of block scales after the codes), which the pool keeps 256 bytes
apart.  On every path the layer outputs match the oracle, and resize keeps the
oracle simulator's residents, stamps and clock."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import cache as OC, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, expert_fn, gpu, make_bank, oracle_rows
from test_gpu_layer import TOL, run_cached

SHAPES = [("fp8", 256, 128), ("fp8", 256, 384), ("bf16", 256, 128), ("mxfp4", 256, 128)]


def _slots_hold_their_records(sc, recs, n_ids, n_slots, what):
    sfi, ios, _, _ = M.ft_cache_snapshot(sc.handle, n_ids, n_slots)
    S = recs.shape[1]
    held = 0
    for s in range(n_slots):
        if ios[s] >= 0:
            got = M.ft_cache_read_slot(sc.handle, s, S)
            assert np.array_equal(got, recs[ios[s]]), f"{what}: slot {s} differs from bank record {ios[s]}"
            held += 1
    return held


@gpu
@pytest.mark.parametrize("fmt,d,f", SHAPES)
def test_fills_and_resize_copy_whole_records(fmt, d, f):
    """Cold cache, every miss filled (B_P = B_H): decode calls (GEMV) and
    T = 5 calls (GEMM) against the oracle, slot bytes against the bank; then
    resizes to fewer and to more slots against the simulator, with calls
    after each."""
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=2, d=d, f=f, E=16, k=4, slots=16, fmt=fmt, bp_mbps=60000,
                                        bh_mbps=60000)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sim = OC.SlotCacheSim(cfg.layers, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 5, cfg.bp_mbps, cfg.bh_mbps)
    try:
        exs = [expert_fn(recs, cfg, l, maxsize=16) for l in range(cfg.layers)]
        n_ids = cfg.layers * cfg.E

        def call(l, T, seed):
            x = synth.tokens(cfg, T, seed, l)
            ids, w, _ = OR.route(x, synth.router(cfg, l), cfg.k)
            sim.classify(l, ids)
            y, _ = run_cached(sc, l, x, ids, w)
            assert_close_rel(y, oracle_rows(x, ids, w, exs[l], range(T)), TOL[fmt], f"{fmt} layer {l} T {T}")

        for i, T in enumerate((1, 1, 5, 1, 5)):
            call(i % 2, T, 300 + i)
        held = _slots_hold_their_records(sc, recs, n_ids, cfg.slots, "after fills")
        assert held == sum(1 for u in sim.id_of_slot if u >= 0) and held >= 8
        M.ft_cache_resize(sc.handle, 10)
        sim.resize(10)
        sfi, ios, st, clk = M.ft_cache_snapshot(sc.handle, n_ids, 10)
        s_sfi, s_ios, s_st, s_clk = sim.arrays()
        assert np.array_equal(sfi, s_sfi) and np.array_equal(ios, s_ios) and np.array_equal(st, s_st)
        assert clk == s_clk
        assert _slots_hold_their_records(sc, recs, n_ids, 10, "after resize") == sum(1 for u in s_ios if u >= 0)
        for i, T in enumerate((1, 5)):
            call(i % 2, T, 400 + i)
        # and back up: the residents keep their slots' order, the new slots start empty
        M.ft_cache_resize(sc.handle, 24)
        sim.resize(24)
        sfi, ios, st, clk = M.ft_cache_snapshot(sc.handle, n_ids, 24)
        s_sfi, s_ios, s_st, s_clk = sim.arrays()
        assert np.array_equal(sfi, s_sfi) and np.array_equal(ios, s_ios) and np.array_equal(st, s_st)
        assert clk == s_clk
        assert _slots_hold_their_records(sc, recs, n_ids, 24, "after growth") == sum(1 for u in s_ios if u >= 0)
        for i, T in enumerate((5, 1, 5)):
            call(i % 2, T, 450 + i)
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
@pytest.mark.parametrize("fmt,d,f", SHAPES)
def test_streamed_layer_load_copies_whole_records(fmt, d, f):
    """STREAMED: a layer's E records are loaded into a full-layer buffer
    (slots b*E .. b*E + E - 1); the layer output matches the oracle and every
    buffer slot holds its bank record."""
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=2, d=d, f=f, E=16, k=4, slots=32, fmt=fmt)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    T = 5
    sc = SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, 2 * cfg.E, T, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        for l in range(cfg.layers):
            x = synth.tokens(cfg, T, 500 + l, l)
            ids, w, _ = OR.route(x, synth.router(cfg, l), cfg.k)
            xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
            y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
            M.ft_moe_forward(sc.handle, l, M.FT_MODE_STREAMED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), T,
                             y.data_ptr(), st)
            torch.cuda.synchronize()
            ex = expert_fn(recs, cfg, l, maxsize=16)
            assert_close_rel(bf16_bits_to_f64(y), oracle_rows(x, ids, w, ex, range(T)), TOL[fmt],
                             f"{fmt} streamed layer {l}")
            b = l % 2
            for e in range(cfg.E):
                got = M.ft_cache_read_slot(sc.handle, b * cfg.E + e, cfg.S)
                assert np.array_equal(got, recs[l * cfg.E + e]), f"buffer {b} slot {e} differs from its record"
        assert M.ft_cache_stats(sc.handle).error_flags == 0
    finally:
        sc.close()
        bank.close()


@gpu
def test_short_host_bank_is_refused():
    """A pinned bank whose allocation ends before layers * experts records is
    refused when the cache is created (nothing is launched); a bank of the
    full size is accepted, also when it starts inside a larger allocation."""
    from moe_expert_execution_amd.tensors import PinnedBank
    cuda()
    cfg = synth.CONFIGS["tiny"].with_(layers=2)
    need = cfg.layers * cfg.E * cfg.S
    mk = lambda ptr: SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, cfg.fmt, ptr, cfg.slots, 4, cfg.bp_mbps,
                               cfg.bh_mbps)
    short = PinnedBank(need - 4096)
    try:
        with pytest.raises(M.FtError) as ei:
            mk(short.ptr)
        assert ei.value.status == M.FT_ERR_ARG, str(ei.value)
    finally:
        short.close()
    big = PinnedBank(need + 8192)
    try:
        mk(big.ptr + 4096).close()
        with pytest.raises(M.FtError) as ei:
            mk(big.ptr + 8192 + 256)
        assert ei.value.status == M.FT_ERR_ARG, str(ei.value)
    finally:
        big.close()
