"""The bandwidth profiler (ft_cache_profile) on the real fill and host paths,
and q* from a measured profile (ft_cache_set_profile) against the oracle's
simulator run with the same profile."""
import numpy as np
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import ClassifyBuffers, SlotCache
from oracle import cache as OC, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, expert_fn, gpu, make_bank


@gpu
def test_profile_measures_both_paths_then_feeds_q():
    cuda()
    cfg = synth.CONFIGS["decode"].with_(layers=1, slots=64)
    bank = make_bank(cfg)                                   # 128 records of 9.4 MB
    recs = bank.records(cfg.S)
    st = torch.cuda.current_stream().cuda_stream
    T = 4
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "bf16", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
    wr = synth.router(cfg, 0)
    wr_d = torch.from_numpy(wr.view(np.int16)).cuda()

    def route(step):
        x = synth.tokens(cfg, T, 50 + step)
        ids, w = OR.route(x, wr, cfg.k)[:2]
        return x, ids.astype(np.int32), w.astype(np.float32)

    # some state first (a classify whose fills are still pending), which the profiler must clear
    x, ids, w = route(0)
    ids_d = torch.from_numpy(ids.reshape(-1)).cuda()
    M.ft_cache_classify(sc.handle, 0, ids_d.data_ptr(), T, None, st)

    prof = M.ft_cache_profile(sc.handle, 16)
    assert 1_000 < prof.bp_mbps < 200_000, prof.bp_mbps      # a PCIe link: 1 .. 200 GB/s
    assert 1_000 < prof.bh_mbps < 5_000_000, prof.bh_mbps    # host memory through the workers
    assert prof.max_fetch == -1
    sfi, ios, stamp, clk = M.ft_cache_snapshot(sc.handle, cfg.E, cfg.slots)
    assert (sfi == -1).all() and (ios == -1).all() and (stamp == 0).all() and clk == 1

    M.ft_cache_set_profile(sc.handle, prof)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, prof.bp_mbps, prof.bh_mbps, -1)
    out = ClassifyBuffers(T * cfg.k)
    ex = expert_fn(recs, cfg, 0)
    y = torch.empty((T, cfg.d), dtype=torch.int16, device="cuda")
    for step in range(6):
        x, ids, w = route(step + 1)
        ids_d = torch.from_numpy(ids.reshape(-1)).cuda()
        M.ft_cache_classify(sc.handle, 0, ids_d.data_ptr(), T, out.struct, st)
        got = out.host()
        r = sim.classify(0, ids)
        assert (got["n_uniq"], got["hits"], got["m"], got["q"]) == (len(r.uniq), r.hits, r.m, r.q), step
        assert got["cls"] == r.cls and got["uniq"] == r.uniq, step
        # the layer output after the profiler's reset is still the oracle's
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        wd = torch.from_numpy(w.reshape(-1)).cuda()
        M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), ids_d.data_ptr(), wd.data_ptr(), T,
                         y.data_ptr(), st)
        from oracle import moe as OM
        ref = OM.moe_layer(x, ids, w, ex)
        assert_close_rel(bf16_bits_to_f64(y), ref, 2e-2, f"step {step}")
    assert M.ft_cache_stats(sc.handle).error_flags == 0
    sc.close()
    bank.close()
