"""The block-FP8 configuration run as configured, through the CACHED path:
one layer, d = 4096, E = 256, top-8, f = 2048, e4m3 weights with 128 x 128
fp32 block scales, a 64-slot cache that starts cold for each token count,
B_P/B_H = 20/60 GB/s, Zipf(1.1) expert popularity; T = 1, 64, 2048 tokens per
call for 256, 256 and 16 steps.

Every call's control step (unique set, classes, q, evictions, host-run ids,
rewritten routes) is compared bit for bit with the oracle's simulator, the
maps and counters after the run too; every output row of the listed steps is
compared with the oracle's fp64 layer (5e-2 of its largest value).  Pages:
"The Expert Cache That Follows the Router", sections "One logical expert, two
physical levels of memory" (block-FP8 records) and "How residency follows
demand without leaving the device"."""
import time

import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import ClassifyBuffers, SlotCache
from oracle import cache as OC

from gpu_util import (assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, gpu, make_bank, oracle_layer_all_rows,
                      record_decoder)

TOL = 5e-2


@pytest.fixture(scope="module")
def fp8_bank():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cfg = synth.CONFIGS["fp8"]
    bank = make_bank(cfg)
    yield cfg, bank
    bank.close()


@gpu
@pytest.mark.parametrize("T,steps,float_steps", [(1, 256, tuple(range(0, 256, 8))), (64, 256, (0, 1, 128, 255)),
                                                 (2048, 16, (0, 15))])
def test_fp8_config_as_configured(fp8_bank, T, steps, float_steps):
    cuda()
    cfg, bank = fp8_bank
    assert steps == cfg.steps[cfg.tokens.index(T)]
    recs = bank.records(cfg.S)
    sc = SlotCache(1, cfg.E, cfg.k, cfg.d, cfg.f, "fp8", bank.ptr, cfg.slots, T, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(1, cfg.E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    out = ClassifyBuffers(T * cfg.k)
    dec = record_decoder(recs, cfg, 0)
    y = torch.zeros((T, cfg.d), dtype=torch.int16, device="cuda")
    hits = fills = host = 0
    try:
        for step in range(steps):
            x = synth.tokens(cfg, T, 300 + step, T)
            ids, w = synth.zipf_routes(cfg, T, step)
            xd, idd, wd = dev_u16(x), dev(ids.astype(np.int32)), dev(w)
            t0 = time.perf_counter()
            M.ft_cache_classify(sc.handle, 0, idd.data_ptr(), T, out.struct, st)
            M.ft_moe_forward(sc.handle, 0, M.FT_MODE_CACHED, xd.data_ptr(), idd.data_ptr(), wd.data_ptr(), T,
                             y.data_ptr(), st)
            got = out.host()                      # synchronises
            t_call = time.perf_counter() - t0
            r = sim.classify(0, ids)
            where = f"T {T} step {step}"
            assert (got["n_uniq"], got["hits"], got["m"], got["q"]) == (len(r.uniq), r.hits, r.m, r.q), where
            assert got["uniq"] == r.uniq and got["cls"] == r.cls and got["slot"] == r.slot, where
            assert got["ev_slot"] == [v for v, _, _ in r.evictions], where
            assert got["ev_old"] == [o for _, o, _ in r.evictions], where
            assert got["ev_new"] == [u for _, _, u in r.evictions], where
            assert got["cpu_ids"] == r.cpu, where
            assert np.array_equal(idd.cpu().numpy(), r.routes), where
            hits, fills, host = hits + r.hits, fills + r.q, host + r.m - r.q
            if step in float_steps:
                assert_close_rel(bf16_bits_to_f64(y), oracle_layer_all_rows(x, ids, w, dec), TOL, where)
            if T >= 2048 or step % 32 == 31 or step in float_steps:
                print(f"fp8 T={T}: step {step + 1} of {steps} checked (call {t_call * 1e3:.1f} ms)", flush=True)
        sfi, ios, stamp, clock = M.ft_cache_snapshot(sc.handle, cfg.E, cfg.slots)
        osfi, oios, ostamp, oclock = sim.arrays()
        assert np.array_equal(sfi, osfi) and np.array_equal(ios, oios)
        assert np.array_equal(stamp, ostamp) and clock == oclock
        s = M.ft_cache_stats(sc.handle)
        assert (s.hits, s.fills, s.cpu_experts, s.error_flags) == (hits, fills, host, 0)
        assert fills > 0 and host > 0 and hits > 0
        print(f"fp8 T={T}: {steps} steps, hits {hits}, fills {fills}, host experts {host}")
    finally:
        sc.close()
