"""ft_moe_forward_noalloc through the C ABI against ft_moe_forward.

Two caches built alike see the same calls: one runs the CACHED forward, the
other the variant whose per-call scratch comes from the static per-GPU array.
Two calls in a row, the second with fewer tokens (a smaller piece of the
array, which still holds the first call's contents).  The same kernels run in
the same order, so outputs, rewritten routes and cache state must agree bit
for bit, and both outputs must match the oracle (2e-2 of the largest value
for bf16 weights, 5e-2 for MXFP4).  Calls the array cannot serve are refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, dev, dev_u16, gpu, make_bank, oracle_layer_all_rows, \
    record_decoder

TOL = {"bf16": 2e-2, "mxfp4": 5e-2}


@gpu
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_noalloc_forward_equals_forward(fmt):
    cuda()
    base = synth.CONFIGS["decode"] if fmt == "bf16" else synth.CONFIGS["mxfp4"]
    cfg = base.with_(layers=2, E=16, slots=12, bp_mbps=20000, bh_mbps=60000)
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    mk = lambda: SlotCache(cfg.layers, cfg.E, cfg.k, cfg.d, cfg.f, fmt, bank.ptr, cfg.slots, 8, cfg.bp_mbps,
                           cfg.bh_mbps)
    a, b = mk(), mk()
    st = torch.cuda.current_stream().cuda_stream
    lib = M.lib()
    try:
        # refused before anything is enqueued: more than 4 tokens
        x8 = torch.zeros((8, cfg.d), dtype=torch.int16, device="cuda")
        r8 = torch.zeros((8, cfg.k), dtype=torch.int32, device="cuda")
        w8 = torch.zeros((8, cfg.k), dtype=torch.float32, device="cuda")
        assert lib.ft_moe_forward_noalloc(b.handle, 0, x8.data_ptr(), r8.data_ptr(), w8.data_ptr(), 5, x8.data_ptr(),
                                          st) == M.FT_ERR_UNSUPPORTED, M.ft_last_error()
        for call, (layer, T) in enumerate(((0, 4), (1, 1))):
            x = synth.tokens(cfg, T, 700 + call, layer)
            ids, w, _ = OR.route(x, synth.router(cfg, layer), cfg.k)
            xd, wd = dev_u16(x), dev(w)
            ra, rb = dev(ids.astype(np.int32)), dev(ids.astype(np.int32))
            ya = torch.full((T, cfg.d), 7, dtype=torch.int16, device="cuda")
            yb = torch.full((T, cfg.d), 9, dtype=torch.int16, device="cuda")
            M.ft_cache_classify(a.handle, layer, ra.data_ptr(), T, None, st)
            M.ft_moe_forward(a.handle, layer, M.FT_MODE_CACHED, xd.data_ptr(), ra.data_ptr(), wd.data_ptr(), T,
                             ya.data_ptr(), st)
            M.ft_cache_classify(b.handle, layer, rb.data_ptr(), T, None, st)
            M.ft_moe_forward_noalloc(b.handle, layer, xd.data_ptr(), rb.data_ptr(), wd.data_ptr(), T, yb.data_ptr(), st)
            torch.cuda.synchronize()
            where = f"{fmt} call {call} (T {T})"
            assert torch.equal(ra, rb), where
            assert torch.equal(ya, yb), f"{where}: outputs differ"
            n_ids = cfg.layers * cfg.E
            sa, sb = M.ft_cache_snapshot(a.handle, n_ids, cfg.slots), M.ft_cache_snapshot(b.handle, n_ids, cfg.slots)
            for u, v in zip(sa[:3], sb[:3]):
                assert np.array_equal(u, v), where
            assert sa[3] == sb[3], where
            ref = oracle_layer_all_rows(x, ids, w, record_decoder(recs, cfg, layer))
            assert_close_rel(bf16_bits_to_f64(yb), ref, TOL[fmt], where)
            assert (ra.cpu().numpy() < 0).any() and (ra.cpu().numpy() >= 0).any(), "both branches should run"
        ca, cb = M.ft_cache_stats(a.handle), M.ft_cache_stats(b.handle)
        assert ca.error_flags == 0 and cb.error_flags == 0
        assert (ca.hits, ca.fills, ca.cpu_experts) == (cb.hits, cb.fills, cb.cpu_experts)
    finally:
        a.close()
        b.close()
        bank.close()
