"""Parity of the decode configuration at its full size, in the launch
configuration the benchmark times: 48 layers, d=2048, E=128, top-8, f=768,
bf16, one token per call, 1,024 slots from cold and the whole 6,144-record
host bank pinned; per call ft_moe_route, ft_cache_classify and a CACHED
ft_moe_forward on one stream, all calls issued before one sync.

Every call's rewritten routes are compared bit for bit with those of the
oracle's slot-cache simulator fed by the oracle's routing (so the GPU's ids
are checked through them), every call's weights with the oracle's, and every
call's output with the oracle's fp64 layer.  With q about m/3 and at least
one fill per call, every call here has fills and host experts; the first
step's calls have no hits (the cold start), later ones mix hits in."""
import numpy as np
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import cache as OC, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, gpu, make_bank, oracle_layer_all_rows, record_decoder

STEPS = 6


@gpu
def test_decode_full_config():
    cuda()
    cfg = synth.CONFIGS["decode"]
    L, E, k, d = cfg.layers, cfg.E, cfg.k, cfg.d
    bank = make_bank(cfg)
    recs = bank.records(cfg.S)
    sc = SlotCache(L, E, k, d, cfg.f, "bf16", bank.ptr, cfg.slots, 1, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(L, E, cfg.slots, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        xs_np = [synth.ar1_tokens(cfg, l, STEPS) for l in range(L)]
        wr_np = [synth.router(cfg, l) for l in range(L)]
        xs = torch.stack([torch.from_numpy(x.view(np.int16)) for x in xs_np]).cuda()
        wr = torch.stack([torch.from_numpy(w_.view(np.int16)) for w_ in wr_np]).cuda()
        n = STEPS * L
        routes = torch.empty((n, k), dtype=torch.int32, device="cuda")
        w = torch.empty((n, k), dtype=torch.float32, device="cuda")
        y = torch.empty((n, d), dtype=torch.int16, device="cuda")
        for s in range(STEPS):
            for l in range(L):
                i = s * L + l
                xp = xs[l, s].data_ptr()
                M.ft_moe_route(sc.shape, xp, wr[l].data_ptr(), 1, routes[i].data_ptr(), w[i].data_ptr(), st)
                M.ft_cache_classify(sc.handle, l, routes[i].data_ptr(), 1, None, st)
                M.ft_moe_forward(sc.handle, l, M.FT_MODE_CACHED, xp, routes[i].data_ptr(), w[i].data_ptr(), 1,
                                 y[i].data_ptr(), st)
        torch.cuda.synchronize()
        routes_h, w_h = routes.cpu().numpy(), w.cpu().numpy()

        calls, kinds = [], {"no_hits": [], "hits": []}
        hits = fills = host = 0
        for s in range(STEPS):
            for l in range(L):
                i = s * L + l
                x = xs_np[l][s:s + 1]
                ids_o, w_o, _ = OR.route(x, wr_np[l], k)
                r = sim.classify(l, ids_o)
                where = f"step {s} layer {l}"
                assert np.array_equal(routes_h[i], r.routes.reshape(-1)), where
                np.testing.assert_allclose(w_h[i], w_o.reshape(-1), rtol=1e-6, atol=0, err_msg=where)
                calls.append((l, x, ids_o, w_o))
                hits, fills, host = hits + r.hits, fills + r.q, host + r.m - r.q
                kinds["hits" if r.hits else "no_hits"].append(i)
        assert fills > 0 and host > 0 and all(kinds.values()), {key: len(v) for key, v in kinds.items()}
        s_ = M.ft_cache_stats(sc.handle)
        assert (s_.hits, s_.fills, s_.cpu_experts, s_.error_flags) == (hits, fills, host, 0)

        y_h = bf16_bits_to_f64(y)
        for i, (l, x, ids_o, w_o) in enumerate(calls):
            ref = oracle_layer_all_rows(x, ids_o, w_o, record_decoder(recs, cfg, l))
            assert_close_rel(y_h[i:i + 1], ref, 2e-2, f"call {i} (step {i // L}, layer {l})")
    finally:
        sc.close()
        bank.close()
