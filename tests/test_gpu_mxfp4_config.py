"""The MXFP4 configuration run as configured: 61 MoE layers, d = 7168, E = 256,
top-8, f = 2048, e2m1 weights with an e8m0 scale per 32 along K.

The 61-layer host bank (15,616 records, 365 GB) cannot be pinned on one host,
so the layers' banks alias: layer l reads the pinned records of physical layer
l mod 4 (ft_cache_create_layers).  Flat ids stay per layer, so every control
decision is that of 61 distinct layers; only the weight values repeat.

 - decode: one token per call, 128 steps x 61 layers from a cold cache of
   7,385 slots (60% of 288e9 bytes of HBM), B_P/B_H = 20/60 GB/s, per-layer
   AR(1) hidden states; every call's ids (through the rewritten routes),
   weights and control outputs against the oracle, the outputs of all
   layers at the first and the last step against the oracle's fp64 layer;
 - prefill: a 4,096-token chunk streamed through all 61 layers with the
   full-layer double buffer (2E = 512 slots), the next layer prefetched;
   every layer's routing ids bit-exact, every output row of two layers (one
   per buffer) against the oracle.

Pages: METAL MEDIA summary, Figure 3 caption (an MXFP4 model of this size);
"The Expert Cache That Follows the Router", section "One logical expert, two
physical levels of memory" (MXFP4 banks); txtmix article, "prefill 不是稀疏的"
(the pool streamed layer by layer during prefill)."""
import numpy as np
import pytest
import torch

import moe_expert_execution_amd as M
import synth
from moe_expert_execution_amd.tensors import SlotCache
from oracle import cache as OC, route as OR

from gpu_util import assert_close_rel, bf16_bits_to_f64, cuda, gpu, make_bank, oracle_layer_all_rows, record_decoder

L_PHYS = 4
TOL = 5e-2


@pytest.fixture(scope="module")
def mx_banks():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    cfg = synth.CONFIGS["mxfp4"]
    bank = make_bank(cfg.with_(layers=L_PHYS))
    ptrs = [bank.ptr + (l % L_PHYS) * cfg.E * cfg.S for l in range(cfg.layers)]
    yield cfg, bank, ptrs
    bank.close()


def decoder(bank, cfg, layer):
    return record_decoder(bank.records(cfg.S), cfg, layer % L_PHYS)


@gpu
def test_mxfp4_decode_as_configured(mx_banks):
    cuda()
    cfg, bank, ptrs = mx_banks
    L, E, k, d, N, steps = cfg.layers, cfg.E, cfg.k, cfg.d, cfg.slots, cfg.steps[cfg.tokens.index(1)]
    assert N == 7385
    sc = SlotCache(L, E, k, d, cfg.f, "mxfp4", ptrs, N, 1, cfg.bp_mbps, cfg.bh_mbps)
    sim = OC.SlotCacheSim(L, E, N, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    try:
        xs_np = [synth.ar1_tokens(cfg, l, steps) for l in range(L)]
        wr_np = [synth.router(cfg, l) for l in range(L)]
        xs = torch.stack([torch.from_numpy(x.view(np.int16)) for x in xs_np]).cuda()
        wr = torch.stack([torch.from_numpy(w_.view(np.int16)) for w_ in wr_np]).cuda()
        n = steps * L
        routes = torch.empty((n, k), dtype=torch.int32, device="cuda")
        w = torch.empty((n, k), dtype=torch.float32, device="cuda")
        y = torch.empty((n, d), dtype=torch.int16, device="cuda")
        counts = torch.zeros((n, 4), dtype=torch.int32, device="cuda")
        arr = {a: torch.full((n, k), -7, dtype=torch.int32, device="cuda")
               for a in ("uniq", "slot", "ev_slot", "ev_old", "ev_new", "cpu_ids")}
        cls = torch.full((n, k), 255, dtype=torch.uint8, device="cuda")
        for s in range(steps):
            for l in range(L):
                i = s * L + l
                xp = xs[l, s].data_ptr()
                out = M.FtClassifyOut(counts[i].data_ptr(), arr["uniq"][i].data_ptr(), cls[i].data_ptr(),
                                      arr["slot"][i].data_ptr(), arr["ev_slot"][i].data_ptr(),
                                      arr["ev_old"][i].data_ptr(), arr["ev_new"][i].data_ptr(),
                                      arr["cpu_ids"][i].data_ptr(), k)
                M.ft_moe_route(sc.shape, xp, wr[l].data_ptr(), 1, routes[i].data_ptr(), w[i].data_ptr(), st)
                M.ft_cache_classify(sc.handle, l, routes[i].data_ptr(), 1, out, st)
                M.ft_moe_forward(sc.handle, l, M.FT_MODE_CACHED, xp, routes[i].data_ptr(), w[i].data_ptr(), 1,
                                 y[i].data_ptr(), st)
            if s % 32 == 31:
                torch.cuda.synchronize()
                print(f"mxfp4 decode: step {s + 1} of {steps} done", flush=True)
        torch.cuda.synchronize()
        routes_h, w_h, counts_h, cls_h = routes.cpu().numpy(), w.cpu().numpy(), counts.cpu().numpy(), cls.cpu().numpy()
        arr_h = {a: v.cpu().numpy() for a, v in arr.items()}
        hits = fills = host = 0
        compare = []
        for s in range(steps):
            for l in range(L):
                i = s * L + l
                x = xs_np[l][s:s + 1]
                ids_o, w_o, _ = OR.route(x, wr_np[l], k)
                r = sim.classify(l, ids_o)
                where = f"step {s} layer {l}"
                nu = len(r.uniq)
                assert np.array_equal(routes_h[i], r.routes.reshape(-1)), where
                np.testing.assert_allclose(w_h[i], w_o.reshape(-1), rtol=1e-6, atol=0, err_msg=where)
                assert list(counts_h[i]) == [nu, r.hits, r.m, r.q], where
                assert arr_h["uniq"][i, :nu].tolist() == r.uniq and cls_h[i, :nu].tolist() == r.cls, where
                assert arr_h["slot"][i, :nu].tolist() == r.slot, where
                assert arr_h["ev_slot"][i, :r.q].tolist() == [v for v, _, _ in r.evictions], where
                assert arr_h["ev_old"][i, :r.q].tolist() == [o for _, o, _ in r.evictions], where
                assert arr_h["ev_new"][i, :r.q].tolist() == [u for _, _, u in r.evictions], where
                assert arr_h["cpu_ids"][i, :r.m - r.q].tolist() == r.cpu, where
                hits, fills, host = hits + r.hits, fills + r.q, host + r.m - r.q
                if s in (0, steps - 1):
                    compare.append((i, l, x, ids_o, w_o))
            if s % 16 == 15:
                print(f"mxfp4 decode: control of step {s + 1} of {steps} bit-exact", flush=True)
        sfi, ios, stamp, clock = M.ft_cache_snapshot(sc.handle, L * E, N)
        osfi, oios, ostamp, oclock = sim.arrays()
        assert np.array_equal(sfi, osfi) and np.array_equal(ios, oios)
        assert np.array_equal(stamp, ostamp) and clock == oclock
        stt = M.ft_cache_stats(sc.handle)
        assert (stt.hits, stt.fills, stt.cpu_experts, stt.error_flags) == (hits, fills, host, 0)
        assert hits > 0 and fills > 0 and host > 0
        print(f"mxfp4 decode: {n} calls, control bit-exact; hits {hits}, fills {fills}, host experts {host}", flush=True)
        y_h = bf16_bits_to_f64(y)
        for j, (i, l, x, ids_o, w_o) in enumerate(compare):
            ref = oracle_layer_all_rows(x, ids_o, w_o, decoder(bank, cfg, l))
            assert_close_rel(y_h[i:i + 1], ref, TOL, f"call {i} (step {i // L}, layer {l})")
            if j % 20 == 19:
                print(f"mxfp4 decode: outputs of {j + 1} of {len(compare)} calls within tolerance", flush=True)
    finally:
        sc.close()


@gpu
def test_mxfp4_prefill_stream_as_configured(mx_banks):
    cuda()
    cfg, bank, ptrs = mx_banks
    L, E, k, d, T = cfg.layers, cfg.E, cfg.k, cfg.d, cfg.tokens[0]
    assert T == 4096
    sc = SlotCache(L, E, k, d, cfg.f, "mxfp4", ptrs, 2 * E, T, cfg.bp_mbps, cfg.bh_mbps)
    st = torch.cuda.current_stream().cuda_stream
    compare_layers = (1, L - 1)          # buffer 1 and buffer 0
    try:
        x_np = synth.tokens(cfg, T, 7)
        x = torch.from_numpy(x_np.view(np.int16)).cuda()
        ids = torch.empty((L, T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((L, T, k), dtype=torch.float32, device="cuda")
        ys = {l: torch.empty((T, d), dtype=torch.int16, device="cuda") for l in compare_layers}
        y_other = torch.empty((T, d), dtype=torch.int16, device="cuda")
        wr_np = [synth.router(cfg, l) for l in range(L)]
        for l in range(L):
            wr = torch.from_numpy(wr_np[l].view(np.int16)).cuda()
            M.ft_moe_route(sc.shape, x.data_ptr(), wr.data_ptr(), T, ids[l].data_ptr(), w[l].data_ptr(), st)
        for l in range(L):
            M.ft_moe_forward(sc.handle, l, M.FT_MODE_STREAMED | M.FT_PREFETCH_NEXT, x.data_ptr(), ids[l].data_ptr(),
                             w[l].data_ptr(), T, ys.get(l, y_other).data_ptr(), st)
            if l % 16 == 15:
                torch.cuda.synchronize()
                print(f"mxfp4 prefill: layer {l + 1} of {L} done", flush=True)
        torch.cuda.synchronize()
        stt = M.ft_cache_stats(sc.handle)
        assert stt.error_flags == 0 and stt.layers_streamed == L
        ids_h, w_h = ids.cpu().numpy(), w.cpu().numpy()
        oracle_routes = {}
        for l in range(L):
            ids_o, w_o, _ = OR.route(x_np, wr_np[l], k)
            if l % 16 == 15:
                print(f"mxfp4 prefill: routing of layer {l + 1} of {L} checked", flush=True)
            assert np.array_equal(ids_h[l], ids_o), f"routing ids of layer {l}"
            np.testing.assert_allclose(w_h[l], w_o, rtol=1e-6, atol=0, err_msg=f"weights of layer {l}")
            if l in compare_layers:
                oracle_routes[l] = (ids_o, w_o)
        for l in compare_layers:
            ids_o, w_o = oracle_routes[l]
            ref = oracle_layer_all_rows(x_np, ids_o, w_o, decoder(bank, cfg, l))
            assert_close_rel(bf16_bits_to_f64(ys[l]), ref, TOL, f"prefill layer {l}")
            print(f"mxfp4 prefill: layer {l} all {T} rows within tolerance", flush=True)
    finally:
        sc.close()
