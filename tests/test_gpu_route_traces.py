"""GPU routing (ft_moe_route) against the oracle's routing over whole traces,
in the launch configuration each path uses: ids bit-exact (ordered), weights
within 1e-6 relative.  The oracle's smallest relative gap between adjacent
logits among a token's top k+1 is printed: an id mismatch is only possible
where it approaches the ~1e-15 of fp64 summation order.

 - decode: 48 layers x 256 steps, one token per call (12,288 calls), the
   per-layer AR(1) hidden states through each layer's router;
 - prefill: the 8,192-token chunk through each of the 24 streamed layers'
   routers (the matrix-core path);
 - MXFP4 layers (d = 7168, E = 256): the 4,096-token prefill chunk through
   all 61 routers, and 128 decode steps x 61 layers one token per call.

Routing is the first step of the layer ("Making Large MoE Models Practical on
a Single Machine", section 1: each token selects k of the layer's E experts)."""
import numpy as np
import torch

import moe_expert_execution_amd as M
import synth
from oracle import route as OR

from gpu_util import cuda, gpu


def check(ids_gpu, w_gpu, ids_ref, w_ref, what):
    bad = np.nonzero((ids_gpu != ids_ref).any(axis=-1))
    assert bad[0].size == 0, f"{what}: {bad[0].size} tokens with other ids, first at {[b[:3] for b in bad]}"
    np.testing.assert_allclose(w_gpu, w_ref, rtol=1e-6, atol=0, err_msg=what)


def route_one_token_calls(cfg, steps, xs_np):
    """ft_moe_route with T = 1 for every (step, layer), in call order."""
    L, k = cfg.layers, cfg.k
    shp = M.shape(L, cfg.E, k, cfg.d, cfg.f, cfg.fmt)
    st = torch.cuda.current_stream().cuda_stream
    xs = torch.stack([torch.from_numpy(x.view(np.int16)) for x in xs_np]).cuda()
    wr = torch.stack([torch.from_numpy(synth.router(cfg, l).view(np.int16)) for l in range(L)]).cuda()
    ids = torch.empty((L, steps, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, steps, k), dtype=torch.float32, device="cuda")
    for s in range(steps):
        for l in range(L):
            M.ft_moe_route(shp, xs[l, s].data_ptr(), wr[l].data_ptr(), 1, ids[l, s].data_ptr(), w[l, s].data_ptr(), st)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


@gpu
def test_route_decode_trace_full():
    cuda()
    cfg = synth.CONFIGS["decode"]
    steps = cfg.steps[0]
    xs_np = [synth.ar1_tokens(cfg, l, steps) for l in range(cfg.layers)]
    ids, w = route_one_token_calls(cfg, steps, xs_np)
    gap = np.inf
    for l in range(cfg.layers):
        ids_o, w_o, g = OR.route(xs_np[l], synth.router(cfg, l), cfg.k)
        gap = min(gap, g)
        check(ids[l], w[l], ids_o, w_o, f"decode layer {l}")
    print(f"decode trace: {cfg.layers * steps} calls bit-exact; smallest top-{cfg.k + 1} logit gap {gap:.3e}")


@gpu
def test_route_prefill_chunk_all_layers():
    cuda()
    cfg = synth.CONFIGS["prefill"]
    T, k = cfg.tokens[0], cfg.k
    x_np = synth.tokens(cfg, T, 7)
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    shp = M.shape(cfg.layers, cfg.E, k, cfg.d, cfg.f, "bf16")
    st = torch.cuda.current_stream().cuda_stream
    gap = np.inf
    for l in range(cfg.stream_layers):
        wr_np = synth.router(cfg, l)
        wr = torch.from_numpy(wr_np.view(np.int16)).cuda()
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), T, ids.data_ptr(), w.data_ptr(), st)
        torch.cuda.synchronize()
        ids_o, w_o, g = OR.route(x_np, wr_np, k)
        gap = min(gap, g)
        check(ids.cpu().numpy(), w.cpu().numpy(), ids_o, w_o, f"prefill layer {l}")
    print(f"prefill chunk: {cfg.stream_layers} layers x {T} tokens bit-exact; smallest gap {gap:.3e}")


@gpu
def test_route_mxfp4_config_all_layers():
    cuda()
    cfg = synth.CONFIGS["mxfp4"]
    L, k = cfg.layers, cfg.k
    Tp, steps = cfg.tokens[0], cfg.steps[1]
    st = torch.cuda.current_stream().cuda_stream
    shp = M.shape(L, cfg.E, k, cfg.d, cfg.f, "mxfp4")
    x_np = synth.tokens(cfg, Tp, 7)
    x = torch.from_numpy(x_np.view(np.int16)).cuda()
    gap = np.inf
    for l in range(L):
        wr_np = synth.router(cfg, l)
        wr = torch.from_numpy(wr_np.view(np.int16)).cuda()
        ids = torch.empty((Tp, k), dtype=torch.int32, device="cuda")
        w = torch.empty((Tp, k), dtype=torch.float32, device="cuda")
        M.ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), Tp, ids.data_ptr(), w.data_ptr(), st)
        torch.cuda.synchronize()
        ids_o, w_o, g = OR.route(x_np, wr_np, k)
        gap = min(gap, g)
        check(ids.cpu().numpy(), w.cpu().numpy(), ids_o, w_o, f"mxfp4 prefill layer {l}")
    xs_np = [synth.ar1_tokens(cfg, l, steps) for l in range(L)]
    ids, w = route_one_token_calls(cfg, steps, xs_np)
    for l in range(L):
        ids_o, w_o, g = OR.route(xs_np[l], synth.router(cfg, l), k)
        gap = min(gap, g)
        check(ids[l], w[l], ids_o, w_o, f"mxfp4 decode layer {l}")
    print(f"mxfp4: {L} layers x {Tp} prefill tokens and {L * steps} decode calls bit-exact; smallest gap {gap:.3e}")
