"""Decode-time expert miss rate versus cache capacity, replayed on identical
routing traces.

A trace holds the routed expert ids of every decode step and layer
(ids[step, layer, token, j]).  The same trace is replayed through four
placement policies, and each reports the miss rate: unique layer-experts of a
layer call that are not resident at that call, summed over calls, divided by
the unique layer-experts of all calls.

  freetoken  the library's control (ft_cache_classify on the GPU): global LRU
             residency over every layer, misses admitted by the q* split of
             the profile (host-run misses do not enter the cache);
  lru        the same control with every miss admitted (B_P = B_H gives
             q = m);
  prefill    a static placement chosen from a prompt: the C layer-experts the
             prompt's tokens routed to most often (ties to the lower flat id),
             frozen for the whole decode;
  load       a routing-blind static split fixed at load time: flat ids
             0 .. C-1 (whole layers in order), frozen.

The comparison and its method (miss rate over cache size as a share of the
expert pool, identical traces, LRU against a prefill-updated placement and a
routing-blind split) are those of "The Expert Cache That Follows the Router",
section "How residency follows demand without leaving the device", and of
Figure 4(b) of the FreeToken paper's figure list; "Making Large MoE Models
Practical on a Single Machine", sections 8 and 9, gives the engines' reported
rates; the txtmix article ("decode 的 cache miss 会让 PCIe 闲置") names the
static engines' rules (placement fixed at load; hot experts pinned).  The two
static policies are analysis models of those rules, not GPU code.
"""
import numpy as np

from . import ft_cache_classify, ft_cache_stats, shape as _shape, ft_record_bytes

CAPACITIES = (0.05, 0.10, 0.20, 0.30, 0.40, 0.50, 0.60)


# -- traces -------------------------------------------------------------------

def record_decode_trace(cfg, prompt_steps: int, steps: int):
    """Route the per-layer AR(1) hidden-state stream of `cfg` on the GPU
    (ft_moe_route).  Returns (prompt [P, L, k], decode [S, L, 1, k]) int32."""
    import torch
    import synth
    from . import ft_moe_route
    L, k, n = cfg.layers, cfg.k, prompt_steps + steps
    shp = _shape(L, cfg.E, k, cfg.d, cfg.f, cfg.fmt)
    stream = torch.cuda.current_stream().cuda_stream
    ids = torch.empty((L, n, k), dtype=torch.int32, device="cuda")
    w = torch.empty((L, n, k), dtype=torch.float32, device="cuda")
    for l in range(L):
        x = torch.from_numpy(synth.ar1_tokens(cfg, l, n).view(np.int16)).cuda()
        wr = torch.from_numpy(synth.router(cfg, l).view(np.int16)).cuda()
        ft_moe_route(shp, x.data_ptr(), wr.data_ptr(), n, ids[l].data_ptr(), w[l].data_ptr(), stream)
    torch.cuda.synchronize()
    a = ids.cpu().numpy().transpose(1, 0, 2)           # [n, L, k]
    return np.ascontiguousarray(a[:prompt_steps]), np.ascontiguousarray(a[prompt_steps:, :, None, :])


def record_zipf_trace(cfg, prompt_tokens: int, steps: int):
    """Zipf(1.1)-popularity routes of a one-layer config, one token per step.
    Returns (prompt [P, 1, k], decode [S, 1, 1, k]) int32."""
    import synth
    dec = np.stack([synth.zipf_routes(cfg, 1, s)[0] for s in range(steps)])        # [S, 1, k]
    prompt = synth.zipf_routes(cfg, prompt_tokens, 1 << 20)[0]                     # [P, k]
    return prompt[:, None, :].astype(np.int32), dec[:, None, :, :].astype(np.int32)


# -- static policies ----------------------------------------------------------

def load_time_placement(L: int, E: int, C: int) -> np.ndarray:
    """Routing-blind split: flat ids 0 .. C-1 resident."""
    r = np.zeros(L * E, dtype=bool)
    r[:max(0, min(C, L * E))] = True
    return r


def prefill_placement(prompt: np.ndarray, L: int, E: int, C: int) -> np.ndarray:
    """The C most-routed flat ids of a prompt (prompt [P, L, k] expert ids),
    ties to the lower flat id."""
    counts = np.zeros(L * E, dtype=np.int64)
    P = prompt.shape[0]
    flat = (np.arange(L, dtype=np.int64)[None, :, None] * E + prompt.reshape(P, L, -1)).reshape(-1)
    np.add.at(counts, flat, 1)
    order = np.lexsort((np.arange(L * E), -counts))     # count descending, then flat id ascending
    r = np.zeros(L * E, dtype=bool)
    r[order[:max(0, min(C, L * E))]] = True
    return r


def static_misses(trace: np.ndarray, E: int, resident: np.ndarray):
    """(misses, unique) of a frozen placement over a trace [S, L, T, k]."""
    S, L = trace.shape[:2]
    misses = unique = 0
    for s in range(S):
        for l in range(L):
            u = np.unique(trace[s, l].reshape(-1)).astype(np.int64) + l * E
            unique += u.size
            misses += int(np.count_nonzero(~resident[u]))
    return misses, unique


# -- the library's control ----------------------------------------------------

def gpu_control_misses(trace: np.ndarray, E: int, k: int, slots: int, bp_mbps: int, bh_mbps: int,
                       max_fetch: int = -1):
    """Replay a trace through ft_cache_classify on a cache of `slots` slots
    (records of the smallest shape: the control does not depend on d and f).
    Returns the cache's counters after the replay."""
    import torch
    from .tensors import PinnedBank, SlotCache
    S, L, T = trace.shape[:3]
    shp = _shape(L, E, k, 128, 128, "bf16")
    rb = ft_record_bytes(shp)
    bank = PinnedBank(L * E * rb)
    sc = SlotCache(L, E, k, 128, 128, "bf16", bank.ptr, slots, T, bp_mbps, bh_mbps, max_fetch)
    try:
        stream = torch.cuda.current_stream().cuda_stream
        dev = torch.from_numpy(np.ascontiguousarray(trace, dtype=np.int32)).cuda()
        work = torch.empty_like(dev)
        work.copy_(dev)                      # classify rewrites routes in place
        for s in range(S):
            for l in range(L):
                ft_cache_classify(sc.handle, l, work[s, l].data_ptr(), T, None, stream)
        st = ft_cache_stats(sc.handle).as_dict()
    finally:
        sc.close()
        bank.close()
    return st


def miss_table(prompt: np.ndarray, trace: np.ndarray, E: int, k: int, bp_mbps: int, bh_mbps: int,
               capacities=CAPACITIES, extra_slots=()):
    """Miss rate of every policy at each capacity (share of the L*E pool)."""
    L = trace.shape[1]
    pool = L * E
    sizes = sorted({max(1, int(round(c * pool))) for c in capacities} | set(extra_slots))
    rows = []
    for C in sizes:
        fr = gpu_control_misses(trace, E, k, C, bp_mbps, bh_mbps)
        lru = gpu_control_misses(trace, E, k, C, 1, 1)
        pm, pu = static_misses(trace, E, prefill_placement(prompt, L, E, C))
        lm, lu = static_misses(trace, E, load_time_placement(L, E, C))
        rows.append({
            "slots": C, "capacity": C / pool,
            "freetoken": fr["misses"] / fr["unique"], "lru": lru["misses"] / lru["unique"],
            "prefill": pm / pu, "load": lm / lu,
            "freetoken_fills": fr["fills"], "unique": fr["unique"],
        })
    return rows
