"""Miss-rate replay (placement policies on identical routing traces).

CPU: the two static placements and their miss counting, on traces small enough
to work out by hand.  GPU: the library's control replayed over whole traces
gives exactly the counters of the oracle's LRU simulator fed the same calls."""
import numpy as np
import pytest

from moe_expert_execution_amd import replay as R


def test_load_time_placement_takes_the_first_flat_ids():
    r = R.load_time_placement(2, 4, 3)
    assert r.tolist() == [True, True, True, False, False, False, False, False]
    assert R.load_time_placement(2, 4, 0).sum() == 0
    assert R.load_time_placement(2, 4, 99).all()


def test_prefill_placement_pins_the_most_routed_ids_ties_to_lower():
    # L = 2, E = 4, k = 2; prompt of 3 tokens
    prompt = np.array([[[1, 2], [0, 3]],
                       [[2, 1], [3, 2]],
                       [[2, 0], [3, 1]]], dtype=np.int32)
    # layer 0 counts: e0 1, e1 2, e2 3, e3 0 -> flat 0:1 1:2 2:3 3:0
    # layer 1 counts: e0 1, e1 1, e2 1, e3 3 -> flat 4:1 5:1 6:1 7:3
    assert np.flatnonzero(R.prefill_placement(prompt, 2, 4, 1)).tolist() == [2]
    assert np.flatnonzero(R.prefill_placement(prompt, 2, 4, 3)).tolist() == [1, 2, 7]
    # next: counts 1 at flat 0, 4, 5, 6 -> the lowest flat id first
    assert np.flatnonzero(R.prefill_placement(prompt, 2, 4, 4)).tolist() == [0, 1, 2, 7]


def test_static_misses_counts_unique_layer_experts_per_call():
    E = 4
    trace = np.array([[[[0, 1]], [[2, 2]]],          # step 0: layer 0 {0,1}, layer 1 {2}
                      [[[1, 3]], [[0, 1]]]],         # step 1: layer 0 {1,3}, layer 1 {0,1}
                     dtype=np.int32)                 # [S=2, L=2, T=1, k=2]
    resident = np.zeros(8, dtype=bool)
    resident[[1, 4 + 2]] = True                      # flat 1 (L0 e1) and flat 6 (L1 e2)
    m, u = R.static_misses(trace, E, resident)
    assert u == 2 + 1 + 2 + 2
    assert m == 1 + 0 + 1 + 2


def _locality_trace(rng, S, L, E, k, T=1, stay=0.8):
    """ids with temporal locality: each (layer, token, j) keeps its previous
    expert with probability `stay`; duplicates inside a token are avoided."""
    tr = np.empty((S, L, T, k), dtype=np.int32)
    cur = np.stack([np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]) for _ in range(L)])
    for s in range(S):
        for l in range(L):
            for t in range(T):
                row = cur[l, t].copy()
                for j in range(k):
                    if rng.random() > stay:
                        free = np.setdiff1d(np.arange(E), row)
                        row[j] = rng.choice(free)
                cur[l, t] = row
        tr[s] = cur
    return tr


@pytest.mark.gpu
@pytest.mark.parametrize("L,E,k,T,slots,bp,bh", [(3, 16, 4, 1, 8, 20, 60), (3, 16, 4, 1, 8, 1, 1),
                                                 (2, 64, 8, 2, 23, 20, 60), (4, 32, 2, 1, 1, 25, 50)])
def test_gpu_replay_counters_equal_the_oracle_simulator(L, E, k, T, slots, bp, bh):
    from oracle import cache as OC
    rng = np.random.default_rng(1234 + L * E + slots)
    trace = _locality_trace(rng, 60, L, E, k, T)
    st = R.gpu_control_misses(trace, E, k, slots, bp, bh)
    sim = OC.SlotCacheSim(L, E, slots, bp, bh)
    tot = dict(unique=0, hits=0, misses=0, fills=0, cpu=0, evictions=0)
    for s in range(trace.shape[0]):
        for l in range(L):
            r = sim.classify(l, trace[s, l])
            tot["unique"] += len(r.uniq)
            tot["hits"] += r.hits
            tot["misses"] += r.m
            tot["fills"] += r.q
            tot["cpu"] += r.m - r.q
            tot["evictions"] += sum(1 for _, old, _ in r.evictions if old >= 0)
    got = dict(unique=st["unique"], hits=st["hits"], misses=st["misses"], fills=st["fills"],
               cpu=st["cpu_experts"], evictions=st["evictions"])
    assert got == tot
    assert st["calls"] == trace.shape[0] * L and st["error_flags"] == 0


@pytest.mark.gpu
def test_gpu_replay_of_the_decode_trace_runs_every_policy():
    import synth
    cfg = synth.CONFIGS["decode"]
    prompt, trace = R.record_decode_trace(cfg.with_(layers=4), 16, 24)
    assert prompt.shape == (16, 4, cfg.k) and trace.shape == (24, 4, 1, cfg.k)
    assert trace.min() >= 0 and trace.max() < cfg.E
    rows = R.miss_table(prompt, trace, cfg.E, cfg.k, cfg.bp_mbps, cfg.bh_mbps, capacities=(0.1, 0.5))
    for row in rows:
        for p in ("freetoken", "lru", "prefill", "load"):
            assert 0.0 <= row[p] <= 1.0
    # a cache of the whole pool misses only on first touch
    full = R.gpu_control_misses(trace, cfg.E, cfg.k, 4 * cfg.E, 1, 1)
    assert full["misses"] == len({(l, e) for l in range(4) for e in np.unique(trace[:, l])})
