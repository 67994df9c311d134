"""Pins for the slot-cache simulator (CPU only)."""
from collections import OrderedDict

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.cache import CPU, FILL, HIT, SlotCacheSim
from oracle.qstar import fill_count


class TextbookLRU:
    """collections.OrderedDict LRU of fixed capacity (front = least recent)."""

    def __init__(self, cap):
        self.cap, self.d = cap, OrderedDict()

    def touch(self, u):
        self.d.move_to_end(u)

    def insert(self, u):
        ev = None
        if len(self.d) >= self.cap:
            ev, _ = self.d.popitem(last=False)
        self.d[u] = True
        return ev


def _calls(draw_layers, E, k, n, rng):
    out = []
    for _ in range(n):
        l = int(rng.integers(0, draw_layers))
        T = int(rng.integers(1, 4))
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
        out.append((l, ids))
    return out


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10 ** 6), N=st.integers(1, 12), E=st.integers(2, 9),
       L=st.integers(1, 3), bp=st.sampled_from([60000, 20000, 11800]), k=st.integers(1, 3))
def test_equals_textbook_lru(seed, N, E, L, bp, k):
    k = min(k, E)
    rng = np.random.default_rng(seed)
    sim = SlotCacheSim(L, E, N, bp, 60000)
    lru = TextbookLRU(N)
    for l, ids in _calls(L, E, k, 40, rng):
        r = sim.classify(l, ids)
        uniq = sorted({l * E + int(e) for e in ids.reshape(-1)})
        hits = [u for u in uniq if u in lru.d]
        misses = [u for u in uniq if u not in lru.d]
        for u in hits:
            lru.touch(u)
        evicted = []
        for u in misses[: r.q]:
            ev = lru.insert(u)
            if ev is not None:
                evicted.append(ev)
        assert r.hits == len(hits) and r.m == len(misses)
        assert [old for _, old, _ in r.evictions if old >= 0] == evicted
        assert set(sim.residents()) == set(lru.d)
        assert r.cpu == misses[r.q:]


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10 ** 6), N=st.integers(1, 10), E=st.integers(2, 8),
       bp=st.integers(1000, 90000), mf=st.sampled_from([-1, 0, 1, 2]))
def test_invariants(seed, N, E, bp, mf):
    rng = np.random.default_rng(seed)
    L, k = 2, min(2, E)
    sim = SlotCacheSim(L, E, N, bp, 60000, max_fetch=mf)
    last_clock = sim.clock
    for l, ids in _calls(L, E, k, 30, rng):
        sfi0, ios0, stamp0, clock0 = sim.arrays()
        res0 = set(sim.residents())
        r = sim.classify(l, ids)
        sfi, ios, stamp, clock = sim.arrays()
        # maps are mutual inverses
        for s, u in enumerate(ios):
            if u >= 0:
                assert sfi[u] == s
        for u, s in enumerate(sfi):
            if s >= 0:
                assert ios[s] == u
        assert len(sim.residents()) <= N
        # q follows the closed form and its clamps
        assert r.q == fill_count(r.m, r.hits, N, bp, 60000, mf)
        if r.m > 0 and N - r.hits > 0 and mf != 0:
            assert 1 <= r.q <= r.m
        # classes
        for u, c, s in zip(r.uniq, r.cls, r.slot):
            if c in (HIT, FILL):
                assert sfi[u] == s >= 0
            else:
                assert sfi[u] < 0 and u not in res0
            if c == HIT:
                assert u in res0
        # victims: exactly the q smallest (stamp, slot) keys among slots not hit
        hit_slots = {sfi0[u] for u, c in zip(r.uniq, r.cls) if c == HIT}
        keys = sorted((int(stamp0[s]), s) for s in range(N) if s not in hit_slots)
        assert [v for v, _, _ in r.evictions] == [s for _, s in keys[: r.q]]
        # no hit is evicted; CPU ids do not become resident
        assert all(old not in [u for u, c in zip(r.uniq, r.cls) if c == HIT] for _, old, _ in r.evictions)
        # stamps unique among residents, clock monotone and advanced by hits + q
        st_res = [int(stamp[s]) for s in range(N) if ios[s] >= 0]
        assert len(st_res) == len(set(st_res))
        assert clock == clock0 + r.hits + r.q and clock >= last_clock
        last_clock = clock
        # routes: slot or -(1 + e)
        for (t, j), e in np.ndenumerate(ids):
            u = l * E + int(e)
            assert r.routes[t, j] == (sfi[u] if u not in r.cpu else -(1 + int(e)))


def test_cold_start_then_hits():
    sim = SlotCacheSim(1, 8, 4, 25000, 50000)
    r = sim.classify(0, np.array([[0, 1], [2, 3]]))
    assert r.m == 4 and r.q == 2 and r.cls == [FILL, FILL, CPU, CPU]
    assert [v for v, _, _ in r.evictions] == [0, 1]          # empties, lowest slot first
    r = sim.classify(0, np.array([[1, 0]]))
    assert r.cls == [HIT, HIT] and r.q == 0 and r.routes.tolist() == [[1, 0]]


def test_stream_invalidation_clears_owners():
    E = 4
    sim = SlotCacheSim(3, E, 2 * E, 60000, 60000)
    r = sim.classify(0, np.array([[0, 1], [2, 3]]))
    assert sorted(v for v, _, _ in r.evictions) == [0, 1, 2, 3]
    sim.stream_load(1)          # layer 1 into buffer 1: slots 4..7 (empty)
    assert len(sim.residents()) == 4
    sim.stream_load(0)          # layer 2 into buffer 0: owners of slots 0..3 are cleared
    assert sim.residents() == {}
    assert all(s == 0 for s in sim.stamp)
    r = sim.classify(0, np.array([[0, 1]]))
    assert r.hits == 0 and r.m == 2
    with pytest.raises(ValueError):
        SlotCacheSim(1, 4, 7, 1, 1).stream_load(1)     # buffer 1 needs 2E slots
    with pytest.raises(ValueError):
        SlotCacheSim(1, 4, 3, 1, 1).stream_load(0)     # buffer 0 needs E
    SlotCacheSim(1, 4, 4, 1, 1).stream_load(0)         # the one-buffer variant


def _check_maps(sim):
    res = sim.residents()
    for u, s in res.items():
        assert sim.id_of_slot[s] == u
    for s, u in enumerate(sim.id_of_slot):
        assert u < 0 or sim.slot_for_id[u] == s
    stamps = [sim.stamp[s] for s in res.values()]
    assert len(set(stamps)) == len(stamps) and all(0 < t < sim.clock for t in stamps)


def test_warm_registers_the_streamed_layer_as_residents():
    E = 4
    sim = SlotCacheSim(3, E, 2 * E + 2, 60000, 60000)
    r = sim.classify(0, np.array([[0, 1]]))               # fills take slots 0, 1
    assert [v for v, _ in r.fills] == [0, 1] and sim.clock == 3
    sim.stream_load(1)                                    # layer 1 into buffer 1, then registered
    sim.register_buffer(1, 1)
    assert {u: sim.slot_for_id[u] for u in range(4, 8)} == {4: 4, 5: 5, 6: 6, 7: 7}
    assert [sim.stamp[s] for s in range(4, 8)] == [3, 4, 5, 6] and sim.clock == 7
    sim.stream_load(0)                                    # layer 2 into buffer 0 evicts layer 0's fills
    sim.register_buffer(0, 2)
    assert sim.slot_for_id[0] == sim.slot_for_id[1] == -1
    assert sim.residents() == {4: 4, 5: 5, 6: 6, 7: 7, 8: 0, 9: 1, 10: 2, 11: 3}
    _check_maps(sim)
    r = sim.classify(1, np.array([[0, 3]]))
    assert r.cls == [HIT, HIT] and r.slot == [4, 7]
    r = sim.classify(0, np.array([[0]]))                  # a miss: the empty slots 8, 9 go first
    assert r.cls == [FILL] and r.fills == [(8, 0)]
    _check_maps(sim)


def test_warm_skips_experts_resident_elsewhere():
    E = 4
    sim = SlotCacheSim(2, E, 2 * E + 1, 60000, 60000)
    sim.classify(1, np.array([[2]]))                      # layer 1 expert 2 (flat 6) filled into slot 0
    assert sim.slot_for_id[6] == 0
    sim.stream_load(1)
    clock = sim.clock
    sim.register_buffer(1, 1)
    assert sim.slot_for_id[6] == 0 and sim.id_of_slot[6] == -1 and sim.stamp[6] == 0
    assert [sim.slot_for_id[u] for u in (4, 5, 7)] == [4, 5, 7]
    assert sim.clock == clock + E
    sim.register_buffer(1, 1)                             # again: nothing new, the clock still advances
    assert sim.clock == clock + 2 * E and len(sim.residents()) == 4
    _check_maps(sim)


def test_resize_keeps_most_recent_packed():
    sim = SlotCacheSim(2, 8, 6, 60000, 60000)
    sim.classify(0, np.array([[0, 1, 2]]))
    sim.classify(1, np.array([[0, 1, 2]]))     # fills slots 3..5
    sim.classify(0, np.array([[1]]))           # refresh (layer 0, expert 1) in slot 1
    stamps = {u: sim.stamp[s] for u, s in sim.residents().items()}
    clock = sim.clock
    moves = sim.resize(3)
    kept = sorted(stamps, key=stamps.get, reverse=True)[:3]
    assert set(sim.residents()) == set(kept)
    assert sorted(sim.residents().values()) == [0, 1, 2]
    assert [o for o, _ in moves] == sorted(o for o, _ in moves)
    assert {u: sim.stamp[s] for u, s in sim.residents().items()} == {u: stamps[u] for u in kept}
    assert sim.clock == clock
    sim.resize(10)
    assert len(sim.residents()) == 3 and sim.N == 10
    r = sim.classify(0, np.array([[5, 6]]))
    assert r.q == 2 and all(v >= 3 for v, _, _ in r.evictions)   # new empty slots first


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10 ** 6), N=st.integers(1, 12), N2=st.integers(1, 12), E=st.integers(2, 9),
       L=st.integers(1, 3), k=st.integers(1, 3))
def test_resize_equals_textbook_lru_truncation(seed, N, N2, E, L, k):
    """Resize keeps exactly what a textbook LRU cut down to N2 entries keeps:
    the N2 most recently used entries of a collections.OrderedDict that saw
    the same accesses, in the same recency order; they are packed into slots
    0.. in ascending old-slot order; and the resized cache then goes on to
    behave as a textbook LRU of capacity N2 holding those entries."""
    k = min(k, E)
    rng = np.random.default_rng(seed)
    sim = SlotCacheSim(L, E, N, 60000, 60000)     # q = m while slots allow: every admitted miss is an insert

    def run(lru, n):
        for l, ids in _calls(L, E, k, n, rng):
            r = sim.classify(l, ids)
            uniq = sorted({l * E + int(e) for e in ids.reshape(-1)})
            for u in uniq:
                if u in lru.d:
                    lru.touch(u)
            evicted = [lru.insert(u) for u in [u for u in uniq if u not in lru.d][: r.q]]
            assert [old for _, old, _ in r.evictions if old >= 0] == [e for e in evicted if e is not None]
            assert set(sim.residents()) == set(lru.d)

    lru = TextbookLRU(N)
    run(lru, 30)
    before = {u: s for u, s in sim.residents().items()}
    keep = list(lru.d)[-N2:]                       # the N2 most recent, least recent first
    moves = sim.resize(N2)
    assert set(sim.residents()) == set(keep)
    assert sorted(sim.residents(), key=lambda u: sim.stamp[sim.slot_for_id[u]]) == keep
    assert sorted(sim.residents().values()) == list(range(len(keep)))
    assert [o for o, _ in moves] == sorted(before[u] for u in keep)
    lru2 = TextbookLRU(N2)
    for u in keep:
        lru2.d[u] = True
    run(lru2, 30)
