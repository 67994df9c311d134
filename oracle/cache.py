"""Slot-cache simulator: the control decisions of one MoE layer call.

State ("The Expert Cache That Follows the Router", section "One logical expert,
two physical levels of memory"): a flat logical id i = layer * E + expert, a
map slot_for_id[L*E] (where a logical record lives, -1 absent) and its inverse
id_of_slot[N] (which record owns a slot, -1 empty), plus LRU recency.

One call ("How residency follows demand without leaving the device" on the same
page; hyper.ai summary, section 方法; txtmix article, section "CUDA-graph 兼容的
LRU 缓存"): deduplicate the routed experts, classify each unique id as a hit or
a miss against slot_for_id, derive the fill count q, refresh the hits'
recency, choose LRU victims for the q fills (one scan of the slots yields the
candidates and the fills take the first q), record (victim slot, source row)
per fill, and rewrite the routes into physical slot ids.  Misses that are not
filled run on the host from the host bank and leave residency unchanged
(same page, last section before the close).

Readings where the pages are silent (each is a choice of this reference):
  * unique ids are taken in ascending flat-id order; hits and misses keep it;
  * the fills are the first q misses in that order;
  * recency is a per-slot stamp from a clock that starts at 1; the r-th hit
    gets clock + r, the i-th fill clock + hits + i, then clock += hits + q
    (one stamp per access: hits ascending, then fills ascending);
  * victims are the q smallest (stamp, slot) among slots not hit in this call
    (empty slots have stamp 0, so they go first, lowest slot first); a call
    never evicts its own hits;
  * the i-th fill takes the i-th victim;
  * a CPU-executed miss does not touch recency;
  * a route is rewritten to its slot (hit or fill) or to -(1 + expert) when it
    runs on the host.

Full-layer buffers ("The Expert Cache That Follows the Router", paragraph on
prefill buffers, and the hostile-sequence paragraph): buffer b is slots
[b*E, (b+1)*E); loading a layer into it clears the old owners' maps and
recency.  Streamed contents are not registered as residents, except in the
prefill-warms-decode variant (register_buffer).

Resize (METAL MEDIA summary item 4; hyper.ai 方法, elastic lifetime): at a safe
point the cache is rebuilt for a new slot count.  Reading: keep the
min(N', residents) most recent entries, packed into slots 0.. in ascending old
slot order, with their stamps; the clock is unchanged.
"""
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

from .qstar import fill_count

HIT, FILL, CPU = 0, 1, 2


@dataclass
class ClassifyResult:
    uniq: List[int]                  # ascending unique flat ids
    cls: List[int]                   # HIT / FILL / CPU per unique id
    slot: List[int]                  # slot per unique id, -1 for CPU
    hits: int
    m: int
    q: int
    evictions: List[Tuple[int, int, int]]   # (victim slot, old flat id or -1, new flat id)
    fills: List[Tuple[int, int]]            # (victim slot, source flat id) in fill order
    cpu: List[int]                          # flat ids run on the host
    routes: np.ndarray                      # [T x k] int32: slot or -(1 + expert)


class SlotCacheSim:
    def __init__(self, layers: int, E: int, slots: int, bp_mbps: int, bh_mbps: int, max_fetch: int = -1):
        if slots < 1:
            raise ValueError("slots must be >= 1")
        self.L, self.E, self.N = layers, E, slots
        self.bp, self.bh, self.max_fetch = bp_mbps, bh_mbps, max_fetch
        self.slot_for_id = [-1] * (layers * E)
        self.id_of_slot = [-1] * slots
        self.stamp = [0] * slots
        self.clock = 1
        self.calls = 0

    # -- one layer call -------------------------------------------------
    def classify(self, layer: int, ids) -> ClassifyResult:
        ids = np.asarray(ids)
        if not (0 <= layer < self.L):
            raise ValueError("layer out of range")
        if ids.size and (ids.min() < 0 or ids.max() >= self.E):
            raise ValueError("expert id out of range")
        E = self.E
        uniq = sorted({layer * E + int(e) for e in ids.reshape(-1)})
        hits = [u for u in uniq if self.slot_for_id[u] >= 0]
        misses = [u for u in uniq if self.slot_for_id[u] < 0]
        h, m = len(hits), len(misses)
        q = fill_count(m, h, self.N, self.bp, self.bh, self.max_fetch)

        clock = self.clock
        hit_slots = set()
        for r, u in enumerate(hits):
            s = self.slot_for_id[u]
            self.stamp[s] = clock + r
            hit_slots.add(s)
        # one scan over the slots gives the candidates; the fills take the first q
        cand = sorted((self.stamp[s], s) for s in range(self.N) if s not in hit_slots)
        victims = [s for _, s in cand[:q]]
        assert len(victims) == q

        evictions, fills = [], []
        for i, u in enumerate(misses[:q]):
            v = victims[i]
            old = self.id_of_slot[v]
            if old >= 0:
                self.slot_for_id[old] = -1
            self.id_of_slot[v] = u
            self.slot_for_id[u] = v
            self.stamp[v] = clock + h + i
            evictions.append((v, old, u))
            fills.append((v, u))
        self.clock = clock + h + q
        self.calls += 1

        cpu = misses[q:]
        filled = {u for _, u in fills}
        cls, slot = [], []
        for u in uniq:
            if self.slot_for_id[u] >= 0 and u not in filled:
                cls.append(HIT)
            elif u in filled:
                cls.append(FILL)
            else:
                cls.append(CPU)
            slot.append(self.slot_for_id[u] if cls[-1] != CPU else -1)
        where = dict(zip(uniq, slot))
        routes = np.empty(ids.shape, dtype=np.int32)
        for pos, e in np.ndenumerate(ids):
            s = where[layer * E + int(e)]
            routes[pos] = s if s >= 0 else -(1 + int(e))
        return ClassifyResult(uniq, cls, slot, h, m, q, evictions, fills, cpu, routes)

    # -- full-layer buffers ----------------------------------------------
    def buffer_slots(self, buf: int) -> range:
        """Slots of full-layer buffer `buf` (buffer 1 exists only with >= 2E
        slots; the one-buffer variant uses buffer 0 alone and needs >= E)."""
        if buf not in (0, 1):
            raise ValueError("buffer must be 0 or 1")
        if self.N < (buf + 1) * self.E:
            raise ValueError("full-layer buffer %d needs at least %d slots" % (buf, (buf + 1) * self.E))
        return range(buf * self.E, (buf + 1) * self.E)

    def stream_load(self, buf: int) -> None:
        """Invalidate buffer `buf` before a full layer is copied into it."""
        for s in self.buffer_slots(buf):
            old = self.id_of_slot[s]
            if old >= 0:
                self.slot_for_id[old] = -1
            self.id_of_slot[s] = -1
            self.stamp[s] = 0

    def register_buffer(self, buf: int, layer: int) -> None:
        """Prefill-warms-decode variant (a reading: the pages keep buffer
        contents volatile, and also say a full-layer prefill may warm experts
        for the next phase): after `layer` was computed from buffer `buf`,
        expert e (ascending) becomes a resident in slot buf*E + e with stamp
        clock + e, unless it is already resident elsewhere or the slot is
        taken; then the clock advances by E."""
        E = self.E
        for e, s in enumerate(self.buffer_slots(buf)):
            u = layer * E + e
            if self.slot_for_id[u] < 0 and self.id_of_slot[s] < 0:
                self.slot_for_id[u] = s
                self.id_of_slot[s] = u
                self.stamp[s] = self.clock + e
        self.clock += E

    # -- elastic resize ----------------------------------------------------
    def resize(self, new_slots: int) -> List[Tuple[int, int]]:
        """Rebuild for `new_slots`; returns the (old slot, new slot) moves."""
        if new_slots < 1:
            raise ValueError("slots must be >= 1")
        res = [s for s in range(self.N) if self.id_of_slot[s] >= 0]
        keep = sorted(res, key=lambda s: self.stamp[s], reverse=True)[:new_slots]
        keep.sort()
        sfi = [-1] * (self.L * self.E)
        ios = [-1] * new_slots
        st = [0] * new_slots
        moves = []
        for ns, os_ in enumerate(keep):
            u = self.id_of_slot[os_]
            ios[ns], st[ns], sfi[u] = u, self.stamp[os_], ns
            moves.append((os_, ns))
        self.slot_for_id, self.id_of_slot, self.stamp, self.N = sfi, ios, st, new_slots
        return moves

    # -- views ---------------------------------------------------------------
    def residents(self):
        return {u: s for u, s in enumerate(self.slot_for_id) if s >= 0}

    def arrays(self):
        return (np.asarray(self.slot_for_id, dtype=np.int32), np.asarray(self.id_of_slot, dtype=np.int32),
                np.asarray(self.stamp, dtype=np.uint64), self.clock)
