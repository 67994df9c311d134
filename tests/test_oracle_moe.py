"""Pins for the oracle's SwiGLU expert FFN and weighted combine (CPU only)."""
import math

import numpy as np

import synth
from oracle import formats as F, route as R
from oracle.cache import SlotCacheSim, CPU
from oracle.moe import ffn, moe_layer, moe_layer_partitioned


def _bf(a):
    return synth.f32_to_bf16(np.asarray(a, np.float32))


def test_one_hot_closed_form():
    """x = e_0; the gate/up columns carry chosen pre-activations; silu has exact
    closed forms at 0 and +-ln 3 (sigmoid(ln 3) = 3/4)."""
    d, f = 8, 4
    ln3 = math.log(3.0)
    a = np.array([0.0, ln3, -ln3, 2 * ln3])      # gate pre-activations
    b = np.array([5.0, 2.0, -4.0, 0.5])          # up pre-activations
    Wg = np.zeros((d, f)); Wg[0] = a
    Wu = np.zeros((d, f)); Wu[0] = b
    Wd = np.zeros((f, d))
    Wd[0, 1] = 7.0; Wd[1, 2] = 1.0; Wd[2, 3] = 1.0; Wd[3, 4] = 1.0
    x = np.zeros((1, d)); x[0, 0] = 1.0
    y = ffn(x, Wg, Wu, Wd)[0]
    silu = {0: 0.0, 1: 0.75 * ln3, 2: -0.25 * ln3, 3: 2 * ln3 * 0.9}   # sigmoid(2 ln 3) = 9/10
    want = np.zeros(d)
    want[1] = 7.0 * silu[0] * b[0]
    want[2] = silu[1] * b[1]
    want[3] = silu[2] * b[2]
    want[4] = silu[3] * b[3]
    assert np.allclose(y, want, rtol=1e-15, atol=1e-15)
    # swapping gate and up gives a different answer (the roles are pinned)
    assert not np.allclose(ffn(x, Wu, Wg, Wd)[0], want)


def test_weighted_combine_of_two_experts():
    d, f = 8, 4
    ln3 = math.log(3.0)
    experts = {}
    for e, (col, up) in enumerate([(1, 2.0), (2, -3.0), (3, 1.0)]):
        Wg = np.zeros((d, f)); Wg[0, 0] = ln3
        Wu = np.zeros((d, f)); Wu[0, 0] = up
        Wd = np.zeros((f, d)); Wd[0, col] = 1.0
        experts[e] = (Wg, Wu, Wd)
    x = _bf(np.eye(1, d))
    ids = np.array([[1, 0]])
    w = np.array([[0.75, 0.25]], np.float32)
    y = moe_layer(x, ids, w, experts.__getitem__)
    h = 0.75 * ln3
    want = np.zeros((1, d))
    want[0, 2] = 0.75 * h * -3.0
    want[0, 1] = 0.25 * h * 2.0
    assert np.allclose(y, want, rtol=1e-15, atol=1e-15)


def _brute(x_bits, ids, w, experts):
    x = [[float(v) for v in row] for row in F.bf16_to_f64(x_bits)]
    T, k = ids.shape
    d = len(x[0])
    out = [[0.0] * d for _ in range(T)]
    for t in range(T):
        for j in range(k):
            Wg, Wu, Wd = experts(int(ids[t, j]))
            f = Wg.shape[1]
            h = []
            for n in range(f):
                g = sum(x[t][i] * Wg[i, n] for i in range(d))
                u = sum(x[t][i] * Wu[i, n] for i in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for c in range(d):
                out[t][c] += float(w[t, j]) * sum(h[n] * Wd[n, c] for n in range(f))
    return np.array(out)


def test_brute_force_tiny_random():
    rng = np.random.default_rng(3)
    d, f, E, k, T = 8, 4, 3, 2, 3
    ex = {e: (rng.normal(0, 0.5, (d, f)), rng.normal(0, 0.5, (d, f)), rng.normal(0, 0.5, (f, d))) for e in range(E)}
    x = _bf(rng.normal(0, 1, (T, d)))
    ids = np.array([[0, 2], [1, 0], [2, 1]])
    w = np.array([[0.6, 0.4], [0.3, 0.7], [0.5, 0.5]], np.float32)
    y = moe_layer(x, ids, w, ex.__getitem__)
    assert np.allclose(y, _brute(x, ids, w, ex.__getitem__), rtol=1e-12, atol=1e-14)


def test_linearity_in_down_projection_and_weights():
    c = synth.CONFIGS["tiny"]
    x = synth.tokens(c, 16, 0)
    ids, w, _ = R.route(x, synth.router(c, 0), c.k)
    ex = lambda e: F.decode_record(synth.record(c, 0, e), "bf16", c.d, c.f)
    ex2 = lambda e: (lambda g, u, dn: (g, u, 2.0 * dn))(*ex(e))
    y = moe_layer(x, ids, w, ex)
    assert np.array_equal(moe_layer(x, ids, w, ex2), 2.0 * y)
    w1 = np.zeros_like(w); w1[:, 0] = 1.0
    y1 = moe_layer(x, ids, w1, ex)
    for t in range(16):
        Wg, Wu, Wd = ex(int(ids[t, 0]))
        assert np.allclose(y1[t], ffn(F.bf16_to_f64(x[t:t + 1]), Wg, Wu, Wd)[0], rtol=1e-14, atol=1e-16)


def test_partition_identity_across_profiles():
    """The float output does not depend on how misses split between fills and
    host execution: the same calls under three profiles give the same y."""
    c = synth.CONFIGS["tiny"]
    wr = synth.router(c, 0)
    ex = lambda e: F.decode_record(synth.record(c, 0, e), "bf16", c.d, c.f)
    profiles = [(25000, 50000, -1), (1000, 1000, -1), (25000, 50000, 0)]
    sims = [SlotCacheSim(1, c.E, c.slots, bp, bh, mf) for bp, bh, mf in profiles]
    saw_cpu = saw_fill = False
    for step in range(8):
        x = synth.tokens(c, 16, 100 + step)
        ids, w, _ = R.route(x, wr, c.k)
        ref = moe_layer(x, ids, w, ex)
        for sim in sims:
            r = sim.classify(0, ids)
            host = {u - 0 * c.E for u in r.cpu}
            saw_cpu |= bool(host)
            saw_fill |= r.q > 0
            y = moe_layer_partitioned(x, ids, w, ex, lambda e: e in host)
            assert np.allclose(y, ref, rtol=1e-13, atol=1e-16)
            if not host:
                assert np.array_equal(y, ref)
    assert saw_cpu and saw_fill


def test_hostile_invalidation_sequence():
    """'The Expert Cache That Follows the Router': one request uses layer-0
    experts, another streams other layers through every slot, then the first
    routes back.  Simulated slot bytes must be re-filled from layer 0's bank;
    a stale map would read layer-2 weights."""
    c = synth.CONFIGS["tiny"].with_(layers=3, E=4, k=2, slots=8, bp_mbps=60000, bh_mbps=60000)
    bank = synth.bank(c)                       # [3*4 x S]
    sim = SlotCacheSim(3, c.E, c.slots, c.bp_mbps, c.bh_mbps)
    slot_bytes = [None] * c.slots

    def run(layer, ids, x, w):
        r = sim.classify(layer, ids)
        for v, u in r.fills:
            slot_bytes[v] = bank[u].copy()
        routes = r.routes

        def gpu_or_host(e_route):
            if e_route >= 0:
                return F.decode_record(slot_bytes[e_route], "bf16", c.d, c.f)
            return F.decode_record(bank[layer * c.E + (-e_route - 1)], "bf16", c.d, c.f)
        # evaluate through the physical routes
        y = moe_layer(x, routes + 100, w, lambda rr: gpu_or_host(rr - 100))
        return r, y

    x = synth.tokens(c, 2, 0)
    ids = np.array([[0, 1], [2, 3]])
    w = np.array([[0.5, 0.5], [0.25, 0.75]], np.float32)
    ref = moe_layer(x, ids, w, lambda e: F.decode_record(bank[e], "bf16", c.d, c.f))
    r, y = run(0, ids, x, w)
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-16)
    # request B: layers 1 and 2 streamed into buffers 1 and 0 (every slot)
    for layer in (1, 2):
        b = layer % 2
        sim.stream_load(b)
        for e, s in enumerate(sim.buffer_slots(b)):
            slot_bytes[s] = bank[layer * c.E + e].copy()
    r, y = run(0, ids, x, w)
    assert r.hits == 0 and r.m == 4 and r.q == 4
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-16)
    # what a stale map would have read: layer-2 weights in slots 0..3
    stale = moe_layer(x, ids, w, lambda e: F.decode_record(bank[2 * c.E + e], "bf16", c.d, c.f))
    assert np.abs(stale - ref).max() > 0.1 * np.abs(ref).max()
