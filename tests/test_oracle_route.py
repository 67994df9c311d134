"""Pins for the oracle's top-k softmax routing (CPU only)."""
import itertools
from fractions import Fraction

import numpy as np
import scipy.special
import torch

import synth
from oracle import route as R
from oracle.formats import bf16_to_f64


def _exact_logits(x, wr):
    xf = bf16_to_f64(x)
    wf = bf16_to_f64(wr)
    T, d = xf.shape
    E = wf.shape[1]
    return [[sum(Fraction(float(xf[t, i])) * Fraction(float(wf[i, e])) for i in range(d)) for e in range(E)]
            for t in range(T)]


def test_topk_is_brute_force_best_subset_tiny():
    c = synth.CONFIGS["tiny"]
    x = synth.tokens(c, 16, 0)
    wr = synth.router(c, 0)
    ids, w, gap = R.route(x, wr, c.k)
    Z = _exact_logits(x, wr)
    for t in range(16):
        z = Z[t]
        best = max(itertools.combinations(range(c.E), c.k), key=lambda s: (sum(z[e] for e in s), [-e for e in s]))
        assert set(ids[t].tolist()) == set(best)
        chosen = [z[e] for e in ids[t]]
        assert all(chosen[i] >= chosen[i + 1] for i in range(c.k - 1))
        assert min(chosen) >= max(z[e] for e in range(c.E) if e not in best)
    assert gap > 0


def test_fp64_logits_equal_exact_sums_tiny():
    c = synth.CONFIGS["tiny"]
    x = synth.tokens(c, 4, 3)
    wr = synth.router(c, 0)
    z = R.logits(x, wr)
    Z = _exact_logits(x, wr)
    prod_abs = np.abs(bf16_to_f64(x)) @ np.abs(bf16_to_f64(wr))
    for t in range(4):
        for e in range(c.E):
            # standard bound for an fp64 sum of exact products: (d - 1) * 2^-53 * sum |p_i|
            bound = Fraction(c.d - 1, 2 ** 53) * Fraction(float(prod_abs[t, e])) * 2
            assert abs(Fraction(float(z[t, e])) - Z[t][e]) <= bound


def test_ties_go_to_lower_expert():
    d, E = 128, 8
    x = synth.f32_to_bf16(np.ones((2, d), np.float32))
    wr_f = np.zeros((d, E), np.float32)
    wr_f[:, 5] = 0.5
    wr_f[:, 2] = 0.5          # experts 2 and 5 tie
    wr_f[:, 7] = 0.25
    ids, w, _ = R.route(x, synth.f32_to_bf16(wr_f), 3)
    assert ids[0].tolist() == [2, 5, 7]
    assert w[0, 0] == w[0, 1]


def test_softmax_over_all_experts_is_library_softmax():
    c = synth.CONFIGS["tiny"]
    x = synth.tokens(c, 16, 1)
    wr = synth.router(c, 0)
    ids, w, _ = R.route(x, wr, c.E)          # k = E: renormalised top-k = full softmax
    z = R.logits(x, wr)
    ref = scipy.special.softmax(z, axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w.astype(np.float64), axis=1)
    assert np.allclose(got, ref, rtol=1e-6, atol=0)
    ref_t = torch.softmax(torch.from_numpy(z), dim=1).numpy()
    assert np.allclose(got, ref_t, rtol=1e-6, atol=0)


def test_weights_sum_to_one_and_follow_logit_order():
    c = synth.CONFIGS["decode"]
    x = synth.tokens(c, 64, 0)
    ids, w, _ = R.route(x, synth.router(c, 0), c.k)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert all(len(set(r)) == c.k for r in ids.tolist())
