"""Pins for the fill count q (CPU only)."""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.qstar import fill_count

GOLD = os.path.join(os.path.dirname(__file__), "golden")
BIG = 10 ** 6   # slots: never the binding clamp here


def _rows():
    for l in open(os.path.join(GOLD, "qstar_page_examples.txt")):
        if l.strip() and not l.startswith("#"):
            m, bp, bh, lo, hi, cite = l.split()
            yield int(m), int(bp), int(bh), int(lo), int(hi), cite


@pytest.mark.parametrize("m,bp,bh,lo,hi,cite", list(_rows()))
def test_page_examples(m, bp, bh, lo, hi, cite):
    q = fill_count(m, 0, BIG, bp, bh)
    assert lo <= q <= hi, cite
    assert 0 <= m - q  # the rest run on the host


def _balance_point(m, bp, bh):
    """Solve T_fill(q) = T_cpu(q) by bisection on the two branch times the
    blog's section 5 defines: T_fill = q S / B_P, T_cpu = (m - q) S / (B_H - B_P)."""
    S = 1.0
    lo, hi = 0.0, float(m)
    for _ in range(200):
        mid = (lo + hi) / 2
        if mid * S / bp < (m - mid) * S / (bh - bp):
            lo = mid
        else:
            hi = mid
    return (lo + hi) / 2


def test_rounded_balance_point_random():
    rng = np.random.default_rng(7)
    n = 0
    while n < 2000:
        m = int(rng.integers(1, 300))
        bp = int(rng.integers(1000, 80000))
        bh = int(rng.integers(bp + 1, 200000))
        qb = _balance_point(m, bp, bh)
        if abs(qb - np.floor(qb) - 0.5) < 1e-6:
            continue   # exact half: covered by the explicit tie cases
        want = min(max(int(np.floor(qb + 0.5)), 1), m)
        assert fill_count(m, 0, BIG, bp, bh) == want, (m, bp, bh, qb)
        n += 1


def test_half_ties_round_up():
    # m * B_P / B_H exactly k + 1/2
    assert fill_count(6, 0, BIG, 1000, 4000) == 2     # 1.5 -> 2
    assert fill_count(10, 0, BIG, 1000, 4000) == 3    # 2.5 -> 3
    assert fill_count(2, 0, BIG, 1000, 4000) == 1     # 0.5 -> 1


def test_bh_below_bp_fills_everything():
    for m in range(1, 20):
        assert fill_count(m, 0, BIG, 60000, 30000) == m


def test_clamps():
    assert fill_count(0, 3, 8, 20000, 60000) == 0
    assert fill_count(8, 6, 8, 60000, 60000) == 2        # only 2 evictable slots
    assert fill_count(8, 8, 8, 60000, 60000) == 0        # none evictable: no fill possible
    assert fill_count(8, 0, 8, 20000, 60000, max_fetch=0) == 0
    assert fill_count(8, 0, 8, 60000, 60000, max_fetch=2) == 2
    assert fill_count(8, 0, 8, 20000, 60000, max_fetch=-1) == 3   # round(8/3) = 3


def test_monotone_in_misses():
    for bp, bh in [(20000, 60000), (25000, 50000), (11800, 47500), (52700, 77300)]:
        qs = [fill_count(m, 0, BIG, bp, bh) for m in range(0, 200)]
        assert all(b - a in (0, 1) for a, b in zip(qs, qs[1:]))
        assert all(abs(q - Fraction(m * bp, bh)) <= Fraction(1, 2) or q == 1 for m, q in enumerate(qs) if m)
