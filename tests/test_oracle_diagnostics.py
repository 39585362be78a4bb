"""Pins of the O1-O3 diagnostics oracle (oracle/diagnostics.py) against
closed forms that follow from the definitions (summary page, "Key
observations"), and against index sets produced by the indexer oracle whose
structure is known:

  * "newest positions" rows T_t = {max(0, t-k+1) .. t}: the adjacent overlap
    is min(t+1, k-1), the overlap at distance d is min(t+1, k-d) (>= 0), a
    group's union spans min(t_last+1, k+g-1) positions and its intersection
    max(0, min(t_first+1, k-g+1));
  * Reuse rows are identical within a group: union = intersection = the
    row's length, and the in-group overlaps equal it too;
  * disjoint rows: overlap 0, union = sum of lengths;
  * equal scores give mass j/n; scores 2^-i give (2 - 2^(1-j)) / (2 - 2^(1-n)).
A few planted mistakes must fail these pins.
"""
import numpy as np
import pytest

import oracle
from oracle import diagnostics as dg
from workloads import BF16, exact_random


def _newest_rows(Lq, k):
    idx = np.full((1, Lq, k), -1, dtype=np.int32)
    for t in range(Lq):
        lo = max(0, t - k + 1)
        idx[0, t, :t - lo + 1] = np.arange(lo, t + 1)
    return idx


@pytest.mark.parametrize("Lq,k,d", [(40, 8, 1), (40, 8, 3), (25, 16, 1), (30, 5, 4), (12, 3, 7)])
def test_overlap_closed_form_on_newest_rows(Lq, k, d):
    got = dg.overlap(_newest_rows(Lq, k), d)
    for t in range(Lq):
        want = max(0, min(t + 1, k - d)) if t + d < Lq else -1
        assert got[0, t] == want, (t, got[0, t], want)


@pytest.mark.parametrize("Lq,k,g", [(40, 8, 4), (41, 8, 3), (30, 5, 8), (16, 16, 4), (9, 2, 4)])
def test_group_sets_closed_form_on_newest_rows(Lq, k, g):
    union, inter = dg.group_sets(_newest_rows(Lq, k), g)
    for m in range(union.shape[1]):
        t0, tl = m * g, min((m + 1) * g, Lq) - 1
        gm = tl - t0 + 1
        assert union[0, m] == min(tl + 1, k + gm - 1)
        assert inter[0, m] == max(0, min(t0 + 1, k - gm + 1))


def test_reuse_rows_are_one_set_per_group():
    B, L, H, d, g, topk = 2, 37, 3, 8, 4, 6
    q, w, k = exact_random(3, B, L, L, H, d, BF16)
    idx = oracle.reuse(q, w, k, g, topk)["indices"]
    union, inter = dg.group_sets(idx, g)
    n = (idx >= 0).sum(-1)
    for b in range(B):
        for m in range(union.shape[1]):
            assert union[b, m] == inter[b, m] == n[b, m * g]
    ov = dg.overlap(idx, 1)
    for t in range(L - 1):
        if (t + 1) % g != 0:  # partner in the same group
            np.testing.assert_array_equal(ov[:, t], n[:, t])


def test_disjoint_rows():
    k, Lq, g = 6, 8, 4
    idx = np.arange(Lq * k, dtype=np.int32).reshape(1, Lq, k)
    idx[0, 3, 4:] = -1  # a short row
    ov = dg.overlap(idx, 1)
    assert np.all(ov[0, :-1] == 0) and ov[0, -1] == -1
    union, inter = dg.group_sets(idx, g)
    assert union[0, 0] == 3 * k + 4 and union[0, 1] == 4 * k
    assert np.all(inter == 0)


def test_mass_closed_forms():
    k = 16
    idx = np.tile(np.arange(k, dtype=np.int32), (1, 3, 1))
    sc = np.zeros((1, 3, k), dtype=np.float32)
    sc[0, 0] = 2.0                                      # equal scores
    sc[0, 1] = np.ldexp(1.0, -np.arange(k))[::-1]       # 2^-i, stored in ascending position
    idx[0, 2, 10:] = -1                                 # a row of n = 10 equal scores
    sc[0, 2] = 1.0
    m = dg.mass(idx, sc)
    for f, frac in enumerate(dg.FRACTIONS):
        j = int(frac * k)
        assert m[0, 0, f] == j / k
        assert m[0, 1, f] == pytest.approx((2 - 2.0 ** (1 - j)) / (2 - 2.0 ** (1 - k)), rel=1e-15)
        assert m[0, 2, f] == min(j, 10) / 10
    sc[0, 0] = 0.0
    assert np.all(np.isnan(dg.mass(idx[:, :1], sc[:, :1])))


MUTATIONS = [
    ("for t in range(Lq - d):", "for t in range(Lq - d - 1):"),            # drops the last pair
    ("u, i = set(), set(sets[0])", "u, i = set(), set()"),                  # empty intersection
    ("j = int(frac * k)", "j = int(frac * k) + 1"),                         # one entry too many
    ("return row[:n]", "return row[:n + 1] if n < row.shape[0] else row"),  # counts the -1 pad
    ("for s in sets:", "for s in sets[1:]:"),                               # union misses a member
]


def _mutant(old, new):
    import types
    src = open(dg.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("dg_mutant")
    exec(compile(src.replace(old, new), "dg_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("old,new", MUTATIONS)
def test_planted_mistakes_fail_the_pins(old, new, monkeypatch):
    pins = [lambda: test_overlap_closed_form_on_newest_rows(40, 8, 1),
            lambda: test_overlap_closed_form_on_newest_rows(30, 5, 4),
            lambda: test_group_sets_closed_form_on_newest_rows(41, 8, 3),
            lambda: test_group_sets_closed_form_on_newest_rows(9, 2, 4),
            test_disjoint_rows, test_mass_closed_forms, test_reuse_rows_are_one_set_per_group]
    import sys
    monkeypatch.setattr(sys.modules[__name__], "dg", _mutant(old, new))
    failed = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {new}"
