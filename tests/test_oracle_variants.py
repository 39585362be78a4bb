"""Pins of the oracle's variant knobs: the first / last-query proxy (section
"Ablation Studies", proxy aggregation) and member-causal Reuse (eq. (6) with
each member's own bound s <= t).

Each is checked against the float64 brute force (written independently: whole
score matrices and lexsort), and against special cases that reduce a knob to
another oracle path computed differently:
  * a last-member proxy scores exactly like that member's dense row, and a
    first-member proxy like the dense row of a query carrying the first
    member's q and w at the group's last position;
  * every knob collapses onto dense when g = 1;
  * member-causal Reuse agrees with plain Reuse on each group's last member
    and is the dense-like top-k of the proxy row truncated at t.
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from tests import checks
from workloads import BF16, F32, exact_random, gauss_random

CASES = [
    # B, Lq, Lk, H, d, g, topk, c, dtype
    (1, 24, 24, 2, 4, 4, 5, 9, F32),
    (1, 37, 37, 3, 5, 4, 6, 11, BF16),      # ragged last group
    (2, 19, 19, 2, 8, 3, 4, 7, BF16),       # g = 3
    (1, 4, 40, 3, 6, 4, 7, 12, BF16),       # decode shape
    (2, 6, 33, 2, 4, 3, 5, 10, BF16),       # two decode groups per sequence
    (1, 17, 17, 1, 3, 16, 4, 8, BF16),      # g > half of L
]


def _data(case, seed=0):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    return exact_random(seed, B, Lq, Lk, H, d, dt)


@pytest.mark.parametrize("agg", ["first", "last"])
@pytest.mark.parametrize("case", CASES)
def test_member_proxy_matches_brute_force_bitwise(case, agg):
    """A member proxy involves no arithmetic, so even odd group sizes stay
    exact: Reuse and Refine must equal the float64 brute force bit for bit."""
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    o = oracle.reuse(q, w, k, g, topk, agg=agg)
    bi, bs = brute.reuse(q, w, k, g, topk, dt, agg=agg)
    np.testing.assert_array_equal(o["indices"], bi)
    np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
    o = oracle.refine(q, w, k, g, topk, c, agg=agg)
    bi, bs, bc = brute.refine(q, w, k, g, topk, c, dt, agg=agg)
    np.testing.assert_array_equal(o["indices"], bi)
    np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
    G = o["cand"].shape[1]
    for b in range(B):
        for m in range(G):
            n = o["cand_n"][b, m]
            np.testing.assert_array_equal(o["cand"][b, m, :n], bc[b * G + m])


@pytest.mark.parametrize("case", CASES)
def test_member_causal_reuse_matches_brute_force(case):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    exact = all(s & (s - 1) == 0 for s in {g, Lq % g} - {0})
    o = oracle.reuse(q, w, k, g, topk, member_causal=True)
    bi, bs = brute.reuse(q, w, k, g, topk, dt, member_causal=True)
    if exact:
        np.testing.assert_array_equal(o["indices"], bi)
        np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
    else:
        np.testing.assert_array_equal(o["indices"] >= 0, bi >= 0)
        ok = o["indices"] >= 0
        np.testing.assert_allclose(o["scores"][ok], bs[ok], rtol=1e-6)


@pytest.mark.parametrize("case", CASES)
def test_last_member_proxy_is_the_last_members_dense_row(case):
    """With the last member as proxy, q-bar = q[t_last] and the scan bound is
    t_last, so every Reuse row of the group is that member's dense row."""
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    o = oracle.reuse(q, w, k, g, topk, agg="last")
    dn = oracle.dense(q, w, k, topk)
    for r in range(Lq):
        last = min((r // g + 1) * g, Lq) - 1
        np.testing.assert_array_equal(o["indices"][:, r], dn["indices"][:, last])
        np.testing.assert_array_equal(o["scores"][:, r], dn["scores"][:, last])


@pytest.mark.parametrize("case", CASES)
def test_first_member_proxy_is_a_dense_row_at_the_last_position(case):
    """Move the first member's (q, w) onto the group's last row: the dense row
    there must equal the first-member Reuse row of the group."""
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    o = oracle.reuse(q, w, k, g, topk, agg="first")
    for m in range(-(-Lq // g)):
        r0, last = m * g, min((m + 1) * g, Lq) - 1
        q2, w2 = q.copy(), w.copy()
        q2[:, last], w2[:, last] = q[:, r0], w[:, r0]
        dn = oracle.dense(q2, w2, k, topk, rows=[b * Lq + last for b in range(B)])
        for r in range(r0, last + 1):
            np.testing.assert_array_equal(o["indices"][:, r], dn["indices"][:, last])


@pytest.mark.parametrize("knob", [{"agg": "first"}, {"agg": "last"}, {"member_causal": True}])
def test_knobs_collapse_onto_dense_when_g_is_1(knob):
    q, w, k = exact_random(3, 2, 21, 21, 3, 8, BF16)
    dn = oracle.dense(q, w, k, 5)
    ru = oracle.reuse(q, w, k, 1, 5, **knob)
    np.testing.assert_array_equal(ru["indices"], dn["indices"])
    np.testing.assert_array_equal(ru["scores"], dn["scores"])
    if "agg" in knob:
        rf = oracle.refine(q, w, k, 1, 5, 9, **knob)
        np.testing.assert_array_equal(rf["indices"], dn["indices"])


@pytest.mark.parametrize("agg", ["mean", "first", "last"])
def test_member_causal_reuse_structure(agg):
    """Each member keeps min(k, t+1) entries, all at s <= t; the group's last
    member keeps exactly the plain Reuse row; and every member's set is the
    optimal top-k of the proxy row truncated at its own t."""
    B, Lq, Lk, H, d, g, topk = 1, 40, 40, 4, 16, 8, 6
    q, w, k = gauss_random(5, B, Lq, Lk, H, d, F32)
    mc = oracle.reuse(q, w, k, g, topk, agg=agg, member_causal=True)
    plain = oracle.reuse(q, w, k, g, topk, agg=agg)
    idx = mc["indices"][0]
    for r in range(Lq):
        n = min(topk, r + 1)
        assert np.all(idx[r, :n] >= 0) and np.all(idx[r, n:] == -1)
        assert np.all(idx[r, :n] <= r)
        assert np.all(np.diff(idx[r, :n]) > 0)
    for m in range(Lq // g):
        last = (m + 1) * g - 1
        np.testing.assert_array_equal(idx[last], plain["indices"][0, last])
        row = oracle.proxy_row(q, w, k, g, 0, m, agg=agg)
        for r in range(m * g, last + 1):
            n = min(topk, r + 1)
            checks.check_topk_optimal(idx[r, :n], None, row[:r + 1].astype(np.float64), np.arange(r + 1),
                                      rtol=0.0)


def test_member_causal_with_newest_keys_winning():
    """Scores increase with s (k_s along e1, q along e1): a member at t keeps
    the k newest positions s <= t, which differs from the group's row for
    every member but the last."""
    Lq = Lk = 24
    g, topk = 4, 3
    q = np.zeros((1, Lq, 1, 2), np.float32)
    q[..., 0] = 1.0
    k = np.zeros((1, Lk, 2), np.float32)
    k[0, :, 0] = np.arange(Lk, dtype=np.float32) / 8.0
    w = np.ones((1, Lq, 1), np.float32)
    mc = oracle.reuse(q, w, k, g, topk, member_causal=True)["indices"][0]
    for r in range(Lq):
        n = min(topk, r + 1)
        np.testing.assert_array_equal(mc[r, :n], np.arange(r + 1 - n, r + 1))


def test_rejects_bad_knobs():
    q, w, k = exact_random(0, 1, 8, 8, 2, 4, F32)
    with pytest.raises(ValueError):
        oracle.reuse(q, w, k, 2, 3, agg="median")
    with pytest.raises(ValueError):
        oracle.refine(q, w, k, 2, 3, 4, member_causal=True)  # the knob belongs to Reuse
