"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each pin checks the oracle against something other than itself: a float64
brute force written differently (whole matrices + lexsort), closed forms of
the cost counters (the per-group O(L) / O(L + g c) claims), special cases
that collapse one variant onto another (g = 1, c >= prefix), exact integer
arithmetic, ties with a known answer, and metamorphic relations.

Sources: PIVOT paper summary page (picx.dev), eq. (1) and eqs. (2)-(9);
"Two Variants" cost lines O(L) per group (Reuse) and O(L + g c) (Refine).
"""
import numpy as np
import pytest

import oracle
from oracle import brute
from tests import checks
from workloads import BF16, F32, exact_random, gauss_random

EXACT_CASES = [
    # B, Lq, Lk, H, d, g, topk, c, dtype
    (1, 24, 24, 2, 4, 4, 5, 9, F32),
    (1, 37, 37, 3, 5, 4, 6, 11, BF16),      # ragged last group (37 = 9*4 + 1)
    (2, 19, 19, 2, 8, 3, 4, 7, BF16),       # g = 3: non power-of-two mean
    (1, 10, 10, 2, 4, 4, 16, 32, F32),      # L < k, c >= L
    (1, 4, 40, 3, 6, 4, 7, 12, BF16),       # decode shape: Lq = g < Lk
    (2, 6, 33, 2, 4, 3, 5, 10, BF16),       # two decode groups per sequence
    (1, 64, 64, 4, 8, 8, 8, 16, F32),
    (1, 17, 17, 1, 3, 16, 4, 8, BF16),      # one head, g > half of L
    (1, 9, 9, 2, 2, 1, 3, 3, F32),          # g = 1
]


def _exact(case, seed=0):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    return exact_random(seed, B, Lq, Lk, H, d, dt)


def _pow2_groups(Lq, g):
    """True when every group size is a power of two, so the proxy's mean (and
    hence every later product) stays exact in float32."""
    sizes = {g, Lq - (Lq // g) * g} - {0}
    return all(s & (s - 1) == 0 for s in sizes)


def _assert_rows(o_idx, o_sc, b_idx, b_sc, exact):
    if exact:
        np.testing.assert_array_equal(o_idx, b_idx)
        np.testing.assert_array_equal(o_sc.astype(np.float64), b_sc)
        return
    # a non power-of-two mean is rounded, so later float32 products round too
    np.testing.assert_array_equal(o_idx >= 0, b_idx >= 0)
    ok = o_idx >= 0
    np.testing.assert_allclose(o_sc[ok], b_sc[ok], rtol=1e-6)
    mism = (o_idx != b_idx) & ok
    if mism.any():  # allowed only between scores tied to that tolerance
        np.testing.assert_allclose(o_sc[mism], b_sc[mism], rtol=1e-6)


@pytest.mark.parametrize("case", EXACT_CASES)
def test_dense_matches_float64_brute_force_bitwise(case):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _exact(case)
    o = oracle.dense(q, w, k, topk)
    bi, bs = brute.dense(q, w, k, topk, dt)
    np.testing.assert_array_equal(o["indices"], bi)
    np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)


@pytest.mark.parametrize("case", EXACT_CASES)
def test_reuse_matches_float64_brute_force_bitwise(case):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _exact(case)
    o = oracle.reuse(q, w, k, g, topk)
    bi, bs = brute.reuse(q, w, k, g, topk, dt)
    _assert_rows(o["indices"], o["scores"], bi, bs, _pow2_groups(Lq, g))


@pytest.mark.parametrize("case", EXACT_CASES)
def test_refine_matches_float64_brute_force_bitwise(case):
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _exact(case)
    o = oracle.refine(q, w, k, g, topk, c)
    bi, bs, bc = brute.refine(q, w, k, g, topk, c, dt)
    exact = _pow2_groups(Lq, g)
    _assert_rows(o["indices"], o["scores"], bi, bs, exact)
    if not exact:
        return
    G = o["cand"].shape[1]
    for b in range(B):
        for m in range(G):
            n = o["cand_n"][b, m]
            np.testing.assert_array_equal(o["cand"][b, m, :n], bc[b * G + m])
            assert np.all(o["cand"][b, m, n:] == -1)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_gaussian_inputs_agree_with_float64_within_rounding(seed):
    """Random float inputs: fp32 scores within 1e-5 of float64; the selected
    sets can differ only between elements tied to that tolerance."""
    B, Lq, Lk, H, d, g, topk, c = 1, 48, 48, 4, 16, 4, 6, 12
    q, w, k = gauss_random(seed, B, Lq, Lk, H, d, F32)
    od = oracle.dense(q, w, k, topk)
    bi, bs = brute.dense(q, w, k, topk, F32)
    I = brute.score_matrix(q[0].astype(np.float64), w[0].astype(np.float64), k[0].astype(np.float64))
    for r in range(Lq):
        n = min(topk, r + 1)
        got = od["indices"][0, r, :n]
        np.testing.assert_allclose(od["scores"][0, r, :n], I[r, got], rtol=1e-5, atol=1e-6)
        checks.check_topk_optimal(got, None, I[r, :r + 1], np.arange(r + 1), rtol=1e-5)
    orr = oracle.refine(q, w, k, g, topk, c)
    _, _, bc = brute.refine(q, w, k, g, topk, c, F32)
    qbar, wbar = brute.proxy(q, w, g, F32)
    Ibar = brute.score_matrix(qbar[0], wbar[0], k[0].astype(np.float64))
    for m in range(Lq // g):
        tl = (m + 1) * g - 1
        n = orr["cand_n"][0, m]
        checks.check_topk_optimal(orr["cand"][0, m, :n], None, Ibar[m, :tl + 1], np.arange(tl + 1), rtol=1e-5)


def test_g1_collapses_reuse_and_refine_onto_dense():
    """eq. (4) with g = 1 gives the proxy = the query itself."""
    q, w, k = gauss_random(7, 2, 40, 40, 3, 8, BF16)
    d = oracle.dense(q, w, k, 7)
    r = oracle.reuse(q, w, k, 1, 7)
    f = oracle.refine(q, w, k, 1, 7, 13)
    np.testing.assert_array_equal(d["indices"], r["indices"])
    np.testing.assert_array_equal(d["scores"], r["scores"])
    np.testing.assert_array_equal(d["indices"], f["indices"])
    np.testing.assert_array_equal(d["scores"], f["scores"])


def test_candidates_covering_the_prefix_make_refine_equal_dense():
    """eq. (7) with c >= t_last + 1 keeps every key, so eqs. (8)-(9) are eq. (1)."""
    Lq = 45
    q, w, k = gauss_random(8, 1, Lq, Lq, 4, 8, F32)
    d = oracle.dense(q, w, k, 9)
    f = oracle.refine(q, w, k, 6, 9, Lq)
    np.testing.assert_array_equal(d["indices"], f["indices"])
    np.testing.assert_array_equal(d["scores"], f["scores"])


def test_reuse_rows_identical_within_a_group_and_counts():
    B, Lq, Lk, g, topk = 2, 50, 50, 8, 11
    q, w, k = gauss_random(9, B, Lq, Lk, 4, 8, BF16)
    r = oracle.reuse(q, w, k, g, topk)
    for b in range(B):
        for m in range(-(-Lq // g)):
            rows = r["indices"][b, m * g:min((m + 1) * g, Lq)]
            assert np.all(rows == rows[0])
    checks.check_structure(r["indices"], r["scores"], Lq, Lk, g=g,
                           counts=checks.reuse_counts(B, Lq, Lk, g, topk))


@pytest.mark.parametrize("Lq,Lk,g,c", [(64, 64, 8, 16), (70, 70, 8, 16), (4, 30, 4, 10), (33, 33, 5, 64)])
def test_cost_counters_match_closed_forms(Lq, Lk, g, c):
    """Dense: H*sum_t (t+1). Reuse: H*sum_m (t_last+1), = H*L(L/g+1)/2 when g | L.
    Refine adds H*sum_m g_m*min(c, t_last+1). Dense/Reuse -> g as L grows."""
    H, topk = 3, 4
    q, w, k = gauss_random(10, 1, Lq, Lk, H, 4, F32)
    pos = checks.positions(Lq, Lk)
    tl = checks.group_last_pos(Lq, Lk, g)
    gm = np.minimum((np.arange(len(tl)) + 1) * g, Lq) - np.arange(len(tl)) * g
    assert oracle.dense(q, w, k, topk)["counters"] == (0.0, 0.0, H * float((pos + 1).sum()))
    assert oracle.reuse(q, w, k, g, topk)["counters"] == (H * float((tl + 1).sum()), 0.0, 0.0)
    ref = oracle.refine(q, w, k, g, topk, c)["counters"]
    assert ref == (H * float((tl + 1).sum()), H * float((gm * np.minimum(c, tl + 1)).sum()), 0.0)
    if Lq == Lk and Lq % g == 0:
        assert H * (tl + 1).sum() == H * Lq * (Lq // g + 1) // 2


def test_counter_ratio_tends_to_g():
    """O(L^2) -> O(L^2 / g): the oracle's dense/Reuse dot-product ratio is
    (L+1)/(L/g+1), which tends to g."""
    L, g = 512, 8
    q, w, k = gauss_random(18, 1, L, L, 1, 1, F32)
    dense_dots = oracle.dense(q, w, k, 4)["counters"][2]
    reuse_dots = oracle.reuse(q, w, k, g, 4)["counters"][0]
    assert dense_dots / reuse_dots == pytest.approx((L + 1) / (L / g + 1), rel=1e-12)
    assert abs(dense_dots / reuse_dots - g) < g * g / L


def test_all_equal_keys_select_lowest_positions():
    """Every score ties, so the order falls back to position: [0..k-1]."""
    B, L, H, d, g, topk, c = 1, 30, 2, 4, 4, 5, 9
    q, w, _ = gauss_random(11, B, L, L, H, d, F32)
    k = np.tile(np.float32([0.5, -0.25, 1.0, 0.75]), (B, L, 1))
    for res in (oracle.dense(q, w, k, topk), oracle.reuse(q, w, k, g, topk),
                oracle.refine(q, w, k, g, topk, c)):
        for r in range(L):
            n = min(topk, r + 1)
            np.testing.assert_array_equal(res["indices"][0, r, :n], np.arange(n))


def test_monotone_scores_select_the_newest_positions():
    """k_s = (s+1) e_1 and q along +e_1 with w > 0: the score grows with s, so
    the top-k of a row at t is t-k+1 .. t (Reuse: relative to t_last)."""
    L, H, d, g, topk = 40, 2, 3, 4, 6
    k = np.zeros((1, L, d), np.float32)
    k[0, :, 0] = np.arange(1, L + 1, dtype=np.float32)
    q = np.zeros((1, L, H, d), np.float32)
    q[..., 0] = 0.5
    w = np.full((1, L, H), 0.25, np.float32)
    dd = oracle.dense(q, w, k, topk)["indices"][0]
    ru = oracle.reuse(q, w, k, g, topk)["indices"][0]
    for t in range(L):
        n = min(topk, t + 1)
        np.testing.assert_array_equal(dd[t, :n], np.arange(t + 1 - n, t + 1))
        tl = min((t // g + 1) * g, L) - 1
        n2 = min(topk, tl + 1)
        np.testing.assert_array_equal(ru[t, :n2], np.arange(tl + 1 - n2, tl + 1))


def test_single_head_unit_weight_reduces_to_a_sorted_dot_product():
    """H = 1, w = 1 and positive q, k: eq. (1) is the plain dot product, so the
    dense top-k is numpy's argsort of q.k over the prefix."""
    L, d, topk = 50, 6, 7
    r = np.random.default_rng(12)
    q = r.uniform(0.1, 1.0, (1, L, 1, d)).astype(np.float32)
    k = r.uniform(0.1, 1.0, (1, L, d)).astype(np.float32)
    w = np.ones((1, L, 1), np.float32)
    out = oracle.dense(q, w, k, topk)
    dots = q[0, :, 0].astype(np.float64) @ k[0].astype(np.float64).T
    for t in range(L):
        n = min(topk, t + 1)
        ref = np.sort(np.argsort(-dots[t, :t + 1], kind="stable")[:n])
        np.testing.assert_array_equal(out["indices"][0, t, :n], ref)


def test_head_permutation_and_power_of_two_weight_scaling():
    """Permuting heads jointly in q and w is exact on exact inputs; scaling w
    by 2^n scales every score exactly and keeps the indices."""
    case = (1, 32, 32, 4, 8, 4, 6, 12, BF16)
    q, w, k = _exact(case, seed=5)
    base = oracle.refine(q, w, k, 4, 6, 12)
    perm = np.array([2, 0, 3, 1])
    p = oracle.refine(q[:, :, perm], w[:, :, perm], k, 4, 6, 12)
    np.testing.assert_array_equal(base["indices"], p["indices"])
    np.testing.assert_array_equal(base["scores"], p["scores"])
    s = oracle.refine(q, (w * 8).astype(np.float32), k, 4, 6, 12)
    np.testing.assert_array_equal(base["indices"], s["indices"])
    valid = base["indices"] >= 0
    np.testing.assert_array_equal(base["scores"][valid] * 8, s["scores"][valid])


def test_pool_closed_form():
    """eq. (4) on exact inputs: the proxy is the per-head mean, exactly."""
    q, w, _ = exact_random(13, 1, 20, 20, 3, 4, BF16)
    g = 8
    qbar, wbar = oracle.pool(q, w, g)
    from workloads import bf16_bits_to_f32
    qf = bf16_bits_to_f32(q).astype(np.float64)
    for m in range(3):
        sl = slice(m * g, min((m + 1) * g, 20))
        n = sl.stop - sl.start
        exp_q = qf[0, sl].sum(axis=0) / n
        if n == 8:  # multiples of 1/32: exact in bf16
            np.testing.assert_array_equal(qbar[0, m], exp_q)
        else:       # 4 members: multiples of 1/16, also exact
            np.testing.assert_array_equal(qbar[0, m], exp_q)
        np.testing.assert_array_equal(wbar[0, m], w[0, sl].astype(np.float64).sum(axis=0) / n)


def test_refine_structure_and_subset_of_candidates():
    B, Lq, Lk, g, topk, c = 2, 41, 41, 6, 5, 12
    q, w, k = gauss_random(14, B, Lq, Lk, 4, 8, BF16)
    f = oracle.refine(q, w, k, g, topk, c)
    G = -(-Lq // g)
    tl = checks.group_last_pos(Lq, Lk, g)
    counts = []
    for b in range(B):
        for r in range(Lq):
            m = r // g
            n = f["cand_n"][b, m]
            assert n == min(c, tl[m] + 1)
            C = f["cand"][b, m, :n]
            t = Lk - Lq + r
            counts.append(min(topk, int((C <= t).sum())))
            row = f["indices"][b, r]
            assert set(row[row >= 0].tolist()) <= set(C.tolist())
    checks.check_structure(f["indices"], f["scores"], Lq, Lk, counts=np.array(counts))
    assert f["cand"].shape == (B, G, c)


def test_external_candidates_reproduce_the_member_step():
    """Feeding back the oracle's own C gives the same member rows (the hook the
    GPU parity rule uses to judge Refine past a differing candidate set)."""
    B, Lq, Lk, g, topk, c = 1, 30, 30, 5, 4, 8
    q, w, k = gauss_random(15, B, Lq, Lk, 3, 8, F32)
    f = oracle.refine(q, w, k, g, topk, c)
    f2 = oracle.refine(q, w, k, g, topk, c, cand_in=f["cand"], cand_in_n=f["cand_n"])
    np.testing.assert_array_equal(f["indices"], f2["indices"])
    assert f2["counters"][0] == 0.0


def test_unit_subset_matches_full_run():
    B, Lq, Lk, g, topk, c = 2, 33, 33, 4, 5, 10
    q, w, k = gauss_random(16, B, Lq, Lk, 2, 8, F32)
    full = oracle.refine(q, w, k, g, topk, c)
    G = -(-Lq // g)
    units = [0, 3, G + 2, 2 * G - 1]
    part = oracle.refine(q, w, k, g, topk, c, groups=units)
    for u in units:
        b, m = divmod(u, G)
        rows = slice(m * g, min((m + 1) * g, Lq))
        np.testing.assert_array_equal(part["indices"][b, rows], full["indices"][b, rows])
    assert np.all(part["indices"][0, g:2 * g] == -2)


def test_rejects_bad_arguments():
    q, w, k = gauss_random(17, 1, 8, 8, 2, 4, F32)
    with pytest.raises(ValueError):
        oracle.refine(q, w, k, 2, 5, 4)       # c < k
    with pytest.raises(ValueError):
        oracle.reuse(q, w, k, 0, 3)           # g < 1
    with pytest.raises(ValueError):
        oracle.dense(q, w, k[:, :4], 3)       # Lq > Lk
    with pytest.raises(ValueError):
        oracle.dense(q, w, k, 3, rows=[100])  # unit out of range


@pytest.mark.parametrize("case", [c for c in EXACT_CASES if _pow2_groups(c[1], c[5])])
def test_scores_at_equal_the_brute_force_score_matrices(case):
    """oracle.scores_at (eq. (1) rows and eq. (5) proxies at chosen key
    positions, used by the full-size GPU checks) against the float64 brute
    force's whole matrices, on inputs where every sum is exact: bit for bit,
    every sequence, every row / group, shuffled positions with gaps."""
    B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _exact(case, seed=5)
    kv = brute._f64(k, dt)
    r = np.random.default_rng(9)
    P = min(Lk, 7)
    rows = np.arange(B * Lq)
    pos = np.stack([r.permutation(Lk)[:P] for _ in rows]).astype(np.int32)
    pos[:, -1] = -1                                   # skipped slot
    got = oracle.scores_at(q, w, k, rows, pos)
    qf = brute._f64(q, dt)
    for u in rows:
        b, t = divmod(int(u), Lq)
        ref = brute.score_matrix(qf[b, t][None], np.asarray(w[b, t], np.float64)[None], kv[b])[0]
        np.testing.assert_array_equal(got[u, :-1].astype(np.float64), ref[pos[u, :-1]])
        assert np.isnan(got[u, -1])
    qbar, wbar = brute.proxy(q, w, g, dt)
    G = -(-Lq // g)
    groups = np.arange(B * G)[::-1]                   # any order
    gpos = np.stack([r.permutation(Lk)[:P] for _ in groups]).astype(np.int32)
    got = oracle.scores_at(q, w, k, groups, gpos, g=g)
    for i, u in enumerate(groups):
        b, m = divmod(int(u), G)
        ref = brute.score_matrix(qbar[b, m][None], wbar[b, m][None], kv[b])[0]
        np.testing.assert_array_equal(got[i].astype(np.float64), ref[gpos[i]])


def test_scores_at_agrees_with_the_oracle_rows_on_float_inputs():
    """On Gaussian inputs the selected entries of the oracle's own dense and
    Refine rows carry exactly the scores scores_at gives for them."""
    q, w, k = gauss_random(4, 2, 50, 60, 3, 8, BF16)
    d = oracle.dense(q, w, k, 6)
    rows = np.arange(2 * 50)
    got = oracle.scores_at(q, w, k, rows, d["indices"].reshape(100, 6))
    ok = d["indices"].reshape(100, 6) >= 0
    np.testing.assert_array_equal(got[ok], d["scores"].reshape(100, 6)[ok])
    rf = oracle.refine(q, w, k, 4, 5, 9)
    G = 13
    gp = oracle.scores_at(q, w, k, np.arange(2 * G), rf["cand"].reshape(2 * G, 9), g=4)
    for u in range(2 * G):
        b, m = divmod(u, G)
        n = rf["cand_n"][b, m]
        row = oracle.proxy_row(q, w, k, 4, b, m)
        np.testing.assert_array_equal(gp[u, :n], row[rf["cand"][b, m, :n]])
