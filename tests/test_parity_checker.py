"""The float-rule checker of tests/parity.py on the CPU: fed the oracle's own
outputs it passes; a selection that differs away from the boundary, a wrong
score, a broken order or a wrong count each make it fail. (The GPU tests
rely on it at full size; this pins that it can fail.)"""
import numpy as np
import pytest

import oracle
from tests import parity
from workloads import BF16, gauss_random


@pytest.fixture(scope="module")
def data():
    q, w, k = gauss_random(12, 2, 300, 300, 4, 16, BF16)
    return q, w, k


def test_oracle_rows_pass_every_check(data):
    q, w, k = data
    g, topk, c = 4, 20, 40
    rf = oracle.refine(q, w, k, g, topk, c)
    assert parity.check_refine_groups(q, w, k, g, topk, c, rf["indices"], rf["scores"], rf["cand"],
                                      rf["cand_n"]) == 0
    ru = oracle.reuse(q, w, k, g, topk)
    assert parity.check_reuse_groups(q, w, k, g, topk, ru["indices"], ru["scores"]) == 0
    de = oracle.dense(q, w, k, topk)
    assert parity.check_dense_rows(q, w, k, topk, de["indices"], de["scores"]) == 0
    assert parity.check_dense_rows(q, w, k, topk, de["indices"], None, rows=[0, 7, 599]) == 0


def _far_swap(idx, sc, q, w, k, row, lq):
    """Replace row's best entry by the position with the lowest score of its
    prefix that is not selected (far below the boundary); keep the row sorted."""
    b, r = divmod(row, lq)
    t = k.shape[1] - lq + r
    allpos = np.arange(t + 1)
    s = oracle.scores_at(q, w, k, [row], allpos[None])[0]
    chosen = idx[b, r][idx[b, r] >= 0]
    free = np.setdiff1d(allpos, chosen)
    worst = free[np.argmin(s[free])]
    best = chosen[np.argmax(s[chosen])]
    new = np.sort(np.r_[chosen[chosen != best], worst])
    idx[b, r, :len(new)] = new
    sc[b, r, :len(new)] = s[new]


def test_checker_fails_on_planted_mistakes(data):
    q, w, k = data
    topk = 20
    de = oracle.dense(q, w, k, topk)
    idx, sc = de["indices"].copy(), de["scores"].copy()
    _far_swap(idx, sc, q, w, k, 450, 300)
    with pytest.raises(AssertionError, match="differs"):
        parity.check_dense_rows(q, w, k, topk, idx, sc)
    sc = de["scores"].copy()
    sc[1, 250, 3] *= 1.01
    with pytest.raises(AssertionError, match="score mismatch"):
        parity.check_dense_rows(q, w, k, topk, de["indices"], sc)
    idx = de["indices"].copy()
    idx[0, 200, [2, 3]] = idx[0, 200, [3, 2]]
    with pytest.raises(AssertionError, match="ascending"):
        parity.check_dense_rows(q, w, k, topk, idx, de["scores"])
    idx = de["indices"].copy()
    idx[0, 100, topk - 1] = -1
    with pytest.raises(AssertionError, match="valid counts"):
        parity.check_dense_rows(q, w, k, topk, idx, de["scores"])
    # Refine: a candidate set missing its best candidate
    g, c = 4, 40
    rf = oracle.refine(q, w, k, g, topk, c)
    C = rf["cand"].copy()
    G = C.shape[1]
    b, m = 1, G - 3
    n = rf["cand_n"][b, m]
    tl = min((m + 1) * g, 300) - 1
    ps = oracle.proxy_row(q, w, k, g, b, m)
    cur = C[b, m, :n]
    best = cur[np.argmax(ps[cur])]
    free = np.setdiff1d(np.arange(tl + 1), cur)
    worst = free[np.argmin(ps[free])]
    C[b, m, :n] = np.sort(np.r_[cur[cur != best], worst])
    with pytest.raises(AssertionError, match="differs"):
        parity.check_refine_groups(q, w, k, g, topk, c, rf["indices"], rf["scores"], C, rf["cand_n"],
                                   groups=[b * G + m])
