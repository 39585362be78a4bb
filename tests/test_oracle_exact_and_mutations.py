"""Two more pins of the CPU oracle.

1. The exact-arithmetic workload (L=8192, H=64, d=128, g=8, k=256, c=512;
   q, k in {-3..3}/4, w in {1/8..1}) recomputed in int64: every proxy score
   is an integer multiple of 2^-13 (member scores of 2^-7), so the oracle's
   float32 values, candidate sets and rows must equal the integer result.
2. Pin sensitivity: plausible mistakes planted in a private copy of the
   oracle's C source (never in the oracle itself) must each fail the pins.

Sources: PIVOT paper summary page (picx.dev), eqs. (1), (4)-(9).
"""
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import brute
from tests import checks
from workloads import BF16, EXACT, F32, exact_random, generate


# ------------------------------------------------------------------ integers
@pytest.fixture(scope="module")
def exact_inputs():
    return generate(EXACT)


def _int_inputs(q, w, k):
    from workloads import bf16_bits_to_f32
    qi = np.rint(bf16_bits_to_f32(q) * 4).astype(np.int64)       # q = qi / 4
    ki = np.rint(bf16_bits_to_f32(k) * 4).astype(np.int64)       # k = ki / 4
    wi = np.rint(w.astype(np.float64) * 8).astype(np.int64)      # w = wi / 8
    assert np.all(bf16_bits_to_f32(q) * 4 == qi) and np.all(w * 8 == wi)
    return qi, wi, ki


def _int_rank(num, pos, kk):
    order = np.lexsort((pos, -num))[:kk]
    return np.sort(pos[order])


@pytest.mark.slow
def test_exact_workload_equals_int64_recomputation(exact_inputs):
    q, w, k = exact_inputs
    W = EXACT
    qi, wi, ki = _int_inputs(q, w, k)
    g, topk, c = W.g, W.topk, W.c
    groups = [0, 1, 37, 511, 1022, 1023]
    res = oracle.refine(q, w, k, g, topk, c, groups=groups)
    for m in groups:
        rows = slice(m * g, (m + 1) * g)
        t_last = (m + 1) * g - 1
        pos = np.arange(t_last + 1)
        # eq. (4): qbar = sum/8 of (qi/4) = qsum/32, wbar = wsum/64
        qsum = qi[0, rows].sum(axis=0)                     # [H, d]
        wsum = wi[0, rows].sum(axis=0)                     # [H]
        dots = qsum @ ki[0, :t_last + 1].T                 # qbar.k = dots/128
        num = (wsum[:, None] * np.maximum(dots, 0)).sum(axis=0)   # score = num / 2^13
        prow = oracle.proxy_row(q, w, k, g, 0, m)
        np.testing.assert_array_equal(prow.astype(np.float64) * 8192.0, num.astype(np.float64))
        C = _int_rank(num, pos, c)
        n = res["cand_n"][0, m]
        np.testing.assert_array_equal(res["cand"][0, m, :n], C)
        for r in range(rows.start, rows.stop):
            keep = C[C <= r]
            mdots = qi[0, r] @ ki[0, keep].T               # q.k = mdots/16
            mnum = (wi[0, r][:, None] * np.maximum(mdots, 0)).sum(axis=0)   # score = mnum / 128
            exp_idx = _int_rank(mnum, keep, topk)
            nn = len(exp_idx)
            np.testing.assert_array_equal(res["indices"][0, r, :nn], exp_idx)
            assert np.all(res["indices"][0, r, nn:] == -1)
            got_sc = res["scores"][0, r, :nn].astype(np.float64) * 128.0
            ref_sc = mnum[np.searchsorted(keep, exp_idx)].astype(np.float64)
            np.testing.assert_array_equal(got_sc, ref_sc)


@pytest.mark.slow
def test_exact_workload_dense_rows_equal_int64(exact_inputs):
    q, w, k = exact_inputs
    qi, wi, ki = _int_inputs(q, w, k)
    rows = [0, 5, 255, 256, 4097, 8191]
    res = oracle.dense(q, w, k, EXACT.topk, rows=rows)
    for r in rows:
        pos = np.arange(r + 1)
        dots = qi[0, r] @ ki[0, :r + 1].T
        num = (wi[0, r][:, None] * np.maximum(dots, 0)).sum(axis=0)
        exp_idx = _int_rank(num, pos, EXACT.topk)
        np.testing.assert_array_equal(res["indices"][0, r, :len(exp_idx)], exp_idx)
        np.testing.assert_array_equal(res["scores"][0, r, :len(exp_idx)].astype(np.float64) * 128.0,
                                      num[exp_idx].astype(np.float64))


def test_exact_workload_stays_exact_in_float32(exact_inputs):
    """Headroom of the exact workload: every proxy score is < 2^11 and every
    partial sum a multiple of 2^-13, so float32 (24 bits) holds it exactly."""
    q, w, k = exact_inputs
    qi, wi, ki = _int_inputs(q, w, k)
    m = 1023
    rows = slice(m * 8, (m + 1) * 8)
    dots = qi[0, rows].sum(axis=0) @ ki[0].T
    num = (wi[0, rows].sum(axis=0)[:, None] * np.maximum(dots, 0)).sum(axis=0)
    assert num.max() < 2 ** 24
    assert np.abs(dots).max() * 128 < 2 ** 24


# ------------------------------------------------------------ planted errors
_SRC = os.path.join(os.path.dirname(oracle.__file__), "pivot_oracle.c")

_CMP_RANK = """    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);"""

MUTATIONS = {
    "dense_strict_causal": ("for (int64_t s = 0; s <= t; ++s) {", "for (int64_t s = 0; s < t; ++s) {"),
    "relu_dropped": ("float relu = dot > 0.0f ? dot : 0.0f;", "float relu = dot;"),
    "weights_ignored": ("float term = wv[j] * relu;", "float term = relu;"),
    "ties_to_higher_position": (_CMP_RANK, _CMP_RANK.replace("(x->i > y->i) - (x->i < y->i)",
                                                             "(x->i < y->i) - (x->i > y->i)")),
    "short_group_divides_by_g": ("float gm = (float)(r1 - r0);", "float gm = (float)g;"),
    "member_mask_dropped": ("if (s <= t) {", "if (1) {"),
    "proxy_scan_to_first_member": ("int64_t t_last = p->Lk - p->Lq + (r1 - 1);",
                                   "int64_t t_last = p->Lk - p->Lq + r0;"),
    "proxy_not_rounded_to_bf16": ("qbar[i] = p->dtype == 1 ? round_to_bf16(mean) : mean;", "qbar[i] = mean;"),
    "wrong_key_row": ("kf + s * p->d);\n                        row[s].i", "kf + (s > 0 ? s - 1 : 0) * p->d);\n                        row[s].i"),
    "member_causal_uses_group_bound": ("memcpy(cset, row, sizeof(scored_t) * (size_t)(t + 1));\n"
                                       "                        int64_t n = top_k_by_rank(cset, t + 1, topk);",
                                       "memcpy(cset, row, sizeof(scored_t) * (size_t)(t_last + 1));\n"
                                       "                        int64_t n = top_k_by_rank(cset, t_last + 1, topk);"),
    "first_member_proxy_off_by_one": ("widen_query_row(p, q, w, b, r0, qbar, wbar);",
                                      "widen_query_row(p, q, w, b, r0 + (r1 - r0 > 1), qbar, wbar);"),
    "last_member_proxy_is_first": ("widen_query_row(p, q, w, b, r1 - 1, qbar, wbar);",
                                   "widen_query_row(p, q, w, b, r0, qbar, wbar);"),
}


def _pin_battery(lib):
    """A compact subset of the pins, run against the library at ``lib``."""
    cases = [(1, 37, 37, 3, 5, 4, 6, 11, BF16), (1, 4, 40, 3, 6, 4, 7, 12, BF16),
             (1, 32, 32, 4, 8, 8, 8, 16, F32)]
    # g = 3 with w = 1: the proxy mean needs bf16 rounding, everything after
    # it stays exact, so the rounding step itself is pinned
    cases.append((1, 21, 21, 2, 5, 3, 4, 8, BF16))
    for (B, Lq, Lk, H, d, g, topk, c, dt) in cases:
        wl = (0, 0) if g == 3 else (-3, 0)
        q, w, k = exact_random(3, B, Lq, Lk, H, d, dt, w_levels=wl)
        o = oracle.dense(q, w, k, topk, lib_path=lib)
        bi, bs = brute.dense(q, w, k, topk, dt)
        np.testing.assert_array_equal(o["indices"], bi)
        np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
        o = oracle.reuse(q, w, k, g, topk, lib_path=lib)
        bi, bs = brute.reuse(q, w, k, g, topk, dt)
        np.testing.assert_array_equal(o["indices"], bi)
        np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
        o = oracle.refine(q, w, k, g, topk, c, lib_path=lib)
        bi, bs, _ = brute.refine(q, w, k, g, topk, c, dt)
        np.testing.assert_array_equal(o["indices"], bi)
        np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
    # variant knobs: member proxies and member-causal Reuse
    for (B, Lq, Lk, H, d, g, topk, c, dt) in cases[:2]:
        q, w, k = exact_random(5, B, Lq, Lk, H, d, dt)
        for agg in ("first", "last"):
            o = oracle.reuse(q, w, k, g, topk, agg=agg, lib_path=lib)
            bi, bs = brute.reuse(q, w, k, g, topk, dt, agg=agg)
            np.testing.assert_array_equal(o["indices"], bi)
            np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
        o = oracle.reuse(q, w, k, g, topk, member_causal=True, lib_path=lib)
        bi, bs = brute.reuse(q, w, k, g, topk, dt, member_causal=True)
        np.testing.assert_array_equal(o["indices"], bi)
        np.testing.assert_array_equal(o["scores"].astype(np.float64), bs)
    # ties fall back to position
    L = 20
    q, w, _ = exact_random(4, 1, L, L, 2, 4, F32)
    kk = np.tile(np.float32([0.5, -0.25, 1.0, 0.75]), (1, L, 1))
    o = oracle.dense(q, w, kk, 5, lib_path=lib)
    for r in range(L):
        n = min(5, r + 1)
        np.testing.assert_array_equal(o["indices"][0, r, :n], np.arange(n))


def test_pin_battery_passes_on_the_oracle():
    _pin_battery(None)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(_SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mut.c")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(td, f"mut_{name}.so")
        import subprocess
        subprocess.run(["gcc", *oracle.CFLAGS, path, "-o", lib, "-lm"], check=True)
        with pytest.raises(AssertionError):
            _pin_battery(lib)
