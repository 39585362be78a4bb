"""GPU parity at the full sizes of the five measured workloads, in the launch
configuration the benchmark times.

  exact_prefill_L8192   bit for bit with the oracle (every sum is exact):
                        Reuse, Refine and dense on every group / row
  prefill_L32768        float rule on every group (Refine, Reuse) and every
                        row (dense) + every-row structure
  prefill_L131072       Refine and Reuse for g in {4, 8, 16} and dense (g = 1):
                        float rule on 512 evenly spaced groups for Refine g=8,
                        128 for the other Refine and Reuse cases and 64 rows
                        (plus the k boundary) for dense + every-row structure;
                        repeated calls bit-identical
  mtp_decode            Refine, float rule on every group (32 sequences);
                        repeated calls bit-identical
  mtp_decode_ragged     Refine over ragged lengths and 64-key pages (the
                        benchmark's layout), float rule on every sequence
                        against the oracle run on that sequence's own prefix
  tiny_prefill_L512     covered bit for bit in test_gpu_parity.py

The float rule (tests/parity.py) scores the GPU's selected positions with
the oracle's own fp32 arithmetic (oracle.scores_at).
"""
import numpy as np
import pytest

import oracle
from tests import parity
from workloads import DECODE, DECODE_RAGGED, EXACT, LONG_128K, PREFILL_32K, generate, paged_layout, seq_lens, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _sample_groups(G, n, B=1):
    """First, last and evenly spaced groups of each sequence (flat ids)."""
    per = np.unique(np.r_[0, 1, G - 2, G - 1, np.linspace(0, G - 1, n).astype(np.int64)])
    per = per[(per >= 0) & (per < G)]
    return np.concatenate([b * G + per for b in range(B)])


def _np(t):
    return None if t is None else t.cpu().numpy()


# ------------------------------------------------------------------ exact 8K
@pytest.fixture(scope="module")
def exact_data():
    q, w, k = generate(EXACT)
    return q, w, k, to_device(q, w, k)


def test_exact_workload_refine_and_reuse_bitwise(exact_data):
    q, w, k, (tq, tw, tk) = exact_data
    W = EXACT
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    r_i, r_s = pv.index_reuse(tq, tw, tk, W.g, W.topk, return_scores=True)
    torch.cuda.synchronize()
    _say("[exact] GPU done; oracle refine")
    ref = oracle.refine(q, w, k, W.g, W.topk, W.c)
    np.testing.assert_array_equal(_np(f_n), ref["cand_n"])
    np.testing.assert_array_equal(_np(f_c), ref["cand"])
    np.testing.assert_array_equal(_np(f_i), ref["indices"])
    np.testing.assert_array_equal(_np(f_s), ref["scores"])
    _say("[exact] oracle reuse")
    ref = oracle.reuse(q, w, k, W.g, W.topk)
    np.testing.assert_array_equal(_np(r_i), ref["indices"])
    np.testing.assert_array_equal(_np(r_s), ref["scores"])


def test_exact_workload_rank_rows_bitwise(exact_data):
    """The exact 8K workload's Refine rows in rank order (every row of k = 256)
    equal the oracle's rows in rank order bit for bit."""
    q, w, k, (tq, tw, tk) = exact_data
    W = EXACT
    i, sc = pv.index(tq, tw, tk, variant=pv.REFINE, g=W.g, topk=W.topk, c=W.c, order="score", return_scores=True)
    torch.cuda.synchronize()
    _say("[exact] oracle refine, rank order")
    ref = oracle.refine(q, w, k, W.g, W.topk, W.c, order="score")
    np.testing.assert_array_equal(_np(i), ref["indices"])
    np.testing.assert_array_equal(_np(sc), ref["scores"])


def test_exact_workload_dense_bitwise(exact_data):
    q, w, k, (tq, tw, tk) = exact_data
    W = EXACT
    d_i, d_s = pv.index_dense(tq, tw, tk, W.topk, return_scores=True)
    torch.cuda.synchronize()
    d_i, d_s = _np(d_i), _np(d_s)
    parity.structure_all_rows(d_i, W.Lq, W.Lk, W.topk,
                              counts=np.minimum(W.topk, np.arange(W.Lq) + 1)[None])
    _say("[exact] oracle dense, every row")
    ref = oracle.dense(q, w, k, W.topk)
    np.testing.assert_array_equal(d_i, ref["indices"])
    np.testing.assert_array_equal(d_s, ref["scores"])


# ------------------------------------------------------------ float prefill
@pytest.fixture(scope="module")
def prefill32k():
    q, w, k = generate(PREFILL_32K)
    return q, w, k, to_device(q, w, k)


@pytest.fixture(scope="module")
def prefill128k():
    q, w, k = generate(LONG_128K)
    return q, w, k, to_device(q, w, k)


def _refine_case(data, W, g, n_groups):
    q, w, k, (tq, tw, tk) = data
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, g, W.topk, W.c, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    f_i, f_s, f_c, f_n = _np(f_i), _np(f_s), _np(f_c), _np(f_n)
    G = -(-W.Lq // g)
    tl = np.minimum((np.arange(G) + 1) * g, W.Lq) - 1
    np.testing.assert_array_equal(f_n[0], np.minimum(W.c, tl + 1))
    parity.structure_all_rows(f_i, W.Lq, W.Lk, W.topk)
    groups = np.arange(G) if n_groups is None else _sample_groups(G, n_groups)
    d = parity.check_refine_groups(q, w, k, g, W.topk, W.c, f_i, f_s, f_c, f_n, groups)
    _say(f"[{W.name} refine g={g}] {len(groups)} groups checked, {d} boundary swaps")


def _reuse_case(data, W, g, n_groups):
    q, w, k, (tq, tw, tk) = data
    r_i, r_s = pv.index_reuse(tq, tw, tk, g, W.topk, return_scores=True)
    torch.cuda.synchronize()
    r_i, r_s = _np(r_i), _np(r_s)
    G = -(-W.Lq // g)
    tl = np.minimum((np.arange(G) + 1) * g, W.Lq) - 1
    parity.structure_all_rows(r_i, W.Lq, W.Lk, W.topk, g=g,
                              counts=np.minimum(W.topk, tl[np.arange(W.Lq) // g] + 1)[None])
    groups = np.arange(G) if n_groups is None else _sample_groups(G, n_groups)
    d = parity.check_reuse_groups(q, w, k, g, W.topk, r_i, r_s, groups)
    _say(f"[{W.name} reuse g={g}] {len(groups)} groups checked, {d} boundary swaps")


def _dense_case(data, W, n_rows):
    q, w, k, (tq, tw, tk) = data
    d_i, d_s = pv.index_dense(tq, tw, tk, W.topk, return_scores=True)
    torch.cuda.synchronize()
    d_i, d_s = _np(d_i), _np(d_s)
    parity.structure_all_rows(d_i, W.Lq, W.Lk, W.topk, counts=np.minimum(W.topk, np.arange(W.Lq) + 1)[None])
    rows = (np.arange(W.Lq) if n_rows is None else
            np.unique(np.r_[0, 1, 2047, 2048, 2049, np.linspace(0, W.Lq - 1, n_rows).astype(np.int64), W.Lq - 1]))
    d = parity.check_dense_rows(q, w, k, W.topk, d_i, d_s, rows)
    _say(f"[{W.name} dense] {len(rows)} rows checked, {d} boundary swaps")


def test_prefill_32k_refine(prefill32k):
    _refine_case(prefill32k, PREFILL_32K, PREFILL_32K.g, None)


def test_prefill_32k_reuse(prefill32k):
    _reuse_case(prefill32k, PREFILL_32K, PREFILL_32K.g, None)


def test_prefill_32k_dense(prefill32k):
    _dense_case(prefill32k, PREFILL_32K, None)


def test_prefill_32k_32_heads_refine_and_reuse():
    """The 32K workload's generator with 32 indexer heads (the 32-head MFMA
    kernels): 512 evenly spaced Refine and Reuse groups by the float rule."""
    W = PREFILL_32K.replace(H=32, name="prefill_L32768_H32")
    q, w, k = generate(W)
    data = (q, w, k, to_device(q, w, k))
    _refine_case(data, W, W.g, 512)
    _reuse_case(data, W, W.g, 512)


@pytest.mark.parametrize("g", [8, 4, 16])
def test_long_128k_refine(prefill128k, g):
    _refine_case(prefill128k, LONG_128K, g, 512 if g == 8 else 128)


def test_long_128k_repeat_calls_are_bit_identical(prefill128k):
    """Refine g=8 at full size twice (the fused scan, the group and member
    selects): indices, scores and candidate sets identical bit for bit."""
    _, _, _, (tq, tw, tk) = prefill128k
    W = LONG_128K
    a = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    b = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("g", [8, 4, 16])
def test_long_128k_reuse(prefill128k, g):
    _reuse_case(prefill128k, LONG_128K, g, 128)


def test_long_128k_dense(prefill128k):
    _dense_case(prefill128k, LONG_128K, 64)


# ------------------------------------------------------------------- decode
def test_mtp_decode_refine_every_group():
    W = DECODE
    q, w, k = generate(W)
    tq, tw, tk = to_device(q, w, k)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    f_i, f_s, f_c, f_n = _np(f_i), _np(f_s), _np(f_c), _np(f_n)
    assert np.all(f_n == W.c)
    parity.structure_all_rows(f_i, W.Lq, W.Lk, W.topk)
    d = parity.check_refine_groups(q, w, k, W.g, W.topk, W.c, f_i, f_s, f_c, f_n, np.arange(W.B))
    _say(f"[decode] {W.B} groups checked, {d} boundary swaps")
    again = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    for x, y in zip((f_i, f_s, f_c, f_n), again):
        np.testing.assert_array_equal(x, _np(y))


def test_mtp_decode_ragged_paged_refine_every_sequence():
    W = DECODE_RAGGED
    q, w, k = generate(W)
    lens = seq_lens(W)
    pool, table = paged_layout(k, lens, 64, W.seed)
    tq, tw, tpool = to_device(q, w, pool)
    f_i, f_s, f_c, f_n = pv.index_kv(tq, tw, tpool, torch.from_numpy(lens).cuda(), torch.from_numpy(table).cuda(),
                                     page_size=64, lk=W.Lk, variant=pv.REFINE, g=W.g, topk=W.topk, c=W.c,
                                     return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    f_i, f_s, f_c, f_n = _np(f_i), _np(f_s), _np(f_c), _np(f_n)
    assert np.all(f_n == W.c)
    d = 0
    for b in range(W.B):
        n = int(lens[b])
        parity.structure_all_rows(f_i[b:b + 1], W.Lq, n, W.topk)
        d += parity.check_refine_groups(q[b:b + 1], w[b:b + 1], k[b:b + 1, :n], W.g, W.topk, W.c, f_i[b:b + 1],
                                        f_s[b:b + 1], f_c[b:b + 1], f_n[b:b + 1], np.arange(1))
    _say(f"[decode ragged] {W.B} sequences checked, {d} boundary swaps")
