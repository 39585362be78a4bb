"""GPU parity of ragged and paged batches (pivot_index_kv): each sequence b
holds its own number of keys and its queries are the last Lq positions of its
own prefix; keys are contiguous [B, Lk, d] or scattered over a page pool
through a page table. The oracle runs each sequence on its own key prefix
(the same definitions, sequence by sequence), and the paged results must
also equal the contiguous ones bit for bit.

Exact inputs (q, k in {-3..3}/4, w powers of two) make every score exact, so
indices, scores and candidate sets must match bit for bit on the MFMA
kernels (the fused scan and the split-key scan, contiguous and paged keys)
and on the exact-order kernels.
"""
import zlib

import numpy as np
import pytest

import oracle
from tests.parity import to_device
from workloads import BF16, F32, exact_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _oracle_ragged(variant, q, w, k, lens, g, topk, c):
    """Per-sequence oracle: sequence b scored on keys 0 .. lens[b] - 1."""
    B, Lq = q.shape[:2]
    out_i = np.full((B, Lq, topk), -1, dtype=np.int32)
    out_s = np.full((B, Lq, topk), -np.inf, dtype=np.float32)
    for b in range(B):
        qb, wb, kb = q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]]
        if variant == "dense":
            r = oracle.dense(qb, wb, kb, topk)
        elif variant == "reuse":
            r = oracle.reuse(qb, wb, kb, g, topk)
        else:
            r = oracle.refine(qb, wb, kb, g, topk, c)
        out_i[b], out_s[b] = r["indices"][0], r["scores"][0]
    return out_i, out_s


def _paged(k, page, seed):
    """The same keys in a shuffled page pool: (pool [P, page, d], table [B, maxp])."""
    B, Lk, d = k.shape
    maxp = -(-Lk // page)
    r = np.random.default_rng(seed)
    n_pages = B * maxp + 3
    perm = r.permutation(n_pages)[:B * maxp].reshape(B, maxp).astype(np.int32)
    pool = np.zeros((n_pages, page, d), dtype=k.dtype)
    for b in range(B):
        for j in range(maxp):
            rows = k[b, j * page:(j + 1) * page]
            pool[perm[b, j], :rows.shape[0]] = rows
    return pool, perm


def _dev(a):
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


CASES = [
    # name, B, Lq, Lk, H, d, g, topk, c, dtype
    ("mfma_decode", 5, 4, 900, 64, 128, 4, 24, 48, BF16),
    ("mfma_prefill", 2, 300, 700, 64, 128, 8, 16, 32, BF16),
    ("mfma32_decode", 3, 4, 900, 32, 128, 4, 24, 48, BF16),
    ("mfma32_prefill", 2, 300, 700, 32, 128, 8, 16, 32, BF16),
    ("exact_decode", 4, 4, 300, 3, 8, 4, 6, 12, F32),
    ("exact_prefill_bf16", 3, 40, 90, 2, 16, 4, 5, 9, BF16),
]


@pytest.mark.parametrize("path", ["fused", "split"])
@pytest.mark.parametrize("variant", ["dense", "reuse", "refine"])
@pytest.mark.parametrize("page", [0, 16, 48, 64])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_ragged_and_paged_match_oracle_bitwise(case, page, variant, path):
    name, B, Lq, Lk, H, d, g, topk, c, dt = case
    if H not in (32, 64) and path == "split":
        pytest.skip("the exact-order kernels have one scan path")
    seed = zlib.crc32(name.encode()) % 1000
    q, w, k = exact_random(seed, B, Lq, Lk, H, d, dt)
    r = np.random.default_rng(seed)
    lens = r.integers(Lq, Lk + 1, size=B).astype(np.int32)
    lens[0] = Lk
    ref_i, ref_s = _oracle_ragged(variant, q, w, k, lens, g, topk, c)
    tq, tw = _dev(q), _dev(w)
    kw = dict(variant={"dense": pv.DENSE, "reuse": pv.REUSE, "refine": pv.REFINE}[variant], g=g, topk=topk, c=c,
              scan_path=path)
    tl = torch.from_numpy(lens).cuda()
    if page:
        pool, table = _paged(k, page, seed)
        i, s = pv.index_kv(tq, tw, _dev(pool), tl, torch.from_numpy(table).cuda(), page_size=page, lk=Lk,
                           return_scores=True, **kw)
    else:
        i, s = pv.index_kv(tq, tw, _dev(k), tl, return_scores=True, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(i.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(s.cpu().numpy(), ref_s)


@pytest.mark.parametrize("path", ["fused", "split"])
def test_contiguous_ragged_on_both_scan_paths(path):
    B, Lq, Lk, g, topk, c = 3, 500, 1200, 8, 32, 64
    q, w, k = exact_random(41, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([1200, 777, 501], dtype=np.int32)
    tq, tw, tk = _dev(q), _dev(w), _dev(k)
    tl = torch.from_numpy(lens).cuda()
    for variant, v in (("refine", pv.REFINE), ("reuse", pv.REUSE)):
        i, s = pv.index_kv(tq, tw, tk, tl, return_scores=True, variant=v, g=g, topk=topk, c=c, scan_path=path)
        torch.cuda.synchronize()
        ref_i, ref_s = _oracle_ragged(variant, q, w, k, lens, g, topk, c)
        np.testing.assert_array_equal(i.cpu().numpy(), ref_i)
        np.testing.assert_array_equal(s.cpu().numpy(), ref_s)


def test_uniform_kv_call_equals_plain_call():
    B, Lq, Lk, g, topk, c = 4, 4, 2000, 4, 32, 64
    q, w, k = exact_random(43, B, Lq, Lk, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    a = pv.index_refine(tq, tw, tk, g, topk, c)
    b = pv.index_kv(tq, tw, tk, variant=pv.REFINE, g=g, topk=topk, c=c)
    pool, table = _paged(k, 128, 5)
    cc = pv.index_kv(tq, tw, _dev(pool), None, torch.from_numpy(table).cuda(), page_size=128, lk=Lk,
                     variant=pv.REFINE, g=g, topk=topk, c=c)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, cc)


def test_lengths_below_the_query_count_select_nothing_for_early_rows():
    """Dense rows whose position falls below 0 (seq_lens[b] < Lq) are empty;
    the others score the keys that exist."""
    B, Lq, Lk, topk = 2, 8, 64, 4
    q, w, k = exact_random(44, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([5, 64], dtype=np.int32)
    i = pv.index_kv(_dev(q), _dev(w), _dev(k), torch.from_numpy(lens).cuda(), variant=pv.DENSE, topk=topk)
    torch.cuda.synchronize()
    got = i.cpu().numpy()
    assert np.all(got[0, :3] == -1)                     # positions -3 .. -1
    ref = oracle.dense(q[:1, 3:], w[:1, 3:], k[:1, :5], topk)["indices"]
    np.testing.assert_array_equal(got[0, 3:], ref[0])
    np.testing.assert_array_equal(got[1], oracle.dense(q[1:], w[1:], k[1:], topk)["indices"][0])


def test_out_of_range_page_entries_read_the_clamped_page():
    """Table entries outside the pool are clamped into it (first or last
    page), so a malformed table cannot address outside the storage; the
    oracle runs on the keys those clamped pages hold."""
    B, Lq, Lk, g, topk, c, page = 3, 4, 700, 4, 16, 32, 64
    q, w, k = exact_random(51, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([700, 513, 290], dtype=np.int32)
    pool, table = _paged(k, page, 51)
    table = table.copy()
    table[0, 2] = -7
    table[1, 5] = pool.shape[0] + 5
    table[2, 0] = -1
    clamped = np.clip(table, 0, pool.shape[0] - 1)
    kl = np.zeros_like(k)
    for b in range(B):
        for s in range(Lk):
            kl[b, s] = pool[clamped[b, s // page], s % page]
    for variant, v in (("refine", pv.REFINE), ("dense", pv.DENSE)):
        i, s = pv.index_kv(_dev(q), _dev(w), _dev(pool), torch.from_numpy(lens).cuda(), torch.from_numpy(table).cuda(),
                           page_size=page, lk=Lk, return_scores=True, variant=v, g=g, topk=topk, c=c)
        torch.cuda.synchronize()
        ref_i, ref_s = _oracle_ragged(variant, q, w, kl, lens, g, topk, c)
        np.testing.assert_array_equal(i.cpu().numpy(), ref_i)
        np.testing.assert_array_equal(s.cpu().numpy(), ref_s)


def test_lengths_outside_the_capacity_are_clamped():
    """seq_lens above Lk act as Lk and negative ones as 0 (no keys: every row
    of that sequence is empty)."""
    B, Lq, Lk, g, topk, c = 3, 4, 400, 4, 16, 32
    q, w, k = exact_random(52, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([Lk + 100, -3, 250], dtype=np.int32)
    i, s = pv.index_kv(_dev(q), _dev(w), _dev(k), torch.from_numpy(lens).cuda(), return_scores=True,
                       variant=pv.REFINE, g=g, topk=topk, c=c)
    torch.cuda.synchronize()
    got_i, got_s = i.cpu().numpy(), s.cpu().numpy()
    assert np.all(got_i[1] == -1) and np.all(np.isneginf(got_s[1]))
    for b, n in ((0, Lk), (2, 250)):
        ref_i, ref_s = _oracle_ragged("refine", q[b:b + 1], w[b:b + 1], k[b:b + 1], np.array([n]), g, topk, c)
        np.testing.assert_array_equal(got_i[b], ref_i[0])
        np.testing.assert_array_equal(got_s[b], ref_s[0])


@pytest.mark.parametrize("path", ["fused", "split"])
def test_groups_before_their_sequence_start_are_empty(path):
    """A sequence shorter than the query block: whole groups sit before its
    first key (empty candidate sets; the member rows are all -1), the rest
    equal the oracle's prefill on that sequence. Lq - len is a multiple of g,
    so the groups that see keys form a prefill problem of their own."""
    B, Lq, Lk, g, topk, c = 2, 1100, 1100, 4, 16, 32
    q, w, k = exact_random(53, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([1100, 300], dtype=np.int32)
    r0 = Lq - 300
    for variant, v in (("refine", pv.REFINE), ("reuse", pv.REUSE)):
        i, s = pv.index_kv(_dev(q), _dev(w), _dev(k), torch.from_numpy(lens).cuda(), return_scores=True,
                           variant=v, g=g, topk=topk, c=c, scan_path=path)
        torch.cuda.synchronize()
        got_i, got_s = i.cpu().numpy(), s.cpu().numpy()
        assert np.all(got_i[1, :r0] == -1) and np.all(np.isneginf(got_s[1, :r0]))
        ref_i, ref_s = _oracle_ragged(variant, q[1:, r0:], w[1:, r0:], k[1:, :300], np.array([300]), g, topk, c)
        np.testing.assert_array_equal(got_i[1, r0:], ref_i[0])
        np.testing.assert_array_equal(got_s[1, r0:], ref_s[0])
        ref_i, ref_s = _oracle_ragged(variant, q[:1], w[:1], k[:1], np.array([Lk]), g, topk, c)
        np.testing.assert_array_equal(got_i[0], ref_i[0])
        np.testing.assert_array_equal(got_s[0], ref_s[0])


@pytest.mark.parametrize("agg,causal", [("first", False), ("last", False), ("mean", True)])
@pytest.mark.parametrize("page", [0, 64])
def test_ragged_aggregation_and_member_causal_reuse(agg, causal, page):
    """The first / last-member proxies and member-causal Reuse over ragged
    (and paged) keys, against the oracle run sequence by sequence."""
    B, Lq, Lk, g, topk, c = 3, 8, 900, 4, 24, 48
    q, w, k = exact_random(54, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([900, 611, 97], dtype=np.int32)
    variant = "reuse" if causal else "refine"
    cfg = pv.make_config(variant=pv.REUSE if causal else pv.REFINE, g=g, topk=topk, c=c, aggregation=agg,
                         member_causal=causal)
    tl = torch.from_numpy(lens).cuda()
    if page:
        pool, table = _paged(k, page, 54)
        i, s = pv.index_kv(_dev(q), _dev(w), _dev(pool), tl, torch.from_numpy(table).cuda(), page_size=page, lk=Lk,
                           cfg=cfg, return_scores=True)
    else:
        i, s = pv.index_kv(_dev(q), _dev(w), _dev(k), tl, cfg=cfg, return_scores=True)
    torch.cuda.synchronize()
    got_i, got_s = i.cpu().numpy(), s.cpu().numpy()
    for b in range(B):
        qb, wb, kb = q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]]
        if causal:
            r = oracle.reuse(qb, wb, kb, g, topk, agg=agg, member_causal=True)
        else:
            r = oracle.refine(qb, wb, kb, g, topk, c, agg=agg)
        np.testing.assert_array_equal(got_i[b], r["indices"][0], err_msg=f"{variant} {agg} b={b}")
        np.testing.assert_array_equal(got_s[b], r["scores"][0], err_msg=f"{variant} {agg} b={b}")


@pytest.mark.parametrize("path", ["auto", "split"])
@pytest.mark.parametrize("variant", ["refine", "reuse"])
def test_paged_prefill_with_many_groups(variant, path):
    """Paged prefill with 1000 groups: automatically the fused scan (its tile
    DMA reads every key through the page table); forced onto the split-key
    scan, each group gets a single workgroup (four waves sweeping its
    quarters from a staggered start), the longest case of that kernel's
    per-wave loop."""
    B, Lq, Lk, g, topk, c, page = 2, 2000, 2300, 4, 16, 32, 96  # 1000 groups
    q, w, k = exact_random(57, B, Lq, Lk, 64, 128, BF16)
    lens = np.array([2300, 2011], dtype=np.int32)
    pool, table = _paged(k, page, 58)
    v = {"refine": pv.REFINE, "reuse": pv.REUSE}[variant]
    i, s = pv.index_kv(_dev(q), _dev(w), _dev(pool), torch.from_numpy(lens).cuda(), torch.from_numpy(table).cuda(),
                       page_size=page, lk=Lk, return_scores=True, variant=v, g=g, topk=topk, c=c, scan_path=path)
    torch.cuda.synchronize()
    ref_i, ref_s = _oracle_ragged(variant, q, w, k, lens, g, topk, c)
    np.testing.assert_array_equal(i.cpu().numpy(), ref_i)
    np.testing.assert_array_equal(s.cpu().numpy(), ref_s)
