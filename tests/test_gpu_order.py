"""GPU parity of rank-ordered rows (pivot_config.order = PIVOT_ORDER_SCORE)
against the CPU oracle, through the C ABI.

A rank-ordered row lists T_t = TopK(I_{t,:}, k) (PIVOT paper summary, eq. (1);
eqs. (6) and (9) for Reuse and Refine) by score, highest first, equal scores
by lower position, then -1. The oracle's rows are put in that order by
``oracle.rank_order``, itself pinned to the hand-worked example. On exact
inputs (q, k in {-3..3}/4, w powers of two; many equal scores) indices and
scores must match bit for bit: the fused and the split MFMA scans, the
exact-order kernels, every row width the rank pass compiles (1 .. 8192
entries), member-causal Reuse rows of varying length, paged ragged keys and
the allocation-free entry point. At the MTP decode workload's full size
(float inputs) the rank-ordered rows must be the position-ordered rows of
the same call, permuted into rank order.
"""
import zlib

import numpy as np
import pytest

import oracle
from tests.parity import to_device
from workloads import BF16, DECODE, F32, exact_random, generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _np(t):
    return t.cpu().numpy()


def _variant(name):
    return {"dense": pv.DENSE, "reuse": pv.REUSE, "causal": pv.REUSE, "refine": pv.REFINE}[name]


def _gpu(tq, tw, tk, name, g, topk, c, order="score", **kw):
    i, s = pv.index(tq, tw, tk, variant=_variant(name), g=1 if name == "dense" else g, topk=topk,
                    c=c if name == "refine" else 2 * topk, member_causal=name == "causal", order=order,
                    return_scores=True, **kw)
    torch.cuda.synchronize()
    return _np(i), _np(s)


def _oracle(q, w, k, name, g, topk, c):
    if name == "dense":
        return oracle.dense(q, w, k, topk, order="score")
    if name == "refine":
        return oracle.refine(q, w, k, g, topk, c, order="score")
    return oracle.reuse(q, w, k, g, topk, member_causal=name == "causal", order="score")


def _assert_rank_rows(idx, sc):
    """Rank order within every row: scores non-increasing, equal scores by
    ascending position, the -1 padding (score -inf) after every entry."""
    valid = idx >= 0
    n = valid.sum(axis=-1)
    pos = np.arange(idx.shape[-1])
    assert np.array_equal(valid, pos < n[..., None]), "padding must follow the entries"
    assert np.all(np.isneginf(sc[~valid]))
    a_s, b_s = sc[..., :-1], sc[..., 1:]
    a_i, b_i = idx[..., :-1], idx[..., 1:]
    both = valid[..., 1:]
    assert np.all(~both | (a_s >= b_s)), "scores must not increase along a row"
    assert np.all(~both | (a_s > b_s) | (a_i < b_i)), "equal scores must list the lower position first"


MFMA_CASES = [
    # name, B, Lq, Lk, g, topk, c  (H = 64, d = 128 bf16: fused scan from 256 groups, split scan below)
    ("fused_L4096", 1, 4096, 4096, 8, 64, 128),
    ("fused_wide_rows", 1, 2048, 2048, 8, 700, 1500),
    ("decode_split", 4, 4, 8192, 4, 512, 1024),
]


@pytest.mark.parametrize("heads", [64, 32])
@pytest.mark.parametrize("variant", ["dense", "reuse", "causal", "refine"])
@pytest.mark.parametrize("case", MFMA_CASES, ids=[c[0] for c in MFMA_CASES])
def test_mfma_rank_rows_bitwise(case, variant, heads):
    name, B, Lq, Lk, g, topk, c = case
    q, w, k = exact_random(zlib.crc32(name.encode()) % 1000, B, Lq, Lk, heads, 128, BF16)
    print(f"[order] {name} {variant} H={heads}", flush=True)
    tq, tw, tk = to_device(q, w, k)
    gi, gs = _gpu(tq, tw, tk, variant, g, topk, c)
    ref = _oracle(q, w, k, variant, g, topk, c)
    np.testing.assert_array_equal(gi, ref["indices"])
    np.testing.assert_array_equal(gs, ref["scores"])
    _assert_rank_rows(gi, gs)
    # the position-ordered call returns the same entries
    pi, ps = _gpu(tq, tw, tk, variant, g, topk, c, order="position")
    for x, y in ((gi, pi), (gs, ps)):
        np.testing.assert_array_equal(np.sort(x, axis=-1), np.sort(y, axis=-1))


# Every compiled row width of the rank pass (padded to 2^0 .. 2^13 entries),
# on the exact-order kernels (small heads and dims keep the oracle cheap).
WIDTHS = [1, 2, 3, 5, 16, 33, 100, 255, 256, 600, 1025, 2048, 3000, 5000, 8192]


@pytest.mark.parametrize("topk", WIDTHS)
def test_rank_rows_every_width_bitwise(topk):
    L = max(2 * topk, 64)
    q, w, k = exact_random(1000 + topk, 1, L, L, 2, 8, F32, qk_levels=2)
    tq, tw, tk = to_device(q, w, k)
    gi, gs = _gpu(tq, tw, tk, "dense", 1, topk, 0)
    ref = _oracle(q, w, k, "dense", 1, topk, 0)
    np.testing.assert_array_equal(gi, ref["indices"])
    np.testing.assert_array_equal(gs, ref["scores"])
    gi, gs = _gpu(tq, tw, tk, "refine", 4, topk, min(2 * topk, 8192))
    ref = _oracle(q, w, k, "refine", 4, topk, min(2 * topk, 8192))
    np.testing.assert_array_equal(gi, ref["indices"])
    np.testing.assert_array_equal(gs, ref["scores"])


def test_equal_scores_rank_by_position():
    """Every key equal: each row's scores are all equal, so rank order is
    ascending position, the same rows as the default order."""
    L, g, topk = 1024, 8, 100
    q, w, _ = exact_random(7, 1, L, L, 64, 128, BF16)
    k = np.broadcast_to(exact_random(8, 1, 1, 1, 64, 128, BF16)[2], (1, L, 128)).copy()
    tq, tw, tk = to_device(q, w, k)
    for variant in ("dense", "reuse", "refine"):
        ri, rs = _gpu(tq, tw, tk, variant, g, topk, 2 * topk)
        pi, ps = _gpu(tq, tw, tk, variant, g, topk, 2 * topk, order="position")
        np.testing.assert_array_equal(ri, pi)
        np.testing.assert_array_equal(rs, ps)


@pytest.mark.parametrize("H,d,dt", [(64, 128, BF16), (3, 8, F32)])
def test_paged_ragged_rank_rows_bitwise(H, d, dt):
    B, Lq, Lk, g, topk, c, page = 3, 4, 3000, 4, 300, 600, 64
    q, w, k = exact_random(31, B, Lq, Lk, H, d, dt)
    lens = np.array([3000, 1700, 901], dtype=np.int32)
    maxp = -(-Lk // page)
    perm = np.random.default_rng(5).permutation(B * maxp).astype(np.int32).reshape(B, maxp)
    pool = np.zeros((B * maxp, page, d), dtype=k.dtype)
    for b in range(B):
        for j in range(maxp):
            rows = k[b, j * page:(j + 1) * page]
            pool[perm[b, j], :rows.shape[0]] = rows
    tq, tw, tpool = to_device(q, w, pool)
    i, s = pv.index_kv(tq, tw, tpool, torch.from_numpy(lens).cuda(), torch.from_numpy(perm).cuda(),
                       page_size=page, lk=Lk, variant=pv.REFINE, g=g, topk=topk, c=c, order="score",
                       return_scores=True)
    torch.cuda.synchronize()
    i, s = _np(i), _np(s)
    for b in range(B):
        ref = oracle.refine(q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]], g, topk, c, order="score")
        np.testing.assert_array_equal(i[b], ref["indices"][0], err_msg=f"sequence {b}")
        np.testing.assert_array_equal(s[b], ref["scores"][0], err_msg=f"sequence {b}")


def test_static_entry_rank_rows_bitwise():
    L, g, topk, c = 2048, 8, 64, 128
    q, w, k = exact_random(77, 1, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    cfg = pv.make_config(variant=pv.REFINE, g=g, topk=topk, c=c, order="score")
    i, s = pv.index_static(tq, tw, tk, cfg, return_scores=True)
    torch.cuda.synchronize()
    ref = oracle.refine(q, w, k, g, topk, c, order="score")
    np.testing.assert_array_equal(_np(i), ref["indices"])
    np.testing.assert_array_equal(_np(s), ref["scores"])


def test_decode_workload_rank_rows_permute_the_default_rows():
    """MTP decode at full size (B = 32 sequences of 65536 keys, k = 2048,
    c = 4096, float inputs): the rank-ordered call returns each row of the
    position-ordered call, permuted into rank order."""
    W = DECODE
    q, w, k = generate(W)
    tq, tw, tk = to_device(q, w, k)
    pi, ps = _gpu(tq, tw, tk, "refine", W.g, W.topk, W.c, order="position")
    ri, rs = _gpu(tq, tw, tk, "refine", W.g, W.topk, W.c)
    _assert_rank_rows(ri, rs)
    ei, es = oracle.rank_order(pi, ps)  # the ordering rule applied to this call's own rows
    np.testing.assert_array_equal(ri, ei)
    np.testing.assert_array_equal(rs, es)
