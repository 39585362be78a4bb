"""GPU parity of the variant knobs against the CPU oracle, through the C ABI's
config call (``pivot_index``):

  * proxy aggregation (the ablation over how a group becomes its proxy, in the
    summary's Ablation Studies): the per-head mean of eq. (4), or the first /
    last member's own q and w;
  * member-causal Reuse (eq. (6) with each member's own bound s <= t), built
    from the group's top-(k + g - 1) and a per-member select;
  * the short-context guardrail (PIVOT falls back to dense DSA below some
    context length; summary, Efficiency Results), resolved from lk.

Exact inputs (q, k in {-3..3}/4, w powers of two) make every score exact on
both sides, so indices, scores and candidate sets must match bit for bit on the
exact-order kernels and on the bf16 MFMA kernels, on the fused per-group scan
and on the split-key path used for few groups.
"""
import zlib

import numpy as np
import pytest

import oracle
from tests.parity import to_device, bf16_tensor_bits
from workloads import BF16, F32, exact_random, gauss_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(params=["fused", "split"])
def scan_path(request):
    """The fused per-group scan or the split-key scan + block selects
    (pivot_config.scan_path); the exact-order kernels ignore it."""
    return request.param


CASES = [
    # name, B, Lq, Lk, H, d, g, topk, c, dtype
    ("mfma_ragged", 1, 700, 700, 64, 128, 8, 32, 64, BF16),
    ("mfma_g4", 1, 1500, 1500, 64, 128, 4, 16, 32, BF16),
    ("mfma_decode", 4, 4, 777, 64, 128, 4, 24, 48, BF16),
    ("mfma_L_below_k", 1, 40, 40, 64, 128, 8, 64, 128, BF16),
    ("exact_order_f32", 1, 300, 300, 2, 12, 6, 7, 20, F32),
    ("exact_order_bf16", 2, 37, 37, 3, 8, 4, 5, 9, BF16),
    ("exact_order_decode", 3, 4, 300, 2, 16, 4, 6, 12, BF16),
]


def _data(case):
    name, B, Lq, Lk, H, d, g, topk, c, dt = case
    return exact_random(zlib.crc32(name.encode()) % 1000, B, Lq, Lk, H, d, dt)


def _cpu(t):
    return None if t is None else t.cpu().numpy()


@pytest.mark.parametrize("agg", ["first", "last", "mean"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_aggregation_bitwise(case, agg, scan_path):
    name, B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    tq, tw, tk = to_device(q, w, k)
    r_i, r_s = pv.index(tq, tw, tk, variant=pv.REUSE, g=g, topk=topk, aggregation=agg, return_scores=True,
                        scan_path=scan_path)
    f_i, f_s, f_c, f_n = pv.index(tq, tw, tk, variant=pv.REFINE, g=g, topk=topk, c=c, aggregation=agg,
                                  return_scores=True, return_candidates=True, scan_path=scan_path)
    torch.cuda.synchronize()
    ref = oracle.reuse(q, w, k, g, topk, agg=agg)
    np.testing.assert_array_equal(_cpu(r_i), ref["indices"])
    np.testing.assert_array_equal(_cpu(r_s), ref["scores"])
    ref = oracle.refine(q, w, k, g, topk, c, agg=agg)
    np.testing.assert_array_equal(_cpu(f_n), ref["cand_n"])
    np.testing.assert_array_equal(_cpu(f_c), ref["cand"])
    np.testing.assert_array_equal(_cpu(f_i), ref["indices"])
    np.testing.assert_array_equal(_cpu(f_s), ref["scores"])


@pytest.mark.parametrize("agg", ["mean", "first", "last"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_member_causal_reuse_bitwise(case, agg, scan_path):
    name, B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = _data(case)
    tq, tw, tk = to_device(q, w, k)
    i, s = pv.index(tq, tw, tk, variant=pv.REUSE, g=g, topk=topk, aggregation=agg, member_causal=True,
                    return_scores=True, scan_path=scan_path)
    torch.cuda.synchronize()
    ref = oracle.reuse(q, w, k, g, topk, agg=agg, member_causal=True)
    np.testing.assert_array_equal(_cpu(i), ref["indices"])
    np.testing.assert_array_equal(_cpu(s), ref["scores"])
    # every entry respects its own row's causal bound
    t = np.arange(Lq)[None, :, None] + (Lk - Lq)
    got = _cpu(i)
    assert np.all((got == -1) | (got <= t))


def test_member_causal_reuse_float_inputs_match_plain_reuse_on_last_members(scan_path):
    """On Gaussian inputs the last member of a group has the same bound as the
    group, so its member-causal row is the plain Reuse row (same kernels, same
    scores), and every earlier member's row lies inside the group's top-(k+g-1)."""
    L, g, topk = 600, 8, 24
    q, w, k = gauss_random(21, 1, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    mc = _cpu(pv.index(tq, tw, tk, variant=pv.REUSE, g=g, topk=topk, member_causal=True, scan_path=scan_path))
    plain = _cpu(pv.index_reuse(tq, tw, tk, g, topk, scan_path=scan_path))
    wide = _cpu(pv.index_reuse(tq, tw, tk, g, topk + g - 1, scan_path=scan_path))
    torch.cuda.synchronize()
    for m in range(-(-L // g)):
        last = min((m + 1) * g, L) - 1
        np.testing.assert_array_equal(mc[0, last], plain[0, last])
        pool_set = set(wide[0, last][wide[0, last] >= 0].tolist())
        for t in range(m * g, last + 1):
            row = mc[0, t][mc[0, t] >= 0]
            assert len(row) == min(topk, t + 1)
            assert set(row.tolist()) <= pool_set
            assert np.all(row <= t)


def test_pool_aggregation_bitwise():
    for dt, H, d in ((BF16, 64, 128), (F32, 3, 8)):
        q, w, _ = gauss_random(3, 2, 45, 45, H, d, dt)
        tq, tw, _ = to_device(q, w, q[:, :, 0])
        for g in (1, 4, 7):
            for agg in ("first", "last"):
                qb, wb = pv.pool(tq, tw, g, aggregation=agg)
                oq, ow = oracle.pool(q, w, g, agg=agg)
                if dt == BF16:
                    from workloads import f32_to_bf16_bits
                    np.testing.assert_array_equal(bf16_tensor_bits(qb), f32_to_bf16_bits(oq))
                else:
                    np.testing.assert_array_equal(qb.cpu().numpy(), oq)
                np.testing.assert_array_equal(wb.cpu().numpy(), ow)


@pytest.mark.parametrize("auto_variant", [pv.REUSE, pv.REFINE])
def test_auto_guardrail_picks_dense_below_the_threshold(auto_variant):
    L, g, topk, c = 700, 8, 32, 64
    q, w, k = exact_random(31, 1, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    below = pv.make_config(variant=pv.AUTO, g=g, topk=topk, c=c, auto_variant=auto_variant, dense_below=L + 1)
    above = pv.make_config(variant=pv.AUTO, g=g, topk=topk, c=c, auto_variant=auto_variant, dense_below=L)
    assert pv.resolve_variant(1, L, L, 64, 128, torch.bfloat16, below) == pv.DENSE
    assert pv.resolve_variant(1, L, L, 64, 128, torch.bfloat16, above) == auto_variant
    i_below, c_below, _ = pv.index(tq, tw, tk, below, return_candidates=True)
    i_above = pv.index(tq, tw, tk, above)
    torch.cuda.synchronize()
    assert c_below is None
    np.testing.assert_array_equal(_cpu(i_below), oracle.dense(q, w, k, topk)["indices"])
    ref = oracle.refine(q, w, k, g, topk, c) if auto_variant == pv.REFINE else oracle.reuse(q, w, k, g, topk)
    np.testing.assert_array_equal(_cpu(i_above), ref["indices"])


def test_auto_member_causal_applies_only_when_resolved_to_reuse():
    L, g, topk = 300, 4, 16
    q, w, k = exact_random(32, 1, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    cfg = pv.make_config(variant=pv.AUTO, g=g, topk=topk, auto_variant=pv.REUSE, member_causal=True,
                         dense_below=L)
    got = _cpu(pv.index(tq, tw, tk, cfg))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, oracle.reuse(q, w, k, g, topk, member_causal=True)["indices"])
