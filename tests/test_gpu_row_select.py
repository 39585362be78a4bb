"""GPU parity of the few-groups (decode) path against the oracle, aimed at
the block-wide row selects: the group rows (the threshold bin from the split
scan's coarse and fine score counts, the register-resident prefilter into
LDS, the radix select over the bin's keys, the fallbacks to the full row)
and the member rows of the split refine (held in registers up to
c = 4096, streamed beyond).

Exact inputs (q, k in {-3..3}/4, w powers of two) make every score exact, so
candidate sets, indices and scores must match bit for bit, ties included.
"""
import zlib

import numpy as np
import pytest

import oracle
from tests.parity import to_device
from tests.test_gpu_parity import _striped_keys
from workloads import BF16, exact_random, to_storage

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_refine_and_reuse(q, w, k, g, topk, c):
    tq, tw, tk = to_device(q, w, k)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True, return_candidates=True)
    r_i, r_s = pv.index_reuse(tq, tw, tk, g, topk, return_scores=True)
    torch.cuda.synchronize()
    ref = oracle.refine(q, w, k, g, topk, c)
    np.testing.assert_array_equal(f_n.cpu().numpy(), ref["cand_n"])
    np.testing.assert_array_equal(f_c.cpu().numpy(), ref["cand"])
    np.testing.assert_array_equal(f_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(f_s.cpu().numpy(), ref["scores"])
    ref = oracle.reuse(q, w, k, g, topk)
    np.testing.assert_array_equal(r_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(r_s.cpu().numpy(), ref["scores"])


# name, B, Lk, c, topk: member rows in registers (c <= 4096) or streamed
# (c > 4096); group rows selected in registers (prefix <= 16384), through
# the count-driven prefilter (prefix > 2c, the threshold bin and above within
# 12288 entries; the exact select then runs over the threshold bin's keys) or
# streamed (the rest)
CASES = [
    ("c4095_regs", 2, 9000, 4095, 1000),
    ("c4096_regs", 2, 9000, 4096, 2048),
    ("c4097_streamed", 2, 9000, 4097, 2048),
    ("c5000_streamed", 1, 12000, 5000, 3000),
    ("prefilter_c4096", 2, 20000, 4096, 2048),
    ("prefilter_c1024", 2, 30000, 1024, 256),
    ("streamed_row_c5000", 1, 20000, 5000, 2048),  # no prefilter (3c > LDS), row > 16384: streamed select
    ("k1_c1", 2, 3000, 1, 1),
    # one row of 100003 keys: the prefilter reads it in two register segments
    # (65536 entries each, the second ragged) and sums the counts of
    # hundreds of scan splits (both count levels loop over the splits)
    ("prefilter_two_segments", 1, 100003, 4096, 2048),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_decode_shapes_match_oracle_bitwise(case):
    name, B, Lk, c, topk = case
    q, w, k = exact_random(zlib.crc32(name.encode()) % 1000, B, 4, Lk, 64, 128, BF16)
    _check_refine_and_reuse(q, w, k, 4, topk, c)


@pytest.mark.parametrize("hot_sampled", [True, False], ids=["hot_every_16th", "cold_every_16th"])
def test_row_prefilter_on_periodic_hot_keys(hot_sampled):
    """Rows whose hot keys sit on every 16th position (or everywhere else):
    the threshold bin comes from the scan's exact counts, so either way the
    prefilter keeps exactly the entries at or above it."""
    Lk, c, topk = 40000, 1024, 256
    r = np.random.default_rng(21)
    q = to_storage(r.integers(1, 4, size=(1, 4, 64, 128)).astype(np.float64) / 4.0, BF16)
    w = np.ldexp(1.0, r.integers(-3, 1, size=(1, 4, 64))).astype(np.float32)
    k = _striped_keys(Lk, 5, hot_sampled, "pos")
    _check_refine_and_reuse(q, w, k, 4, topk, c)


def test_all_equal_scores_select_the_earliest_positions():
    """Every key equal: every score ties, and each row keeps the earliest
    positions (the common-prefix shortcut of the register select)."""
    B, Lk, c, topk = 2, 9000, 2048, 512
    q, w, _ = exact_random(31, B, 4, Lk, 64, 128, BF16)
    k = np.tile(exact_random(32, 1, 1, 1, 1, 128, BF16)[2], (B, Lk, 1))
    _check_refine_and_reuse(q, w, k, 4, topk, c)


def test_crowded_threshold_bin_falls_back_to_the_full_row():
    """All but the first 100 keys equal: the bin holding the c-th largest
    score holds about 40000 entries, more than the LDS prefilter takes, so
    the group select streams the full row (and ties go to the lower
    position)."""
    B, Lk, c, topk = 1, 40000, 1024, 256
    q, w, k = exact_random(33, B, 4, Lk, 64, 128, BF16)
    k[:, 100:] = k[:, 100:101]
    _check_refine_and_reuse(q, w, k, 4, topk, c)
