"""GPU parity of the O1-O3 diagnostics (pivot_index_stats) against the CPU
oracle (oracle/diagnostics.py) on index rows produced by the indexer:
integer overlaps, unions and intersections bit for bit; the score-mass
shares within the bound of fp32 summation, |err| <= 2 n 2^-24 (two sums of
at most n positive terms and one division, relative to a share <= 1)."""
import numpy as np
import pytest

from oracle import diagnostics as dg
from tests.parity import to_device
from workloads import BF16, exact_random, gauss_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check(idx, sc, g, d=1):
    ti, ts = torch.from_numpy(idx).cuda(), torch.from_numpy(sc).cuda()
    got = pv.index_stats(ti, ts, d=d, g=g)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got["overlap"].cpu().numpy(), dg.overlap(idx, d))
    u, i = dg.group_sets(idx, g)
    np.testing.assert_array_equal(got["union"].cpu().numpy(), u)
    np.testing.assert_array_equal(got["inter"].cpu().numpy(), i)
    m = got["mass"].cpu().numpy().astype(np.float64)
    ref = dg.mass(idx, sc)
    n = (idx >= 0).sum(-1)[..., None]
    assert np.array_equal(np.isnan(m), np.isnan(ref))
    ok = ~np.isnan(ref)
    bound = np.broadcast_to(2 * n * 2.0 ** -24 + 2.0 ** -24, m.shape)
    assert np.all(np.abs(m - ref)[ok] <= bound[ok])


@pytest.mark.parametrize("variant", ["dense", "reuse", "refine"])
@pytest.mark.parametrize("seed", [0, 1])
def test_stats_of_indexer_rows_match_oracle(variant, seed):
    B, L, g, topk, c = 2, 700, 8, 32, 64
    q, w, k = exact_random(seed, B, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    if variant == "dense":
        i, s = pv.index_dense(tq, tw, tk, topk, return_scores=True)
    elif variant == "reuse":
        i, s = pv.index_reuse(tq, tw, tk, g, topk, return_scores=True)
    else:
        i, s = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True)
    torch.cuda.synchronize()
    idx, sc = i.cpu().numpy(), s.cpu().numpy()
    sc = np.where(idx >= 0, sc, 0.0).astype(np.float32)
    for d in (1, g - 1):
        _check(idx, sc, g, d)


@pytest.mark.parametrize("k,g", [(2048, 8), (1000, 16), (37, 5), (4096, 4), (3, 2)])
def test_stats_edge_widths(k, g):
    r = np.random.default_rng(k)
    B, Lq = 2, 3 * g + 1
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    sc = np.zeros((B, Lq, k), dtype=np.float32)
    for b in range(B):
        for t in range(Lq):
            n = int(r.integers(0, k + 1)) if t % 3 else k       # some full, some short, some empty rows
            pos = np.sort(r.choice(4 * k, size=n, replace=False)).astype(np.int32)
            idx[b, t, :n] = pos
            sc[b, t, :n] = (r.random(n) ** 4).astype(np.float32)  # long-tailed
            if t == 1:
                sc[b, t, :n] = 1.0                              # ties everywhere
    _check(idx, sc, g, 1)
    _check(idx, sc, g, 2)


def test_stats_on_gaussian_refine_rows():
    L, g, topk, c = 600, 8, 24, 48
    q, w, k = gauss_random(5, 1, L, L, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    i, s = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True)
    torch.cuda.synchronize()
    idx, sc = i.cpu().numpy(), s.cpu().numpy()
    _check(idx, np.where(idx >= 0, sc, 0.0).astype(np.float32), g)


@pytest.mark.parametrize("span", [1 << 16, 1 << 17, (1 << 17) + 1, 1 << 24])
def test_stats_positions_around_the_bitmap_limit(span):
    """Rows and groups whose positions stay below 2^17 take the bitmap kernels,
    the others the sorted-array search and the merge kernel; a call mixes
    both, and some rows hold position span - 1 (2^17 itself for the third
    case: the first value past the bitmaps)."""
    k, g = 512, 8
    B, Lq = 2, 3 * g + 5
    r = np.random.default_rng(span % 1009)
    idx = np.full((B, Lq, k), -1, dtype=np.int32)
    sc = np.zeros((B, Lq, k), dtype=np.float32)
    for b in range(B):
        for t in range(Lq):
            hi = span if (t // g) % 2 == 0 else min(span, 1 << 12)  # alternate groups: wide, narrow
            n = int(r.integers(1, k + 1)) if t % 4 else k
            pos = r.choice(hi, size=n, replace=False)
            if t % 3 == 0:
                pos[0] = hi - 1
            pos = np.unique(pos).astype(np.int32)
            idx[b, t, :pos.size] = pos
            sc[b, t, :pos.size] = r.random(pos.size).astype(np.float32)
    # neighbouring rows share about half their entries, so overlaps are not all zero
    idx[:, 1::2] = np.where(r.random(idx[:, 1::2].shape) < 0.5, idx[:, 0:-1:2][:, : idx[:, 1::2].shape[1]], idx[:, 1::2])
    for b in range(B):
        for t in range(Lq):
            row = idx[b, t]
            v = np.unique(row[row >= 0])
            idx[b, t] = -1
            idx[b, t, :v.size] = v
            sc[b, t, v.size:] = 0.0
    _check(idx, sc, g, 1)
    _check(idx, sc, g, 3)


def test_mass_with_crowded_and_sparse_bins():
    """Score mass where the bin of a sought rank holds many equal keys (the
    search falls back to all keys) next to rows whose bins are small (the
    search runs over the compacted bin)."""
    k, g = 2048, 8
    B, Lq = 1, 16
    r = np.random.default_rng(77)
    idx = np.tile(np.arange(k, dtype=np.int32), (B, Lq, 1))
    sc = np.zeros((B, Lq, k), dtype=np.float32)
    for t in range(Lq):
        if t % 2 == 0:  # crowded: most scores equal, a few far above
            sc[0, t] = 1.0
            sc[0, t, r.choice(k, size=40, replace=False)] = 100.0 + r.random(40).astype(np.float32)
        else:           # spread: log-uniform over six decades
            sc[0, t] = np.exp(r.uniform(-7, 7, size=k)).astype(np.float32)
    _check(idx, sc, g, 1)
