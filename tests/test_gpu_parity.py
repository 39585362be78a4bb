"""GPU parity against the CPU oracle on small and edge-case problems.

Two kernel families are checked:
  * the exact-order kernels (f32, and bf16 shapes other than H=64, d=128):
    their scores follow the oracle's fp32 order, so indices, scores and
    candidate sets must match bit for bit on any input;
  * the bf16 MFMA kernels (H=64, d=128): bit for bit on inputs whose every
    sum is exact (q, k in {-3..3}/4, w powers of two), within the float rule
    (tests/parity.py) on Gaussian inputs.
Sizes span several 64-key tiles, ragged tails, buffer compactions and the
degenerate cases (L < k, c >= prefix, g = 1, g > L, decode shapes, ties).
"""
import zlib

import numpy as np
import pytest

import oracle
from oracle import brute
from tests import checks
from tests.parity import compare_row, check_candidates, to_device, bf16_tensor_bits
from workloads import BF16, F32, TINY, exact_random, gauss_random, generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _gpu_all(q, w, k, g, topk, c, path="auto"):
    tq, tw, tk = to_device(q, w, k)
    d_i, d_s = pv.index_dense(tq, tw, tk, topk, return_scores=True, scan_path=path)
    r_i, r_s = pv.index_reuse(tq, tw, tk, g, topk, return_scores=True, scan_path=path)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True, return_candidates=True,
                                         scan_path=path)
    torch.cuda.synchronize()
    cpu = lambda t: t.cpu().numpy()
    return {"dense": (cpu(d_i), cpu(d_s)), "reuse": (cpu(r_i), cpu(r_s)),
            "refine": (cpu(f_i), cpu(f_s), cpu(f_c), cpu(f_n))}


def _oracle_all(q, w, k, g, topk, c):
    return {"dense": oracle.dense(q, w, k, topk), "reuse": oracle.reuse(q, w, k, g, topk),
            "refine": oracle.refine(q, w, k, g, topk, c)}


def _assert_bitwise(gpu, ref):
    for v in ("dense", "reuse", "refine"):
        np.testing.assert_array_equal(gpu[v][0], ref[v]["indices"], err_msg=f"{v} indices")
        np.testing.assert_array_equal(gpu[v][1], ref[v]["scores"], err_msg=f"{v} scores")
    np.testing.assert_array_equal(gpu["refine"][3], ref["refine"]["cand_n"])
    np.testing.assert_array_equal(gpu["refine"][2], ref["refine"]["cand"])


EXACT_ORDER_CASES = [
    # name, B, Lq, Lk, H, d, g, topk, c, dtype
    ("ragged_bf16", 2, 37, 37, 3, 8, 4, 5, 9, BF16),
    ("f32_many_tiles", 1, 300, 300, 2, 12, 6, 7, 20, F32),
    ("decode_shape", 3, 4, 300, 2, 16, 4, 6, 12, BF16),
    ("two_decode_groups", 2, 6, 200, 3, 8, 3, 5, 10, F32),
    ("L_below_k", 1, 10, 10, 2, 8, 4, 16, 32, F32),
    ("c_covers_prefix", 1, 90, 90, 2, 8, 5, 6, 200, BF16),
    ("g1", 1, 70, 70, 2, 8, 1, 4, 8, F32),
    ("g_beyond_L", 1, 20, 20, 2, 8, 32, 3, 6, F32),
    ("topk1", 1, 130, 130, 2, 8, 4, 1, 1, BF16),
    ("compactions", 1, 2000, 2000, 2, 8, 8, 8, 16, F32),
    ("k_at_cap_edges", 1, 700, 700, 2, 8, 4, 64, 65, BF16),
]


@pytest.mark.parametrize("case", EXACT_ORDER_CASES, ids=[c[0] for c in EXACT_ORDER_CASES])
def test_exact_order_kernels_match_oracle_bitwise(case):
    name, B, Lq, Lk, H, d, g, topk, c, dt = case
    q, w, k = gauss_random(zlib.crc32(name.encode()) % 1000, B, Lq, Lk, H, d, dt)
    _assert_bitwise(_gpu_all(q, w, k, g, topk, c), _oracle_all(q, w, k, g, topk, c))


def test_tiny_workload_bitwise():
    """L=512, H=4, d=32, g=4, k=16, c=32, f32 Gaussian: the exact-order path."""
    W = TINY
    q, w, k = generate(W)
    _assert_bitwise(_gpu_all(q, w, k, W.g, W.topk, W.c), _oracle_all(q, w, k, W.g, W.topk, W.c))


MFMA_EXACT_CASES = [
    # name, B, Lq, Lk, g, topk, c, w_levels
    ("ragged_700", 1, 700, 700, 8, 32, 64, (-3, 0)),
    ("g4_compactions", 1, 1500, 1500, 4, 16, 32, (-3, 0)),
    ("g3_unit_w", 1, 200, 200, 3, 10, 20, (0, 0)),
    ("decode_batch", 4, 4, 777, 4, 24, 48, (-3, 0)),
    ("L_below_k", 1, 40, 40, 8, 64, 128, (-3, 0)),
    ("g16", 2, 160, 160, 16, 12, 40, (-3, 0)),
]


@pytest.fixture(params=["fused", "split"])
def scan_path(request):
    """Run a test on the fused per-group scan ("fused") and on the split-key
    scan + block selects used for few groups ("split")."""
    return request.param


@pytest.mark.parametrize("case", MFMA_EXACT_CASES, ids=[c[0] for c in MFMA_EXACT_CASES])
def test_mfma_kernels_bitwise_on_exact_inputs(case, scan_path):
    name, B, Lq, Lk, g, topk, c, wl = case
    q, w, k = exact_random(zlib.crc32(name.encode()) % 1000, B, Lq, Lk, 64, 128, BF16, w_levels=wl)
    _assert_bitwise(_gpu_all(q, w, k, g, topk, c, scan_path), _oracle_all(q, w, k, g, topk, c))


MFMA32_EXACT_CASES = [c for c in MFMA_EXACT_CASES if c[0] in ("ragged_700", "g4_compactions", "decode_batch",
                                                                 "L_below_k", "g16")]


@pytest.mark.parametrize("case", MFMA32_EXACT_CASES, ids=[c[0] for c in MFMA32_EXACT_CASES])
def test_mfma_32_heads_bitwise_on_exact_inputs(case, scan_path):
    """The MFMA kernels compiled for 32 indexer heads (two 16-head row blocks
    per group): bit for bit on exact inputs, both scan paths."""
    name, B, Lq, Lk, g, topk, c, wl = case
    q, w, k = exact_random(zlib.crc32(name.encode()) % 1000 + 7, B, Lq, Lk, 32, 128, BF16, w_levels=wl)
    _assert_bitwise(_gpu_all(q, w, k, g, topk, c, scan_path), _oracle_all(q, w, k, g, topk, c))


def test_mfma_all_equal_keys_fall_back_to_position(scan_path):
    L, g, topk, c = 200, 8, 16, 32
    q, w, _ = exact_random(5, 1, L, L, 64, 128, BF16)
    k = np.tile(exact_random(6, 1, 1, 1, 1, 128, BF16)[2], (1, L, 1))
    gpu = _gpu_all(q, w, k, g, topk, c, scan_path)
    for v in ("dense", "refine"):
        idx = gpu[v][0][0]
        for t in range(L):
            n = min(topk, t + 1)
            np.testing.assert_array_equal(idx[t, :n], np.arange(n))
    np.testing.assert_array_equal(gpu["reuse"][0], oracle.reuse(q, w, k, g, topk)["indices"])


@pytest.mark.parametrize("seed,H", [(1, 64), (2, 64), (3, 32)])
def test_mfma_kernels_float_rule_on_gaussian_inputs(seed, H, scan_path):
    B, L, g, topk, c = 1, 600, 8, 24, 48
    q, w, k = gauss_random(seed, B, L, L, H, 128, BF16)
    gpu = _gpu_all(q, w, k, g, topk, c, scan_path)
    ref = _oracle_all(q, w, k, g, topk, c)
    qf = q.view(np.uint16)
    from workloads import bf16_bits_to_f32
    q64 = bf16_bits_to_f32(qf).astype(np.float64)
    k64 = bf16_bits_to_f32(k).astype(np.float64)
    w64 = w.astype(np.float64)
    I = brute.score_matrix(q64[0], w64[0], k64[0])
    qbar, wbar = brute.proxy(q, w, g, BF16)
    Ibar = brute.score_matrix(qbar[0], wbar[0], k64[0])
    G = -(-L // g)
    for t in range(L):
        compare_row(gpu["dense"][0][0, t], gpu["dense"][1][0, t], ref["dense"]["indices"][0, t],
                    ref["dense"]["scores"][0, t], lambda p: I[t, p], f"dense row {t}")
        m = t // g
        compare_row(gpu["reuse"][0][0, t], gpu["reuse"][1][0, t], ref["reuse"]["indices"][0, t],
                    ref["reuse"]["scores"][0, t], lambda p: Ibar[m, p], f"reuse row {t}")
    # Refine: candidates at the boundary only; member rows judged on the GPU's C
    f_i, f_s, f_c, f_n = gpu["refine"]
    ref_given = oracle.refine(q, w, k, g, topk, c, cand_in=f_c, cand_in_n=f_n)
    for m in range(G):
        tl = min((m + 1) * g, L) - 1
        n = f_n[0, m]
        check_candidates(f_c[0, m, :n], ref["refine"]["cand"][0, m, :ref["refine"]["cand_n"][0, m]],
                         Ibar[m, :tl + 1], f"C of group {m}")
    for t in range(L):
        compare_row(f_i[0, t], f_s[0, t], ref_given["indices"][0, t], ref_given["scores"][0, t],
                    lambda p: I[t, p], f"refine row {t}")


def test_pool_bitwise():
    for dt, H, d in ((BF16, 64, 128), (F32, 3, 8), (BF16, 2, 16)):
        q, w, _ = gauss_random(3, 2, 45, 45, H, d, dt)
        tq, tw, _ = to_device(q, w, q[:, :, 0])
        for g in (1, 4, 7):
            qb, wb = pv.pool(tq, tw, g)
            oq, ow = oracle.pool(q, w, g)
            got = bf16_tensor_bits(qb) if dt == BF16 else qb.cpu().numpy()
            if dt == BF16:
                from workloads import f32_to_bf16_bits
                np.testing.assert_array_equal(got, f32_to_bf16_bits(oq))
            else:
                np.testing.assert_array_equal(got, oq)
            np.testing.assert_array_equal(wb.cpu().numpy(), ow)


@pytest.mark.parametrize("H,d,dt", [(64, 128, BF16), (3, 8, F32)])
def test_proxy_score_rows(H, d, dt):
    B, L, g = 1, 333, 8
    q, w, k = gauss_random(4, B, L, L, H, d, dt)
    tq, tw, tk = to_device(q, w, k)
    qb, wb = pv.pool(tq, tw, g)
    rows = pv.proxy_scores(qb, wb, tk, g, L).cpu().numpy()
    G = -(-L // g)
    for m in range(G):
        ref = oracle.proxy_row(q, w, k, g, 0, m)
        tl = len(ref)
        if (H, d) == (64, 128):
            np.testing.assert_allclose(rows[0, m, :tl], ref, rtol=2e-5, atol=1e-5 * np.abs(ref).max())
        else:
            np.testing.assert_array_equal(rows[0, m, :tl], ref)
        assert np.all(np.isneginf(rows[0, m, tl:]))


def test_repeat_runs_are_bit_identical():
    q, w, k = gauss_random(8, 1, 1000, 1000, 64, 128, BF16)
    a = _gpu_all(q, w, k, 8, 32, 64)
    b = _gpu_all(q, w, k, 8, 32, 64)
    for v in a:
        for x, y in zip(a[v], b[v]):
            np.testing.assert_array_equal(x, y)


def test_side_stream_and_preallocated_workspace():
    q, w, k = gauss_random(9, 1, 256, 256, 64, 128, BF16)
    tq, tw, tk = to_device(q, w, k)
    need = pv.workspace_size(pv.REFINE, 1, 256, 256, 64, 128, torch.bfloat16, 8, 16, 32)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        idx = pv.index_refine(tq, tw, tk, 8, 16, 32, workspace=ws, stream=s)
    s.synchronize()
    ref = pv.index_refine(tq, tw, tk, 8, 16, 32)
    torch.cuda.synchronize()
    assert torch.equal(idx, ref)
    with pytest.raises(pv.PivotError):
        pv.index_refine(tq, tw, tk, 8, 16, 32, workspace=ws[:need // 2])


# The fused scan samples 256-key tiles 0, 32, 64, ... (while a group's prefix
# spans at most 512 tiles); the few-groups row select samples every 16th
# score. Keys that are hot exactly where a sample looks (or exactly where it
# does not) make the sampled threshold too high (forcing the exact re-run)
# or too low (forcing buffer compactions).
SCAN_TILE, SAMPLE_STRIDE, SAMPLE_SIGMAS = 256, 32, 6.0


def _striped_keys(L, seed, hot_sampled, stripe="tile"):
    """Exact keys where the positions a threshold sample looks at are all
    "hot" (hot_sampled=True) or all "cold" (False) relative to the rest: the
    256-key tiles at multiples of 32 (the fused scan's sample, stripe="tile")
    or every 16th position (the block select's sample, stripe="pos"). With
    positive queries, hot keys score far above cold ones."""
    r = np.random.default_rng([seed, 7])
    cold = r.integers(-3, 4, size=(1, L, 128)).astype(np.float64) / 4.0
    hot = r.integers(2, 4, size=(1, L, 128)).astype(np.float64) / 4.0
    unit = np.arange(L) // SCAN_TILE if stripe == "tile" else np.arange(L)
    sampled = (unit % (SAMPLE_STRIDE if stripe == "tile" else 16)) == 0
    use_hot = sampled if hot_sampled else ~sampled
    k = np.where(use_hot[None, :, None], hot, cold)
    from workloads import to_storage
    return to_storage(k, BF16)


def _fused_scan_paths(q, w, k, g, K):
    """A model of the fused scan's sampled threshold on the oracle's proxy
    scores (exact inputs, so the same scores): per group, whether the sample
    sets a threshold that leaves fewer than K survivors (the exact re-run) or
    more than the buffer holds (compactions). Counts of each."""
    L = q.shape[1]
    G = -(-L // g)
    cap = -(-max(2 * K, K + 64) // 64) * 64
    redo = compact = 0
    groups = np.arange(G // 2, G, 16)  # groups whose prefix spans two sampled tiles or more
    rows = oracle.scores_at(q, w, k, groups, np.tile(np.arange(L, dtype=np.int32), (len(groups), 1)), g=g)
    for m, full in zip(groups, rows):
        tl = min((m + 1) * g, L) - 1
        hi = min((m // 8) * 8 + 7, G - 1)
        ntiles = (min((hi + 1) * g, L) - 1) // SCAN_TILE + 1
        if ntiles * SCAN_TILE <= 4 * K or tl + 1 <= 2 * K:
            continue
        row = full[:tl + 1]
        pos = np.arange(tl + 1)
        smp = row[(pos // SCAN_TILE) % SAMPLE_STRIDE == 0]
        nsv = len(smp)
        expect = np.float32(K) * np.float32(nsv) / np.float32(tl + 1)
        r = int(np.ceil(expect + np.float32(SAMPLE_SIGMAS) * np.sqrt(expect) + np.float32(8.0)))
        if r >= nsv:
            continue
        tau = np.sort(smp)[::-1][r - 1]
        kept = int((row > tau).sum())
        redo += kept < K
        compact += kept > cap
    return redo, compact


@pytest.mark.parametrize("stripe", ["tile", "pos"])
@pytest.mark.parametrize("hot_sampled", [True, False], ids=["sample_too_high", "sample_too_low"])
def test_mfma_sampled_threshold_stays_exact(hot_sampled, stripe, scan_path):
    """Keys that make a threshold sample unrepresentative must still give the
    exact top-K: a too high sample forces the exact re-run, a too low one
    compactions. For the fused scan a model of its sample on the oracle's
    scores confirms that the stripes reach those paths."""
    L, g, topk, c = 2 * SAMPLE_STRIDE * SCAN_TILE, 8, 128, 256
    r = np.random.default_rng(11)
    q = r.integers(1, 4, size=(1, L, 64, 128)).astype(np.float64) / 4.0
    from workloads import to_storage
    q = to_storage(q, BF16)
    w = np.ldexp(1.0, r.integers(-3, 1, size=(1, L, 64))).astype(np.float32)
    k = _striped_keys(L, 3, hot_sampled, stripe)
    if stripe == "tile" and scan_path == "fused":
        redo, compact = _fused_scan_paths(q, w, k, g, c)
        if hot_sampled:
            assert redo > 0, "the stripes should make the sampled threshold too high"
        else:
            assert compact > 0, "the stripes should make the sampled threshold too low"
    tq, tw, tk = to_device(q, w, k)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True, return_candidates=True,
                                         scan_path=scan_path)
    r_i, r_s = pv.index_reuse(tq, tw, tk, g, topk, return_scores=True, scan_path=scan_path)
    d_i, d_s = pv.index_dense(tq, tw, tk, topk, return_scores=True, scan_path=scan_path)
    torch.cuda.synchronize()
    ref = oracle.refine(q, w, k, g, topk, c)
    np.testing.assert_array_equal(f_n.cpu().numpy(), ref["cand_n"])
    np.testing.assert_array_equal(f_c.cpu().numpy(), ref["cand"])
    np.testing.assert_array_equal(f_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(f_s.cpu().numpy(), ref["scores"])
    ref = oracle.reuse(q, w, k, g, topk)
    np.testing.assert_array_equal(r_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(r_s.cpu().numpy(), ref["scores"])
    rows = np.r_[0:64, 1000:1010, 8190:8200, L - 96:L]
    ref = oracle.dense(q, w, k, topk, rows=rows)
    np.testing.assert_array_equal(d_i.cpu().numpy()[0, rows], ref["indices"][0, rows])
    np.testing.assert_array_equal(d_s.cpu().numpy()[0, rows], ref["scores"][0, rows])


# Exact inputs on the fused path at the headline's selection sizes, so every
# slab count of the register selects runs on data whose result is unique:
# group select K = c = 4096 (survivor buffer of 8192: 128 slabs), K = k =
# 2048 (64 slabs) and K = 700 (1408: 32 slabs), the member select over c =
# 4096 (64 slabs), and c = 5000 (buffer beyond the register selects: the
# streaming radix select, and the in-kernel member select of the refine).
SLAB_CASES = [
    # name, L, g, topk, c
    ("k2048_c4096", 16384, 8, 2048, 4096),
    ("k700_c1400", 12288, 8, 700, 1400),
    ("k3000_c5000", 16384, 8, 3000, 5000),
]


@pytest.mark.parametrize("case", SLAB_CASES, ids=[c[0] for c in SLAB_CASES])
def test_fused_selects_bitwise_at_every_slab_count(case):
    name, L, g, topk, c = case
    q, w, k = exact_random(zlib.crc32(name.encode()) % 1000, 1, L, L, 64, 128, BF16, w_levels=(-3, 0))
    tq, tw, tk = to_device(q, w, k)
    print(f"[slabs] {name}: GPU", flush=True)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True, return_candidates=True,
                                         scan_path="fused")
    r_i, r_s = pv.index_reuse(tq, tw, tk, g, topk, return_scores=True, scan_path="fused")
    d_i, d_s = pv.index_dense(tq, tw, tk, topk, return_scores=True, scan_path="fused")
    torch.cuda.synchronize()
    print(f"[slabs] {name}: oracle refine", flush=True)
    ref = oracle.refine(q, w, k, g, topk, c)
    np.testing.assert_array_equal(f_n.cpu().numpy(), ref["cand_n"])
    np.testing.assert_array_equal(f_c.cpu().numpy(), ref["cand"])
    np.testing.assert_array_equal(f_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(f_s.cpu().numpy(), ref["scores"])
    print(f"[slabs] {name}: oracle reuse", flush=True)
    ref = oracle.reuse(q, w, k, g, topk)
    np.testing.assert_array_equal(r_i.cpu().numpy(), ref["indices"])
    np.testing.assert_array_equal(r_s.cpu().numpy(), ref["scores"])
    rows = np.unique(np.r_[0:40, topk - 8:topk + 8, np.linspace(0, L - 1, 160).astype(np.int64), L - 40:L])
    ref = oracle.dense(q, w, k, topk, rows=rows)
    np.testing.assert_array_equal(d_i.cpu().numpy()[0, rows], ref["indices"][0, rows])
    np.testing.assert_array_equal(d_s.cpu().numpy()[0, rows], ref["scores"][0, rows])
