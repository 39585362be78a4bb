"""The indexer captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

A call only enqueues kernels on the caller's stream (no allocation, memset,
copy or host synchronisation inside the library), so a decode loop can
capture one call and replay it per step: one graph launch instead of four or
five kernel launches. Every replay here runs on new inputs copied into the
captured buffers, with eager work and synchronisations between replays, and
must equal an eager call on the same inputs bit for bit (exact inputs: also
the oracle).
"""
import numpy as np
import pytest

import oracle
from tests.parity import to_device
from workloads import BF16, exact_random, paged_layout

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    return graph, out


# name, B, Lq, Lk, g, topk, c: the few-groups path (split scan, block
# selects, split refine) and the fused path (>= 256 groups)
CASES = [
    ("decode_few_groups", 4, 4, 3000, 4, 64, 128),
    ("prefill_fused", 1, 2048, 2048, 8, 64, 128),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("variant", ["refine", "reuse", "refine_rank"])
def test_graph_replays_equal_eager_calls(case, variant):
    name, B, Lq, Lk, g, topk, c = case
    q0, w0, k0 = exact_random(61, B, Lq, Lk, 64, 128, BF16)
    tq, tw, tk = to_device(q0, w0, k0)
    vid = pv.REUSE if variant == "reuse" else pv.REFINE
    need = pv.workspace_size(vid, B, Lq, Lk, 64, 128, torch.bfloat16, g, topk, c)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rank = pv.make_config(variant=pv.REFINE, g=g, topk=topk, c=c, order="score")

    def call(workspace):
        if variant == "refine_rank":  # the rank-order pass after the selects
            return pv.index(tq, tw, tk, rank, return_scores=True, workspace=workspace)
        if variant == "refine":
            return pv.index_refine(tq, tw, tk, g, topk, c, return_scores=True, workspace=workspace)
        return pv.index_reuse(tq, tw, tk, g, topk, return_scores=True, workspace=workspace)

    graph, (g_idx, g_sc) = _capture(lambda: call(ws))
    ws_eager = torch.empty_like(ws)
    for step, seed in enumerate((62, 63, 64)):
        q, w, k = exact_random(seed, B, Lq, Lk, 64, 128, BF16)
        nq, nw, nk = to_device(q, w, k)
        tq.copy_(nq)
        tw.copy_(nw)
        tk.copy_(nk)
        graph.replay()
        torch.cuda.synchronize()
        got_i, got_s = g_idx.clone(), g_sc.clone()
        ref_i, ref_s = call(ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i), f"{name} {variant} replay {step}: indices differ from the eager call"
        assert torch.equal(got_s, ref_s), f"{name} {variant} replay {step}: scores differ from the eager call"
        if step == 0:
            ref = (oracle.reuse(q, w, k, g, topk) if variant == "reuse" else
                   oracle.refine(q, w, k, g, topk, c, order="score" if variant == "refine_rank" else "position"))
            np.testing.assert_array_equal(got_i.cpu().numpy(), ref["indices"])
            np.testing.assert_array_equal(got_s.cpu().numpy(), ref["scores"])


def test_graph_replay_of_a_paged_decode_step():
    B, Lq, Lk, g, topk, c, page = 3, 4, 900, 4, 32, 64, 64
    lens = np.array([900, 517, 300], dtype=np.int32)
    q0, w0, k0 = exact_random(71, B, Lq, Lk, 64, 128, BF16)
    pool0, table = paged_layout(k0, lens, page, 0)
    tq, tw, tpool = to_device(q0, w0, pool0)
    tl = torch.from_numpy(lens).cuda()
    tt = torch.from_numpy(table).cuda()
    cfg = pv.make_config(variant=pv.REFINE, g=g, topk=topk, c=c)

    def call():
        return pv.index_kv(tq, tw, tpool, tl, tt, page_size=page, lk=Lk, cfg=cfg, return_scores=True)

    graph, (g_idx, g_sc) = _capture(call)
    for seed in (73, 74):
        q, w, k = exact_random(seed, B, Lq, Lk, 64, 128, BF16)
        pool, table_again = paged_layout(k, lens, page, 0)
        assert np.array_equal(table_again, table)  # same page placement, new contents
        nq, nw, npool = to_device(q, w, pool)
        tq.copy_(nq)
        tw.copy_(nw)
        tpool.copy_(npool)
        graph.replay()
        torch.cuda.synchronize()
        got_i, got_s = g_idx.clone(), g_sc.clone()
        ref_i, ref_s = call()
        torch.cuda.synchronize()
        assert torch.equal(got_i, ref_i) and torch.equal(got_s, ref_s)
        for b in range(B):
            ref = oracle.refine(q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]], g, topk, c)
            np.testing.assert_array_equal(got_i[b].cpu().numpy(), ref["indices"][0])
            np.testing.assert_array_equal(got_s[b].cpu().numpy(), ref["scores"][0])
