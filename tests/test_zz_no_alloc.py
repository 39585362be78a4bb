"""pivot_index_static (for callers that cannot allocate: its scratch is a
static device array in the library) against pivot_index with a caller
workspace: the same kernels, so the outputs must agree bit for bit. Each
case makes two calls in a row through the static scratch, the second on a
smaller problem, so stale scratch contents from the first call must not
leak into the second."""
import numpy as np
import pytest

from tests.parity import to_device
from workloads import BF16, gauss_random

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import sparse_attention_indexer_proxy_amd as pv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu(pivot_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(*a):
    print(*a, flush=True)


def _pair(q, w, k, cfg):
    tq, tw, tk = to_device(q, w, k)
    a = pv.index_static(tq, tw, tk, cfg, return_scores=True, return_candidates=True)
    b = pv.index(tq, tw, tk, cfg, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    for x, y, name in zip(a, b, ("indices", "scores", "candidates", "counts")):
        if x is None or y is None:
            assert x is None and y is None, name
            continue
        np.testing.assert_array_equal(x.cpu().numpy(), y.cpu().numpy(), err_msg=name)


# name, variant, first (B, Lq, Lk), second (B, Lq, Lk), g, topk, c
CASES = [
    ("refine_prefill_fused_then_split", pv.REFINE, (1, 3000, 3000), (1, 1000, 1000), 8, 64, 128),
    ("reuse_prefill", pv.REUSE, (1, 4096, 4096), (1, 2100, 2100), 8, 128, 0),
    ("dense_prefill", pv.DENSE, (1, 2500, 2500), (1, 700, 700), 1, 96, 0),
    ("refine_mtp_decode", pv.REFINE, (32, 4, 65536), (8, 4, 20000), 4, 2048, 4096),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_static_scratch_matches_workspace_call_twice(case):
    name, variant, first, second, g, topk, c = case
    cfg = pv.make_config(variant=variant, g=g, topk=topk, c=c if c else 2 * topk)
    for i, (B, Lq, Lk) in enumerate((first, second)):
        _say(f"[no-alloc] {name} call {i + 1}: B={B} Lq={Lq} Lk={Lk}")
        q, w, k = gauss_random(100 + i, B, Lq, Lk, 64, 128, BF16)
        _pair(q, w, k, cfg)


def test_static_scratch_refuses_a_call_beyond_its_size():
    B, L = 1, 32768
    q, w, k = gauss_random(3, B, 8, 8, 64, 128, BF16)  # any data: refused before use
    tq, tw, tk = to_device(q, w, k)
    big_q = torch.empty((B, L, 64, 128), dtype=torch.bfloat16, device="cuda")
    big_w = torch.empty((B, L, 64), dtype=torch.float32, device="cuda")
    big_k = torch.empty((B, L, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pv.PivotError) as e:
        pv.index_static(big_q, big_w, big_k, variant=pv.REFINE, g=8, topk=2048, c=4096)
    assert e.value.status == 3
    # a fitting call still works after the refusal
    _pair(q, w, k, pv.make_config(variant=pv.REFINE, g=4, topk=4, c=8))
