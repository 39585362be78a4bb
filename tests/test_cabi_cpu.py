"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before anything reaches HIP."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_proxy_amd as pv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pivot.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pivot_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("pivot_index_dense", "pivot_index_reuse", "pivot_index_refine", "pivot_workspace_size"):
        assert n in names


def test_library_exports_every_declared_symbol(pivot_lib):
    missing = [n for n in _declared() if not hasattr(pivot_lib, n)]
    assert not missing, f"not exported: {missing}"
    assert set(_declared()) == set(pv.EXPORTED)


def test_abi_version_matches_header(pivot_lib):
    m = re.search(r"#define PIVOT_ABI_VERSION (\d+)", open(HEADER).read())
    assert pivot_lib.pivot_abi_version() == int(m.group(1))


def _prob(B=1, Lq=64, Lk=64, H=64, D=128, dt=1):
    return pv.Problem(B, Lq, Lk, H, D, dt)


def _ws(pivot_lib, prob, variant, g, topk, c):
    out = ctypes.c_size_t(0)
    st = pivot_lib.pivot_workspace_size(ctypes.byref(prob), variant, g, topk, c, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,variant,g,topk,c,expect", [
    (dict(Lq=65, Lk=64), pv.REUSE, 8, 16, 0, 1),      # lq > lk
    (dict(B=0), pv.DENSE, 1, 16, 0, 1),               # empty batch
    (dict(), pv.REUSE, 0, 16, 0, 1),                  # g < 1
    (dict(), pv.DENSE, 1, 0, 0, 1),                   # topk < 1
    (dict(), pv.REFINE, 8, 16, 8, 1),                 # c < topk
    (dict(dt=7), pv.DENSE, 1, 16, 0, 1),              # unknown dtype
    (dict(D=12), pv.DENSE, 1, 16, 0, 2),              # bf16 dim not a multiple of 8
    (dict(H=0), pv.DENSE, 1, 16, 0, 1),
    (dict(Lk=2 ** 31, Lq=4), pv.DENSE, 1, 16, 0, 1),  # positions must fit int32
    (dict(), 9, 1, 16, 0, 1),                         # unknown variant
])
def test_workspace_size_rejects_bad_arguments(pivot_lib, kw, variant, g, topk, c, expect):
    st, _ = _ws(pivot_lib, _prob(**kw), variant, g, topk, c)
    assert st == expect
    assert pivot_lib.pivot_last_error().decode()


def test_workspace_size_grows_with_the_problem(pivot_lib):
    sizes = [_ws(pivot_lib, _prob(Lq=L, Lk=L), pv.REFINE, 8, 64, 128)[1] for L in (64, 512, 4096)]
    assert sizes[0] < sizes[1] < sizes[2]
    st, dense = _ws(pivot_lib, _prob(Lq=512, Lk=512), pv.DENSE, 1, 64, 0)
    assert st == 0 and dense > 0


def test_index_calls_validate_before_launch(pivot_lib):
    prob = _prob()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below fails validation
    idx = ctypes.c_void_p(1 << 21)
    # null q
    assert pivot_lib.pivot_index_dense(ctypes.byref(prob), None, fake, fake, 16, idx, None, fake, 1 << 30,
                                       None) == 1
    # workspace too small
    assert pivot_lib.pivot_index_reuse(ctypes.byref(prob), fake, fake, fake, 8, 16, idx, None, fake, 16,
                                       None) == 3
    assert "workspace" in pivot_lib.pivot_last_error().decode()
    # c < topk
    assert pivot_lib.pivot_index_refine(ctypes.byref(prob), fake, fake, fake, 8, 16, 4, idx, None, None, None,
                                        fake, 1 << 30, None) == 1
    # null problem
    assert pivot_lib.pivot_index_dense(None, fake, fake, fake, 16, idx, None, fake, 1 << 30, None) == 1
    assert pivot_lib.pivot_pool(ctypes.byref(prob), 0, fake, fake, fake, fake, None) == 1
    assert pivot_lib.pivot_proxy_scores(ctypes.byref(prob), 8, None, fake, fake, fake, None) == 1


def test_status_strings(pivot_lib):
    for s in range(5):
        assert pivot_lib.pivot_status_str(s).decode()
    assert pivot_lib.pivot_status_str(99).decode() == "unknown status"


def test_python_binding_raises_on_bad_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 8, 2, 8)
    w = torch.zeros(1, 8, 2)
    k = torch.zeros(1, 8, 8)
    with pytest.raises(ValueError):
        pv.index_dense(q, w, k, 4)          # host tensors are refused
    with pytest.raises(ValueError):
        pv.index_dense(q, w[:, :4], k, 4)   # shape mismatch


def _cfg(**kw):
    cfg = pv.Config()
    cfg.variant, cfg.g, cfg.topk, cfg.c = pv.REFINE, 8, 16, 32
    cfg.auto_variant = pv.REFINE
    for key, v in kw.items():
        setattr(cfg, key, v)
    return cfg


def test_config_init_defaults(pivot_lib):
    cfg = pv.Config()
    assert pivot_lib.pivot_config_init(ctypes.byref(cfg)) == 0
    assert (cfg.variant, cfg.g, cfg.topk, cfg.c) == (pv.REFINE, 8, 2048, 4096)
    assert (cfg.aggregation, cfg.member_causal, cfg.auto_variant, cfg.dense_below) == (0, 0, pv.REFINE, 0)
    assert pivot_lib.pivot_config_init(None) == 1


@pytest.mark.parametrize("kw,expect", [
    (dict(aggregation=3), 1),                                   # unknown aggregation
    (dict(member_causal=2), 1),
    (dict(member_causal=1), 1),                                 # Refine already masks per member
    (dict(variant=pv.DENSE, member_causal=1), 1),
    (dict(variant=pv.AUTO, auto_variant=pv.DENSE), 1),          # AUTO must fall back to a PIVOT variant
    (dict(variant=7), 1),
    (dict(variant=pv.REUSE, member_causal=1, topk=4000, g=200), 2),  # top-(k+g-1) above 4096
    (dict(variant=pv.REUSE, member_causal=1, topk=4000, g=97), 0),   # exactly 4096
    (dict(variant=pv.REUSE, member_causal=1), 0),
    (dict(variant=pv.AUTO, auto_variant=pv.REUSE, member_causal=1), 0),
    (dict(aggregation=2), 0),
    (dict(order=2), 1),                                         # unknown row order
    (dict(reserved=1), 1),
    (dict(order=1), 0),                                         # rank order, topk 16
    (dict(order=1, topk=8192, c=8192), 0),                      # the rank pass's widest row
    (dict(order=1, topk=8193, c=8200), 2),
    (dict(order=0, topk=8193, c=8200), 0),
])
def test_config_validation(pivot_lib, kw, expect):
    prob = _prob(Lq=4096, Lk=4096)
    out = ctypes.c_size_t(0)
    st = pivot_lib.pivot_index_workspace_size(ctypes.byref(prob), ctypes.byref(_cfg(**kw)), ctypes.byref(out))
    assert st == expect, pivot_lib.pivot_last_error().decode()
    if expect == 0:
        assert out.value > 0


def test_auto_resolves_by_key_count(pivot_lib):
    def resolved(lk, **kw):
        v = ctypes.c_int32(-1)
        prob = _prob(Lq=lk, Lk=lk)
        assert pivot_lib.pivot_resolve_variant(ctypes.byref(prob), ctypes.byref(_cfg(**kw)), ctypes.byref(v)) == 0
        return v.value

    d = pv.DENSE_BELOW_DEFAULT
    assert resolved(d - 1, variant=pv.AUTO) == pv.DENSE
    assert resolved(d, variant=pv.AUTO) == pv.REFINE
    assert resolved(d, variant=pv.AUTO, auto_variant=pv.REUSE) == pv.REUSE
    assert resolved(99, variant=pv.AUTO, dense_below=100) == pv.DENSE
    assert resolved(100, variant=pv.AUTO, dense_below=100) == pv.REFINE
    assert resolved(10, variant=pv.REUSE) == pv.REUSE   # explicit variants are never rewritten
    m = re.search(r"#define PIVOT_DENSE_BELOW_DEFAULT (\d+)", open(HEADER).read())
    assert int(m.group(1)) == pv.DENSE_BELOW_DEFAULT


def test_member_causal_workspace_holds_the_wider_selection(pivot_lib):
    prob = _prob(Lq=4096, Lk=4096)
    sizes = []
    for causal in (0, 1):
        out = ctypes.c_size_t(0)
        cfg = _cfg(variant=pv.REUSE, member_causal=causal)
        assert pivot_lib.pivot_index_workspace_size(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(out)) == 0
        sizes.append(out.value)
    assert sizes[1] > sizes[0]


def test_config_call_validates_before_launch(pivot_lib):
    prob = _prob()
    fake = ctypes.c_void_p(1 << 20)
    idx = ctypes.c_void_p(1 << 21)
    assert pivot_lib.pivot_index(ctypes.byref(prob), None, fake, fake, fake, idx, None, None, None, fake, 1 << 30,
                                 None) == 1
    cfg = _cfg(member_causal=1)
    assert pivot_lib.pivot_index(ctypes.byref(prob), ctypes.byref(cfg), fake, fake, fake, idx, None, None, None,
                                 fake, 1 << 30, None) == 1
    cfg = _cfg(variant=pv.REUSE)
    assert pivot_lib.pivot_index(ctypes.byref(prob), ctypes.byref(cfg), fake, fake, fake, idx, None, None, None,
                                 fake, 16, None) == 3
    assert pivot_lib.pivot_pool_ex(ctypes.byref(prob), 4, 5, fake, fake, fake, fake, None) == 1


def test_index_stats_validates_before_launch(pivot_lib):
    fake = ctypes.c_void_p(1 << 20)
    out = ctypes.c_void_p(1 << 21)
    call = pivot_lib.pivot_index_stats
    assert call(1, 8, 16, None, None, 1, 1, out, None, None, None, None) == 1       # null indices
    assert call(1, 8, 16, fake, None, 1, 1, None, None, None, None, None) == 1      # no output
    assert call(1, 8, 5000, fake, None, 1, 1, out, None, None, None, None) == 2     # k too wide
    assert call(1, 8, 16, fake, None, 0, 1, out, None, None, None, None) == 1       # d < 1
    assert call(1, 8, 16, fake, None, 1, 65, None, out, None, None, None) == 1      # g > 64
    assert call(1, 8, 4096, fake, None, 1, 8, None, None, out, None, None) == 2     # g * k > 16384
    assert call(1, 8, 16, fake, None, 1, 1, None, None, None, out, None) == 1       # mass without scores
    assert call(0, 8, 16, fake, None, 1, 1, out, None, None, None, None) == 1


@pytest.mark.parametrize("H,D,dt", [(64, 128, 0), (48, 128, 1), (64, 64, 1), (16, 128, 1)])
def test_shapes_without_mfma_are_refused_above_the_exact_kernel_limit(pivot_lib, H, D, dt):
    """f32 and bf16 shapes other than (32 or 64 heads, dim 128) run the
    exact-order kernels only up to 2^36 multiply-adds per call: no slow
    fallback at size."""
    big = _prob(Lq=131072, Lk=131072, H=H, D=D, dt=dt)
    st, _ = _ws(pivot_lib, big, pv.REFINE, 8, 2048, 4096)
    assert st == 2
    assert "MFMA" in pivot_lib.pivot_last_error().decode()
    small = _prob(Lq=512, Lk=512, H=4, D=32, dt=0)  # the tiny f32 workload
    assert _ws(pivot_lib, small, pv.DENSE, 1, 16, 0)[0] == 0
    for heads in (64, 32):  # bf16, 64 or 32 heads, dim 128: any size
        mfma = _prob(Lq=131072, Lk=131072, H=heads)
        assert _ws(pivot_lib, mfma, pv.DENSE, 1, 2048, 0)[0] == 0
        assert _ws(pivot_lib, mfma, pv.REFINE, 8, 2048, 4096)[0] == 0


def test_config_scan_path_is_checked(pivot_lib):
    cfg = pv.make_config(variant=pv.REFINE, g=8, topk=16, c=32)
    prob = _prob()
    out = ctypes.c_size_t(0)
    for path in (0, 1, 2):
        cfg.scan_path = path
        assert pivot_lib.pivot_index_workspace_size(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(out)) == 0
    cfg.scan_path = 3
    assert pivot_lib.pivot_index_workspace_size(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(out)) == 1
    with pytest.raises(ValueError):
        pv.make_config(scan_path="elsewhere")


def test_rank_order_needs_the_score_buffer(pivot_lib):
    """PIVOT_ORDER_SCORE sorts rows by their scores: a call without the score
    output is refused before anything is enqueued (no device needed)."""
    prob = _prob(Lq=4096, Lk=4096)
    fake = ctypes.c_void_p(4096)  # never dereferenced: the check comes first
    st = pivot_lib.pivot_index(ctypes.byref(prob), ctypes.byref(_cfg(order=1)), fake, fake, fake, fake, None, None,
                               None, fake, 1 << 30, None)
    assert st == 1
    assert "scores" in pivot_lib.pivot_last_error().decode()


def test_config_struct_matches_header():
    """The binding's Config mirrors pivot_config field by field (48 bytes)."""
    text = open(HEADER).read()
    end = text.index("} pivot_config;")
    body = text[text.rindex("typedef struct {", 0, end):end]
    names = re.findall(r"(?:int32_t|int64_t)\s+(\w+);", body)
    assert names == [f[0] for f in pv.Config._fields_]
    assert ctypes.sizeof(pv.Config) == 48
