"""PIVOT group-shared sparse-attention indexer on MI355X (gfx950).

Thin Python binding of ``libpivot.so`` (C ABI in ``include/pivot.h``): it
checks tensors, allocates outputs and workspace with torch and passes raw
device pointers plus the current HIP stream. Every step of the indexer runs
in the library's HIP kernels; there is no other implementation behind these
functions, and they raise if the library is missing.

Tensors: q [B, Lq, H, d] (or [Lq, H, d]) bf16/f32, w [B, Lq, H] f32,
k [B, Lk, d] (or [Lk, d]) in q's dtype, all on one CUDA (HIP) device.
Outputs: int32 indices [B, Lq, topk], each row the selected positions in
ascending order followed by -1; optional f32 scores aligned with them.
Query row r of a sequence sits at position Lk - Lq + r.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["PivotError", "index_dense", "index_reuse", "index_refine", "index", "index_kv", "index_static", "resolve_variant", "pool",
           "index_stats",
           "proxy_scores", "workspace_size", "library_path", "load_library", "timing_enable", "timing_read",
           "make_config", "Config", "DENSE", "REUSE", "REFINE", "AUTO", "AGGREGATIONS", "SCAN_PATHS", "ORDERS", "DENSE_BELOW_DEFAULT",
           "STAGES"]

DENSE, REUSE, REFINE, AUTO = 0, 1, 2, 3
AGGREGATIONS = {"mean": 0, "first": 1, "last": 2}
SCAN_PATHS = {"auto": 0, "fused": 1, "split": 2}  # pivot_scan_path of the header
ORDERS = {"position": 0, "score": 1}  # pivot_order of the header
DENSE_BELOW_DEFAULT = 8192  # PIVOT_DENSE_BELOW_DEFAULT of the header
_F32, _BF16 = 0, 1
_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libpivot.so")
_lib = None

EXPORTED = ("pivot_workspace_size", "pivot_index_dense", "pivot_index_reuse", "pivot_index_refine",
            "pivot_config_init", "pivot_resolve_variant", "pivot_index_workspace_size", "pivot_index",
            "pivot_index_kv", "pivot_index_kv_workspace_size", "pivot_index_static",
            "pivot_pool", "pivot_pool_ex", "pivot_proxy_scores", "pivot_index_stats", "pivot_timing_enable",
            "pivot_timing_read",
            "pivot_status_str", "pivot_last_error", "pivot_abi_version")
STAGES = ("pool", "scan", "select", "refine", "scan_select", "order")


class PivotError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"pivot status {status}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("lq", ctypes.c_int64), ("lk", ctypes.c_int64),
                ("heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Config(ctypes.Structure):
    """pivot_config of the header."""
    _fields_ = [("variant", ctypes.c_int32), ("g", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("c", ctypes.c_int32), ("aggregation", ctypes.c_int32), ("member_causal", ctypes.c_int32),
                ("auto_variant", ctypes.c_int32), ("scan_path", ctypes.c_int32), ("dense_below", ctypes.c_int64),
                ("order", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Keys(ctypes.Structure):
    """pivot_keys of the header."""
    _fields_ = [("k", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load libpivot.so (built in-tree by ``build.py``); raise if absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m sparse_attention_indexer_proxy_amd.build`")
    lib = ctypes.CDLL(p)
    P = ctypes.POINTER(Problem)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.pivot_workspace_size.argtypes = [P, i32, i32, i32, i32, ctypes.POINTER(sz)]
    lib.pivot_index_dense.argtypes = [P, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.pivot_index_reuse.argtypes = [P, vp, vp, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.pivot_index_refine.argtypes = [P, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    C = ctypes.POINTER(Config)
    lib.pivot_config_init.argtypes = [C]
    lib.pivot_resolve_variant.argtypes = [P, C, ctypes.POINTER(i32)]
    lib.pivot_index_workspace_size.argtypes = [P, C, ctypes.POINTER(sz)]
    lib.pivot_index.argtypes = [P, C, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.pivot_index_static.argtypes = [P, C, vp, vp, vp, vp, vp, vp, vp, vp]
    KP = ctypes.POINTER(Keys)
    lib.pivot_index_kv.argtypes = [P, C, vp, vp, KP, vp, vp, vp, vp, vp, sz, vp]
    lib.pivot_index_kv_workspace_size.argtypes = [P, C, KP, ctypes.POINTER(sz)]
    lib.pivot_pool.argtypes = [P, i32, vp, vp, vp, vp, vp]
    lib.pivot_pool_ex.argtypes = [P, i32, i32, vp, vp, vp, vp, vp]
    lib.pivot_proxy_scores.argtypes = [P, i32, vp, vp, vp, vp, vp]
    lib.pivot_index_stats.argtypes = [ctypes.c_int64, ctypes.c_int64, i32, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    for name in ("pivot_index_stats", "pivot_index_kv", "pivot_index_kv_workspace_size","pivot_workspace_size", "pivot_index_dense", "pivot_index_reuse", "pivot_index_refine",
                 "pivot_config_init", "pivot_resolve_variant", "pivot_index_workspace_size", "pivot_index",
                 "pivot_index_static",
                 "pivot_pool", "pivot_pool_ex", "pivot_proxy_scores"):
        getattr(lib, name).restype = ctypes.c_int
    lib.pivot_timing_enable.argtypes = [i32]
    lib.pivot_timing_enable.restype = ctypes.c_int
    lib.pivot_timing_read.argtypes = [vp, vp]
    lib.pivot_timing_read.restype = ctypes.c_int
    lib.pivot_status_str.argtypes = [ctypes.c_int]
    lib.pivot_status_str.restype = ctypes.c_char_p
    lib.pivot_last_error.restype = ctypes.c_char_p
    lib.pivot_abi_version.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise PivotError(status, f"{lib.pivot_status_str(status).decode()}: {lib.pivot_last_error().decode()}")


def _stream_ptr(stream, device):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return _BF16
    if dt == torch.float32:
        return _F32
    raise TypeError(f"q and k must be bfloat16 or float32 (got {dt})")


def _prepare(q, w, k):
    squeeze = q.dim() == 3
    if squeeze:
        q, w = q.unsqueeze(0), w.unsqueeze(0)
        k = k.unsqueeze(0) if k.dim() == 2 else k
    if q.dim() != 4 or w.dim() != 3 or k.dim() != 3:
        raise ValueError("expected q [B,Lq,H,d], w [B,Lq,H], k [B,Lk,d]")
    B, Lq, H, D = q.shape
    if tuple(w.shape) != (B, Lq, H) or k.shape[0] != B or k.shape[2] != D:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, w {tuple(w.shape)}, k {tuple(k.shape)}")
    if k.dtype != q.dtype:
        raise TypeError("k must have q's dtype")
    if w.dtype != torch.float32:
        raise TypeError("w must be float32")
    for name, t in (("q", q), ("w", w), ("k", k)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != q.device:
            raise ValueError("q, w and k must be on one device")
    q, w, k = q.contiguous(), w.contiguous(), k.contiguous()
    prob = Problem(B, Lq, k.shape[1], H, D, _dtype_code(q.dtype))
    return prob, q, w, k, squeeze


def workspace_size(variant: int, B: int, Lq: int, Lk: int, H: int, D: int, dtype, g: int = 1, topk: int = 1,
                   c: int = 0) -> int:
    prob = Problem(B, Lq, Lk, H, D, _dtype_code(dtype))
    out = ctypes.c_size_t(0)
    _check(load_library().pivot_workspace_size(ctypes.byref(prob), variant, g, topk, c, ctypes.byref(out)))
    return out.value


def _workspace(prob, variant, g, topk, c, device, workspace):
    need = ctypes.c_size_t(0)
    _check(load_library().pivot_workspace_size(ctypes.byref(prob), variant, g, topk, c, ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _outputs(prob, topk, device, return_scores, cfg=None):
    """Index rows and, when asked for or needed as the rank-order sort key,
    score rows."""
    need = return_scores or (cfg is not None and cfg.order == ORDERS["score"])
    idx = torch.empty((prob.batch, prob.lq, topk), dtype=torch.int32, device=device)
    sc = torch.empty((prob.batch, prob.lq, topk), dtype=torch.float32, device=device) if need else None
    return idx, sc


def _finish(squeeze, *ts):
    out = tuple(t[0] if (squeeze and t is not None) else t for t in ts)
    return out if len(out) > 1 else out[0]


def index_dense(q, w, k, topk: int, *, return_scores: bool = False, workspace=None, stream=None,
                scan_path: str = "auto"):
    """eq. (1): every query keeps the top-k of its prefix s <= t. scan_path
    ("auto", "fused", "split") picks the scan kernels (pivot_scan_path)."""
    if scan_path != "auto":
        return index(q, w, k, make_config(variant=DENSE, g=1, topk=topk, scan_path=scan_path),
                     return_scores=return_scores, workspace=workspace, stream=stream)
    prob, q, w, k, sq = _prepare(q, w, k)
    ws, wsb = _workspace(prob, DENSE, 1, topk, 0, q.device, workspace)
    idx, sc = _outputs(prob, topk, q.device, return_scores)
    _check(load_library().pivot_index_dense(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k), topk, _ptr(idx),
                                            _ptr(sc), _ptr(ws), wsb, _stream_ptr(stream, q.device)))
    return _finish(sq, idx, sc) if return_scores else _finish(sq, idx)


def index_reuse(q, w, k, g: int, topk: int, *, return_scores: bool = False, workspace=None, stream=None,
                scan_path: str = "auto"):
    """eqs. (4)-(6): one proxy scan per group of g rows; its top-k is every
    member's row."""
    if scan_path != "auto":
        return index(q, w, k, make_config(variant=REUSE, g=g, topk=topk, scan_path=scan_path),
                     return_scores=return_scores, workspace=workspace, stream=stream)
    prob, q, w, k, sq = _prepare(q, w, k)
    ws, wsb = _workspace(prob, REUSE, g, topk, 0, q.device, workspace)
    idx, sc = _outputs(prob, topk, q.device, return_scores)
    _check(load_library().pivot_index_reuse(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k), g, topk, _ptr(idx),
                                            _ptr(sc), _ptr(ws), wsb, _stream_ptr(stream, q.device)))
    return _finish(sq, idx, sc) if return_scores else _finish(sq, idx)


def index_refine(q, w, k, g: int, topk: int, c: int | None = None, *, return_scores: bool = False,
                 return_candidates: bool = False, workspace=None, stream=None, scan_path: str = "auto"):
    """eqs. (4)-(5), (7)-(9): one proxy scan per group keeps c candidates
    (default 2k); each member re-scores them and keeps its own top-k.
    With return_candidates, also returns C [B, G, c] (ascending, -1 pad) and
    |C| [B, G]."""
    c = 2 * topk if c is None else c
    if scan_path != "auto":
        return index(q, w, k, make_config(variant=REFINE, g=g, topk=topk, c=c, scan_path=scan_path),
                     return_scores=return_scores, return_candidates=return_candidates, workspace=workspace,
                     stream=stream)
    prob, q, w, k, sq = _prepare(q, w, k)
    ws, wsb = _workspace(prob, REFINE, g, topk, c, q.device, workspace)
    idx, sc = _outputs(prob, topk, q.device, return_scores)
    G = -(-prob.lq // g)
    cand = cand_n = None
    if return_candidates:
        cand = torch.empty((prob.batch, G, c), dtype=torch.int32, device=q.device)
        cand_n = torch.empty((prob.batch, G), dtype=torch.int32, device=q.device)
    _check(load_library().pivot_index_refine(ctypes.byref(prob), _ptr(q), _ptr(w), _ptr(k), g, topk, c, _ptr(idx),
                                             _ptr(sc), _ptr(cand), _ptr(cand_n), _ptr(ws), wsb,
                                             _stream_ptr(stream, q.device)))
    outs = [idx]
    if return_scores:
        outs.append(sc)
    if return_candidates:
        outs += [cand, cand_n]
    return _finish(sq, *outs)


def make_config(variant: int = REFINE, g: int = 8, topk: int = 2048, c: int | None = None,
                aggregation: str = "mean", member_causal: bool = False, auto_variant: int = REFINE,
                dense_below: int = 0, scan_path: str = "auto", order: str = "position") -> Config:
    """A pivot_config (c defaults to 2k; dense_below 0 = the library's
    guardrail; scan_path "auto", "fused" or "split"; order "position"
    (ascending positions) or "score" (rank order: score descending, equal
    scores by lower position))."""
    if aggregation not in AGGREGATIONS:
        raise ValueError(f"aggregation must be one of {sorted(AGGREGATIONS)}")
    if scan_path not in SCAN_PATHS:
        raise ValueError(f"scan_path must be one of {sorted(SCAN_PATHS)}")
    if order not in ORDERS:
        raise ValueError(f"order must be one of {sorted(ORDERS)}")
    cfg = Config()
    _check(load_library().pivot_config_init(ctypes.byref(cfg)))
    cfg.variant, cfg.g, cfg.topk = variant, g, topk
    cfg.c = 2 * topk if c is None else c
    cfg.aggregation = AGGREGATIONS[aggregation]
    cfg.member_causal = 1 if member_causal else 0
    cfg.auto_variant, cfg.dense_below = auto_variant, dense_below
    cfg.scan_path = SCAN_PATHS[scan_path]
    cfg.order = ORDERS[order]
    return cfg


def resolve_variant(B: int, Lq: int, Lk: int, H: int, D: int, dtype, cfg: Config) -> int:
    """The variant (DENSE, REUSE or REFINE) a call with ``cfg`` runs."""
    prob = Problem(B, Lq, Lk, H, D, _dtype_code(dtype))
    out = ctypes.c_int32(0)
    _check(load_library().pivot_resolve_variant(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def index(q, w, k, cfg: Config | None = None, *, return_scores: bool = False, return_candidates: bool = False,
          workspace=None, stream=None, **knobs):
    """The indexer under one config: ``cfg`` from ``make_config`` or the
    same keywords (variant, g, topk, c, aggregation, member_causal,
    auto_variant, dense_below, scan_path, order). variant=AUTO is the short-context guardrail:
    dense below ``dense_below`` keys, else ``auto_variant``. Candidates are
    returned (None when the call resolved to another variant) only with
    return_candidates."""
    if cfg is None:
        cfg = make_config(**knobs)
    elif knobs:
        raise TypeError("pass either cfg or keywords")
    prob, q, w, k, sq = _prepare(q, w, k)
    lib = load_library()
    need = ctypes.c_size_t(0)
    _check(lib.pivot_index_workspace_size(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    idx, sc = _outputs(prob, cfg.topk, q.device, return_scores, cfg)
    cand = cand_n = None
    if return_candidates:
        resolved = ctypes.c_int32(0)
        _check(lib.pivot_resolve_variant(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(resolved)))
        if resolved.value == REFINE:
            G = -(-prob.lq // cfg.g)
            cand = torch.empty((prob.batch, G, cfg.c), dtype=torch.int32, device=q.device)
            cand_n = torch.empty((prob.batch, G), dtype=torch.int32, device=q.device)
    _check(lib.pivot_index(ctypes.byref(prob), ctypes.byref(cfg), _ptr(q), _ptr(w), _ptr(k), _ptr(idx), _ptr(sc),
                           _ptr(cand), _ptr(cand_n), _ptr(workspace), wsb, _stream_ptr(stream, q.device)))
    outs = [idx]
    if return_scores:
        outs.append(sc)
    if return_candidates:
        outs += [None if cand is None else _finish(sq, cand), None if cand_n is None else _finish(sq, cand_n)]
    return _finish(sq, *outs) if len(outs) > 1 else _finish(sq, idx)


def index_static(q, w, k, cfg: Config | None = None, *, return_scores: bool = False,
                 return_candidates: bool = False, stream=None, **knobs):
    """pivot_index_static: the indexer with the library's static device
    scratch instead of a workspace (allocates nothing but the outputs made
    here). Same arguments and results as index()."""
    if cfg is None:
        cfg = make_config(**knobs)
    elif knobs:
        raise TypeError("pass either cfg or keywords")
    prob, q, w, k, sq = _prepare(q, w, k)
    lib = load_library()
    idx, sc = _outputs(prob, cfg.topk, q.device, return_scores, cfg)
    cand = cand_n = None
    if return_candidates:
        resolved = ctypes.c_int32(0)
        _check(lib.pivot_resolve_variant(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(resolved)))
        if resolved.value == REFINE:
            G = -(-prob.lq // cfg.g)
            cand = torch.empty((prob.batch, G, cfg.c), dtype=torch.int32, device=q.device)
            cand_n = torch.empty((prob.batch, G), dtype=torch.int32, device=q.device)
    with torch.cuda.device(q.device):
        _check(lib.pivot_index_static(ctypes.byref(prob), ctypes.byref(cfg), _ptr(q), _ptr(w), _ptr(k), _ptr(idx),
                                      _ptr(sc), _ptr(cand), _ptr(cand_n), _stream_ptr(stream, q.device)))
    outs = [idx]
    if return_scores:
        outs.append(sc)
    if return_candidates:
        outs += [None if cand is None else _finish(sq, cand), None if cand_n is None else _finish(sq, cand_n)]
    return _finish(sq, *outs) if len(outs) > 1 else _finish(sq, idx)


def index_kv(q, w, k, seq_lens=None, page_table=None, *, page_size: int = 0, lk: int | None = None,
             cfg: Config | None = None, return_scores: bool = False, return_candidates: bool = False,
             workspace=None, stream=None, **knobs):
    """The indexer over a ragged and/or paged batch (pivot_index_kv).

    q [B, Lq, H, d], w [B, Lq, H]; k is either contiguous [B, Lk, d] or, with
    page_table [B, max_pages] int32, a page pool [num_pages, page_size, d];
    seq_lens [B] int32 gives each sequence's key count (its queries are its
    last Lq positions). lk is the key capacity per sequence (default: k's
    second dimension, or max_pages * page_size when paged). Outputs as for
    index()."""
    if cfg is None:
        cfg = make_config(**knobs)
    elif knobs:
        raise TypeError("pass either cfg or keywords")
    if q.dim() != 4 or w.dim() != 3:
        raise ValueError("expected q [B, Lq, H, d] and w [B, Lq, H]")
    B, Lq, H, D = q.shape
    for name, t in (("q", q), ("w", w), ("k", k)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a device tensor on q's device")
    if k.dtype != q.dtype or w.dtype != torch.float32 or tuple(w.shape) != (B, Lq, H) or k.shape[-1] != D:
        raise ValueError("q, w, k dtypes or shapes do not match")
    q, w, k = q.contiguous(), w.contiguous(), k.contiguous()
    keys = Keys()
    keys.k = k.data_ptr()
    if seq_lens is not None:
        if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,) or seq_lens.device != q.device:
            raise ValueError("seq_lens must be an int32 device tensor [B]")
        seq_lens = seq_lens.contiguous()
        keys.seq_lens = seq_lens.data_ptr()
    if page_table is not None:
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or page_table.shape[0] != B:
            raise ValueError("page_table must be an int32 device tensor [B, max_pages]")
        if k.dim() != 3 or k.shape[1] != page_size:
            raise ValueError("paged k must be [num_pages, page_size, d]")
        page_table = page_table.contiguous()
        keys.page_table = page_table.data_ptr()
        keys.num_pages, keys.page_size, keys.max_pages = k.shape[0], page_size, page_table.shape[1]
        cap = lk if lk is not None else page_table.shape[1] * page_size
    else:
        if k.dim() != 3 or k.shape[0] != B:
            raise ValueError("contiguous k must be [B, Lk, d]")
        cap = lk if lk is not None else k.shape[1]
    prob = Problem(B, Lq, cap, H, D, _dtype_code(q.dtype))
    lib = load_library()
    need = ctypes.c_size_t(0)
    _check(lib.pivot_index_kv_workspace_size(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(keys),
                                             ctypes.byref(need)))
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    idx, sc = _outputs(prob, cfg.topk, q.device, return_scores, cfg)
    cand = cand_n = None
    if return_candidates:
        resolved = ctypes.c_int32(0)
        _check(lib.pivot_resolve_variant(ctypes.byref(prob), ctypes.byref(cfg), ctypes.byref(resolved)))
        if resolved.value == REFINE:
            G = -(-Lq // cfg.g)
            cand = torch.empty((B, G, cfg.c), dtype=torch.int32, device=q.device)
            cand_n = torch.empty((B, G), dtype=torch.int32, device=q.device)
    _check(lib.pivot_index_kv(ctypes.byref(prob), ctypes.byref(cfg), _ptr(q), _ptr(w), ctypes.byref(keys), _ptr(idx),
                              _ptr(sc), _ptr(cand), _ptr(cand_n), _ptr(workspace), wsb, _stream_ptr(stream, q.device)))
    outs = [idx]
    if return_scores:
        outs.append(sc)
    if return_candidates:
        outs += [cand, cand_n]
    return tuple(outs) if len(outs) > 1 else idx


def pool(q, w, g: int, stream=None, aggregation: str = "mean"):
    """eq. (4): proxies qbar [B, G, H, d] (q dtype) and wbar [B, G, H] f32.
    aggregation "first" / "last" takes that member's q and w instead of the
    mean."""
    if aggregation not in AGGREGATIONS:
        raise ValueError(f"aggregation must be one of {sorted(AGGREGATIONS)}")
    prob, q, w, _, sq = _prepare(q, w, q[..., 0, :] if q.dim() == 4 else q[:, 0, :])
    G = -(-prob.lq // g)
    qbar = torch.empty((prob.batch, G, prob.heads, prob.dim), dtype=q.dtype, device=q.device)
    wbar = torch.empty((prob.batch, G, prob.heads), dtype=torch.float32, device=q.device)
    _check(load_library().pivot_pool_ex(ctypes.byref(prob), g, AGGREGATIONS[aggregation], _ptr(q), _ptr(w),
                                        _ptr(qbar), _ptr(wbar), _stream_ptr(stream, q.device)))
    return _finish(sq, qbar, wbar)


def proxy_scores(qbar, wbar, k, g: int, lq: int, stream=None):
    """eq. (5): score rows [B, G, Lk] of the proxies (-inf after t_last).
    ``lq`` is the query row count the groups were formed from."""
    if qbar.dim() == 3:
        qbar, wbar = qbar.unsqueeze(0), wbar.unsqueeze(0)
        k = k.unsqueeze(0) if k.dim() == 2 else k
    B, G, H, D = qbar.shape
    if G != -(-lq // g):
        raise ValueError("qbar's group count does not match lq and g")
    qbar, wbar, k = qbar.contiguous(), wbar.contiguous(), k.contiguous()
    prob = Problem(B, lq, k.shape[1], H, D, _dtype_code(qbar.dtype))
    out = torch.empty((B, G, k.shape[1]), dtype=torch.float32, device=qbar.device)
    _check(load_library().pivot_proxy_scores(ctypes.byref(prob), g, _ptr(qbar), _ptr(wbar), _ptr(k), _ptr(out),
                                             _stream_ptr(stream, qbar.device)))
    return out


def index_stats(indices, scores=None, *, d: int = 1, g: int | None = None, stream=None):
    """O1-O3 diagnostics of index rows [B, Lq, k] (or [Lq, k]): returns a dict
    with "overlap" [B, Lq] (|T_t ∩ T_{t+d}|, -1 past the end), and, when g is
    given, "union" and "inter" [B, ceil(Lq/g)]; with scores, "mass"
    [B, Lq, 3] (share of the row's score mass in its best k/4, k/2, 3k/4)."""
    squeeze = indices.dim() == 2
    if squeeze:
        indices = indices.unsqueeze(0)
        scores = scores.unsqueeze(0) if scores is not None else None
    if indices.dim() != 3 or indices.dtype != torch.int32 or not indices.is_cuda:
        raise ValueError("indices must be an int32 device tensor [B, Lq, k]")
    if scores is not None and (tuple(scores.shape) != tuple(indices.shape) or scores.dtype != torch.float32):
        raise ValueError("scores must be float32 with the shape of indices")
    B, Lq, k = indices.shape
    indices = indices.contiguous()
    scores = scores.contiguous() if scores is not None else None
    dev = indices.device
    out = {"overlap": torch.empty((B, Lq), dtype=torch.int32, device=dev)}
    if g is not None:
        G = -(-Lq // g)
        out["union"] = torch.empty((B, G), dtype=torch.int32, device=dev)
        out["inter"] = torch.empty((B, G), dtype=torch.int32, device=dev)
    if scores is not None:
        out["mass"] = torch.empty((B, Lq, 3), dtype=torch.float32, device=dev)
    _check(load_library().pivot_index_stats(B, Lq, k, _ptr(indices), _ptr(scores), d, g or 1, _ptr(out["overlap"]),
                                            _ptr(out.get("union")), _ptr(out.get("inter")), _ptr(out.get("mass")),
                                            _stream_ptr(stream, dev)))
    return {name: (t[0] if squeeze else t) for name, t in out.items()}


def timing_enable(on: bool = True):
    """Bracket every kernel launched by this thread's calls with hipEvents."""
    _check(load_library().pivot_timing_enable(1 if on else 0))


def timing_read():
    """Wait for the recorded events; return {stage: (total_ms, launches)} and
    forget the records."""
    import numpy as np
    ms = np.zeros(len(STAGES), dtype=np.float64)
    n = np.zeros(len(STAGES), dtype=np.int64)
    _check(load_library().pivot_timing_read(ms.ctypes.data_as(ctypes.c_void_p), n.ctypes.data_as(ctypes.c_void_p)))
    return {name: (float(ms[i]), int(n[i])) for i, name in enumerate(STAGES)}
