"""CPU oracle of the PIVOT indexer (ctypes wrapper around pivot_oracle.c).

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the CPU-baseline
leg of the benchmark are the only callers. The HIP library never imports or
links anything here, and this package never imports the HIP library.

Arrays are numpy: q [B, Lq, H, d] (float32, or uint16 bf16 bit patterns),
w [B, Lq, H] float32, k [B, Lk, d] (same storage as q).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pivot_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_pivot_oracle.so")

DENSE, REUSE, REFINE = 0, 1, 2
AGGREGATIONS = {"mean": 0, "first": 1, "last": 2}
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
          "-Wall", "-Wextra", "-Wno-unused-parameter"]


def build(extra_flags=(), out_path: str | None = None) -> str:
    """Compile the oracle with gcc (float32 arithmetic, no contraction)."""
    out = out_path or _LIB_PATH
    tmp = out + ".tmp"
    cmd = ["gcc", *CFLAGS, *extra_flags, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class _Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("Lq", ctypes.c_int64), ("Lk", ctypes.c_int64),
                ("H", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib_cache: dict = {}


def load(path: str | None = None):
    path = path or _LIB_PATH
    if path in _lib_cache:
        return _lib_cache[path]
    if path == _LIB_PATH and (not os.path.exists(path)
                              or os.path.getmtime(path) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(_Problem)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.oracle_run.argtypes = [P, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_run.restype = ctypes.c_int
    lib.oracle_run2.argtypes = [P, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_run2.restype = ctypes.c_int
    lib.oracle_pool.argtypes = [P, i32, vp, vp, vp, vp]
    lib.oracle_pool.restype = ctypes.c_int
    lib.oracle_pool2.argtypes = [P, i32, i32, vp, vp, vp, vp]
    lib.oracle_pool2.restype = ctypes.c_int
    lib.oracle_proxy_row.argtypes = [P, i32, vp, vp, vp, i64, i64, vp]
    lib.oracle_proxy_row.restype = ctypes.c_int
    lib.oracle_proxy_row2.argtypes = [P, i32, i32, vp, vp, vp, i64, i64, vp]
    lib.oracle_proxy_row2.restype = ctypes.c_int
    lib.oracle_scores_at.argtypes = [P, i32, i32, i32, vp, vp, vp, vp, i64, vp, i64, vp]
    lib.oracle_scores_at.restype = ctypes.c_int
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _problem(q, w, k):
    if q.ndim != 4 or w.ndim != 3 or k.ndim != 3:
        raise ValueError("q [B,Lq,H,d], w [B,Lq,H], k [B,Lk,d] expected")
    B, Lq, H, d = q.shape
    if w.shape != (B, Lq, H) or k.shape[0] != B or k.shape[2] != d:
        raise ValueError("shape mismatch between q, w and k")
    if q.dtype == np.uint16 and k.dtype == np.uint16:
        dt = 1
    elif q.dtype == np.float32 and k.dtype == np.float32:
        dt = 0
    else:
        raise ValueError("q and k must both be float32 or both uint16 (bf16 bits)")
    if w.dtype != np.float32:
        raise ValueError("w must be float32")
    return _Problem(B, Lq, k.shape[1], H, d, dt)


def _c(a):
    return np.ascontiguousarray(a)


def num_threads(lib_path=None) -> int:
    return load(lib_path).oracle_num_threads()


def set_threads(n: int, lib_path=None) -> None:
    """OpenMP threads of later oracle calls in this process (results do not
    depend on it)."""
    if load(lib_path).oracle_set_threads(int(n)) != 0:
        raise ValueError("threads must be >= 1")


def groups_of(Lq: int, g: int) -> int:
    return -(-Lq // g)


def _agg(agg) -> int:
    if agg not in AGGREGATIONS:
        raise ValueError(f"aggregation must be one of {sorted(AGGREGATIONS)}")
    return AGGREGATIONS[agg]


def rank_order(indices, scores):
    """Rows in rank order: the selected entries by score, highest first, equal
    scores by lower position, then the -1 padding (T_t = TopK(I_{t,:}, k) of
    eq. (1), and of eqs. (6) and (9), listed in the order its selection rule
    ranks them; the rows of ``run`` list the same set in ascending position).
    indices [..., k] int32, scores [..., k] float32; returns new arrays."""
    idx = np.asarray(indices)
    sc = np.asarray(scores)
    if idx.shape != sc.shape:
        raise ValueError("indices and scores must have the same shape")
    fi = idx.reshape(-1, idx.shape[-1])
    fs = sc.reshape(-1, sc.shape[-1]).astype(np.float64)
    pad = fi < 0
    # np.lexsort: the last key is the primary one
    order = np.lexsort((fi, -np.where(pad, 0.0, fs), pad), axis=-1)
    out_i = np.take_along_axis(fi, order, axis=-1).reshape(idx.shape).astype(np.int32)
    out_s = np.take_along_axis(sc.reshape(fi.shape), order, axis=-1).reshape(sc.shape).astype(np.float32)
    return out_i, out_s


def run(variant: int, q, w, k, topk: int, g: int = 1, c: int = 0, units=None, cand_in=None,
        cand_in_n=None, want_scores=True, want_cand=True, lib_path=None, agg="mean", member_causal=False,
        order="position"):
    """Run one variant. Returns a dict with 'indices', 'scores' (or None),
    'cand'/'cand_n' (Refine), 'counters' = (proxy, refine, dense) dot counts.
    Rows outside the requested ``units`` stay at -2 (indices) / nan (scores).
    ``agg`` picks the proxy (mean of eq. (4), or the first / last member);
    ``member_causal`` (Reuse) bounds each member's top-k by its own t;
    ``order`` "position" lists each row's set in ascending position, "score"
    in rank order (``rank_order``; needs the scores)."""
    if order not in ("position", "score"):
        raise ValueError('order must be "position" or "score"')
    if order == "score" and not want_scores:
        raise ValueError("rank order needs the scores")
    q, w, k = _c(q), _c(w), _c(k)
    prob = _problem(q, w, k)
    B, Lq = prob.B, prob.Lq
    gg = 1 if variant == DENSE else g
    if gg < 1 or topk < 1:
        raise ValueError("g and topk must be >= 1")
    G = groups_of(Lq, gg)
    idx = np.full((B, Lq, topk), -2, dtype=np.int32)
    sc = np.full((B, Lq, topk), np.nan, dtype=np.float32) if want_scores else None
    cand = cand_n = None
    if variant == REFINE and want_cand and cand_in is None:
        cand = np.full((B, G, c), -2, dtype=np.int32)
        cand_n = np.full((B, G), -2, dtype=np.int32)
    u = None if units is None else np.ascontiguousarray(units, dtype=np.int64)
    if cand_in is not None:
        cand_in = np.ascontiguousarray(cand_in, dtype=np.int32)
        cand_in_n = np.ascontiguousarray(cand_in_n, dtype=np.int32)
        if cand_in.shape != (B, G, c) or cand_in_n.shape != (B, G):
            raise ValueError("cand_in must be [B, G, c] and cand_in_n [B, G]")
    counters = np.zeros(3, dtype=np.float64)
    rc = load(lib_path).oracle_run2(ctypes.byref(prob), variant, g, topk, c, _agg(agg), int(bool(member_causal)),
                                    _ptr(q), _ptr(w), _ptr(k), _ptr(u), 0 if u is None else len(u), _ptr(idx),
                                    _ptr(sc), _ptr(cand), _ptr(cand_n), _ptr(cand_in), _ptr(cand_in_n),
                                    _ptr(counters))
    if rc != 0:
        raise ValueError(f"oracle_run failed with code {rc}")
    if order == "score":
        idx, sc = rank_order(idx, sc)
    return {"indices": idx, "scores": sc, "cand": cand, "cand_n": cand_n,
            "counters": tuple(float(x) for x in counters)}


def dense(q, w, k, topk, rows=None, **kw):
    """eq. (1): per-query top-k of the full prefix. ``rows`` are flat b*Lq+r."""
    return run(DENSE, q, w, k, topk, 1, 0, units=rows, **kw)


def reuse(q, w, k, g, topk, groups=None, **kw):
    """eqs. (4)-(6). ``groups`` are flat b*G+m."""
    return run(REUSE, q, w, k, topk, g, 0, units=groups, **kw)


def refine(q, w, k, g, topk, c, groups=None, **kw):
    """eqs. (4)-(5), (7)-(9). ``groups`` are flat b*G+m."""
    return run(REFINE, q, w, k, topk, g, c, units=groups, **kw)


def pool(q, w, g, lib_path=None, agg="mean"):
    """eq. (4): (qbar [B,G,H,d] float32 holding q-dtype values, wbar [B,G,H]).
    ``agg`` = "first" / "last" takes that member's q and w instead."""
    q, w = _c(q), _c(w)
    B, Lq, H, d = q.shape
    k_stub = np.zeros((B, Lq, d), dtype=q.dtype)
    prob = _problem(q, w, k_stub)
    G = groups_of(Lq, g)
    qbar = np.empty((B, G, H, d), dtype=np.float32)
    wbar = np.empty((B, G, H), dtype=np.float32)
    rc = load(lib_path).oracle_pool2(ctypes.byref(prob), g, _agg(agg), _ptr(q), _ptr(w), _ptr(qbar), _ptr(wbar))
    if rc != 0:
        raise ValueError(f"oracle_pool failed with code {rc}")
    return qbar, wbar


def proxy_row(q, w, k, g, b, m, lib_path=None, agg="mean"):
    """eq. (5): the proxy score row of group m of sequence b over s <= t_last."""
    q, w, k = _c(q), _c(w), _c(k)
    prob = _problem(q, w, k)
    last = min((m + 1) * g, prob.Lq) - 1
    t_last = prob.Lk - prob.Lq + last
    out = np.empty(t_last + 1, dtype=np.float32)
    rc = load(lib_path).oracle_proxy_row2(ctypes.byref(prob), g, _agg(agg), _ptr(q), _ptr(w), _ptr(k), b, m,
                                          _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_proxy_row failed with code {rc}")
    return out


def scores_at(q, w, k, units, pos, g=None, lib_path=None, agg="mean"):
    """Scores of chosen units at chosen key positions, with the oracle's own
    fp32 arithmetic: eq. (1) of query rows (g None; units are flat rows
    b*Lq + r) or eq. (5) of group proxies (g given; units are flat groups
    b*G + m). ``pos`` [len(units), P] int key positions (negative: skipped);
    returns float32 [len(units), P], NaN at skipped positions."""
    q, w, k = _c(q), _c(w), _c(k)
    prob = _problem(q, w, k)
    u = np.ascontiguousarray(units, dtype=np.int64).reshape(-1)
    p = np.ascontiguousarray(pos, dtype=np.int32).reshape(len(u), -1)
    out = np.empty(p.shape, dtype=np.float32)
    rc = load(lib_path).oracle_scores_at(ctypes.byref(prob), 0 if g is None else 1, 1 if g is None else g,
                                         _agg(agg), _ptr(q), _ptr(w), _ptr(k), _ptr(u), len(u), _ptr(p),
                                         p.shape[1], _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_scores_at failed with code {rc}")
    return out
