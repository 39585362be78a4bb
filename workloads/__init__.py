"""Seeded synthetic inputs for the PIVOT indexer (queries, weights, keys).

This module only draws random numbers and rounds them to storage types. It
holds none of the indexer's arithmetic, so both the CPU oracle and the HIP
library can be fed from it without sharing any of the method's code.

Every array is a numpy array:
  * bf16 tensors are returned as ``uint16`` bit patterns (numpy has no bf16);
  * f32 tensors as ``float32``.

Shapes (row-major, contiguous):
  q : [B, Lq, H, d]    w : [B, Lq, H]    k : [B, Lk, d]

Query row r of a sequence sits at position ``Lk - Lq + r`` (prefill has
Lq == Lk; decode holds only the last g rows).

Random streams: ``numpy.random.default_rng([seed, tensor_id, *extra])`` with
tensor ids q=0, k=1, w=2, spike=3, drift=4, residual=5, lengths=6, pages=7.
Values are drawn in
float64 and rounded to float32 (and then to bf16) with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F32 = "f32"
BF16 = "bf16"

TID_Q, TID_K, TID_W, TID_SPIKE, TID_DRIFT, TID_RESID, TID_LENS, TID_PAGES = 0, 1, 2, 3, 4, 5, 6, 7

_CHUNK = 4096  # positions generated per step (bounds the float64 working set)


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------
def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to float32 (numpy's cast is IEEE round-to-nearest-even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (RNE) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value in generated input")
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(x64: np.ndarray, dtype: str) -> np.ndarray:
    f = f64_to_f32(x64)
    return f32_to_bf16_bits(f) if dtype == BF16 else f


# --------------------------------------------------------------------------
# configuration records
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem. ``kind`` selects the value recipe."""
    name: str
    kind: str            # "gauss" | "exact" | "ar1" | "decode" | "decode_ragged"
    B: int
    Lq: int
    Lk: int
    H: int
    d: int
    dtype: str           # F32 | BF16 (storage type of q and k)
    g: int
    topk: int
    c: int
    seed: int = 0

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def groups(self) -> int:
        return -(-self.Lq // self.g)


# The five workloads the indexer is measured and checked on.
TINY = Workload("tiny_prefill_L512", "gauss", 1, 512, 512, 4, 32, F32, 4, 16, 32)
EXACT = Workload("exact_prefill_L8192", "exact", 1, 8192, 8192, 64, 128, BF16, 8, 256, 512)
PREFILL_32K = Workload("prefill_L32768", "ar1", 1, 32768, 32768, 64, 128, BF16, 8, 2048, 4096)
LONG_128K = Workload("prefill_L131072", "ar1", 1, 131072, 131072, 64, 128, BF16, 8, 2048, 4096)
DECODE = Workload("mtp_decode_B32_P65536", "decode", 32, 4, 65536, 64, 128, BF16, 4, 2048, 4096)
# Ragged batched decode: the same recipe, each sequence with its own prefix
# length (seq_lens), keys held in a page pool (paged_layout).
DECODE_RAGGED = Workload("mtp_decode_ragged_B32_P65536", "decode_ragged", 32, 4, 65536, 64, 128, BF16, 4, 2048,
                         4096)

ALL = {w.name: w for w in (TINY, EXACT, PREFILL_32K, LONG_128K, DECODE, DECODE_RAGGED)}
LONG_G_SWEEP = (1, 4, 8, 16)

AR_RHO = 0.95
SPIKE_P = 0.02
SPIKE_AMP = 4.0


# --------------------------------------------------------------------------
# recipes
# --------------------------------------------------------------------------
def _rng(seed: int, tid: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([seed, tid, *extra])


def _gauss(w: Workload):
    """q, k ~ N(0,1), w ~ U(0,1)."""
    rq, rk, rw = _rng(w.seed, TID_Q), _rng(w.seed, TID_K), _rng(w.seed, TID_W)
    q = rq.standard_normal((w.B, w.Lq, w.H, w.d))
    k = rk.standard_normal((w.B, w.Lk, w.d))
    ww = rw.random((w.B, w.Lq, w.H))
    return to_storage(q, w.dtype), f64_to_f32(ww), to_storage(k, w.dtype)


def _exact(w: Workload):
    """q, k in {-3..3}/4 and w in {1/8, 1/4, 1/2, 1}: every sum stays exact."""
    rq, rk, rw = _rng(w.seed, TID_Q), _rng(w.seed, TID_K), _rng(w.seed, TID_W)
    q = rq.integers(-3, 4, size=(w.B, w.Lq, w.H, w.d)).astype(np.float64) / 4.0
    k = rk.integers(-3, 4, size=(w.B, w.Lk, w.d)).astype(np.float64) / 4.0
    ww = np.ldexp(1.0, rw.integers(-3, 1, size=(w.B, w.Lq, w.H)))
    return to_storage(q, w.dtype), f64_to_f32(ww), to_storage(k, w.dtype)


def _ar1_chunks(rng: np.random.Generator, n: int, width: int, rho: float, scale: float = 1.0):
    """Yield (start, block) of an AR(1) process x_t = rho x_{t-1} + scale*eps_t
    with a stationary start x_0 ~ N(0, scale^2 / (1 - rho^2)); float64."""
    prev = None
    for s0 in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s0)
        eps = rng.standard_normal((m, width))
        if scale != 1.0:
            eps *= scale
        out = np.empty_like(eps)
        if prev is None:
            out[0] = eps[0] / np.sqrt(1.0 - rho * rho)
        else:
            np.multiply(prev, rho, out=out[0])
            out[0] += eps[0]
        for t in range(1, m):
            np.multiply(out[t - 1], rho, out=out[t])
            out[t] += eps[t]
        prev = out[-1].copy()
        yield s0, out


def _spiked_keys(w: Workload, b_extra: tuple, drift_rows):
    """k_s = n_s + SPIKE_AMP * unit(z_s) at a Bernoulli(SPIKE_P) set of
    positions, where z_s is the head-summed query direction at s.
    ``drift_rows(s0, s1)`` returns z for positions [s0, s1) in float64."""
    rk = _rng(w.seed, TID_K, *b_extra)
    rs = _rng(w.seed, TID_SPIKE, *b_extra)
    out_dtype = np.uint16 if w.dtype == BF16 else np.float32
    k = np.empty((w.Lk, w.d), dtype=out_dtype)
    for s0 in range(0, w.Lk, _CHUNK):
        m = min(_CHUNK, w.Lk - s0)
        n = rk.standard_normal((m, w.d))
        spike = rs.random(m) < SPIKE_P
        if spike.any():
            z = drift_rows(s0, s0 + m)[spike]
            z /= np.linalg.norm(z, axis=1, keepdims=True)
            n[spike] += SPIKE_AMP * z
        k[s0:s0 + m] = to_storage(n, w.dtype)
    return k


def _ar1_prefill(w: Workload):
    """AR(1) queries per (head, dim), spiked keys along the head-summed query,
    w = |N(0,1)|/8."""
    if w.B != 1 or w.Lq != w.Lk:
        raise ValueError("ar1 recipe is a single prefill sequence")
    L, H, d = w.Lq, w.H, w.d
    out_dtype = np.uint16 if w.dtype == BF16 else np.float32
    q = np.empty((1, L, H, d), dtype=out_dtype)
    zsum = np.empty((L, d), dtype=np.float64)
    for s0, blk in _ar1_chunks(_rng(w.seed, TID_Q), L, H * d, AR_RHO):
        m = blk.shape[0]
        blk = blk.reshape(m, H, d)
        zsum[s0:s0 + m] = blk.sum(axis=1)
        q[0, s0:s0 + m] = to_storage(blk, w.dtype)
    ww = np.abs(_rng(w.seed, TID_W).standard_normal((1, L, H))) / 8.0
    k = _spiked_keys(w, (), lambda a, b: zsum[a:b].copy())
    return q, f64_to_f32(ww), k[None]


def seq_lens(w: Workload) -> np.ndarray:
    """Per-sequence key counts: Lk for every sequence, except the ragged
    decode workload, whose lengths are uniform on [Lk / 4, Lk] (seeded)."""
    if w.kind != "decode_ragged":
        return np.full(w.B, w.Lk, dtype=np.int32)
    r = _rng(w.seed, TID_LENS)
    return r.integers(w.Lk // 4, w.Lk + 1, size=w.B).astype(np.int32)


def paged_layout(k: np.ndarray, lens: np.ndarray, page: int, seed: int = 0):
    """The keys of each sequence copied into a shuffled page pool: returns
    (pool [num_pages, page, d], table [B, ceil(Lk / page)] int32). Pages
    past a sequence's length get no pool page (table entry -1). Only moves
    data."""
    B, Lk, d = k.shape
    maxp = -(-Lk // page)
    used = [int(-(-int(n) // page)) for n in lens]
    n_pages = max(1, sum(used))
    perm = _rng(seed, TID_PAGES).permutation(n_pages).astype(np.int32)
    pool = np.zeros((n_pages, page, d), dtype=k.dtype)
    table = np.full((B, maxp), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        for j in range(used[b]):
            ph = perm[at]
            at += 1
            rows = k[b, j * page:min((j + 1) * page, int(lens[b]))]
            pool[ph, :rows.shape[0]] = rows
            table[b, j] = ph
    return pool, table


def _decode(w: Workload):
    """B independent sequences, Lk-token key prefix each, and a group of Lq
    AR(1) queries at positions Lk-Lq .. Lk-1.

    The head-summed query process z_s (a d-dim AR(1) with innovation variance
    H) is drawn for every position; the query rows are z_s / H plus a
    zero-head-mean residual (the projection of H independent AR(1) rows that
    start stationary at position Lk-Lq). This has the same joint law as H
    independent per-head AR(1) rows summed into z, without drawing all Lk rows.
    """
    B, G, Lk, H, d = w.B, w.Lq, w.Lk, w.H, w.d
    out_dtype = np.uint16 if w.dtype == BF16 else np.float32
    q = np.empty((B, G, H, d), dtype=out_dtype)
    k = np.zeros((B, Lk, d), dtype=out_dtype)
    ww = np.empty((B, G, H), dtype=np.float32)
    lens = seq_lens(w)
    for b in range(B):
        P = int(lens[b])  # this sequence's prefix; rows past it stay zero
        z = np.empty((P, d), dtype=np.float64)
        for s0, blk in _ar1_chunks(_rng(w.seed, TID_DRIFT, b), P, d, AR_RHO, np.sqrt(H)):
            z[s0:s0 + blk.shape[0]] = blk
        resid = np.concatenate([blk for _, blk in
                                _ar1_chunks(_rng(w.seed, TID_RESID, b), G, H * d, AR_RHO)])
        resid = resid.reshape(G, H, d)
        resid -= resid.mean(axis=1, keepdims=True)
        qb = z[P - G:, None, :] / H + resid
        q[b] = to_storage(qb, w.dtype)
        ww[b] = f64_to_f32(np.abs(_rng(w.seed, TID_W, b).standard_normal((G, H))) / 8.0)
        k[b, :P] = _spiked_keys(w.replace(Lk=P), (b,), lambda a, c: z[a:c].copy())
    return q, ww, k


_RECIPES = {"gauss": _gauss, "exact": _exact, "ar1": _ar1_prefill, "decode": _decode, "decode_ragged": _decode}


def generate(w: Workload):
    """Return (q, w, k) numpy arrays for a workload (see module docstring)."""
    return _RECIPES[w.kind](w)


def q_as_f32(q: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(q) if dtype == BF16 else np.asarray(q, dtype=np.float32)


def exact_random(rng_seed: int, B: int, Lq: int, Lk: int, H: int, d: int, dtype: str = F32,
                 qk_levels: int = 3, w_levels=(-3, 0)):
    """Small inputs whose every product and sum is exact in float32 and
    float64: q, k in {-qk_levels..qk_levels}/4 and w a power of two in
    [2**w_levels[0], 2**w_levels[1]]. Used to check the oracle bit for bit."""
    r = np.random.default_rng([rng_seed, 99])
    q = r.integers(-qk_levels, qk_levels + 1, size=(B, Lq, H, d)).astype(np.float64) / 4.0
    k = r.integers(-qk_levels, qk_levels + 1, size=(B, Lk, d)).astype(np.float64) / 4.0
    ww = np.ldexp(1.0, r.integers(w_levels[0], w_levels[1] + 1, size=(B, Lq, H)))
    return to_storage(q, dtype), f64_to_f32(ww), to_storage(k, dtype)


def gauss_random(rng_seed: int, B: int, Lq: int, Lk: int, H: int, d: int, dtype: str = F32):
    """Small N(0,1) inputs with w ~ U(0,1)."""
    r = np.random.default_rng([rng_seed, 98])
    q = r.standard_normal((B, Lq, H, d))
    k = r.standard_normal((B, Lk, d))
    ww = r.random((B, Lq, H))
    return to_storage(q, dtype), f64_to_f32(ww), to_storage(k, dtype)


def to_device(q, w, k, device="cuda"):
    """Copy generated arrays to torch device tensors (bf16 bits -> bfloat16)."""
    import torch
    if q.dtype == np.uint16:
        tq = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to(device).view(torch.bfloat16)
        tk = torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).to(device).view(torch.bfloat16)
    else:
        tq = torch.from_numpy(np.ascontiguousarray(q)).to(device)
        tk = torch.from_numpy(np.ascontiguousarray(k)).to(device)
    tw = torch.from_numpy(np.ascontiguousarray(w)).to(device)
    return tq, tw, tk
