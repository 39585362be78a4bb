"""Float64 brute force of the PIVOT indexer for tiny inputs.

TEST INFRASTRUCTURE ONLY. A second, independent formulation used to pin the
C oracle: it forms whole score matrices in float64 with numpy and selects
with ``numpy.lexsort``, where the oracle loops in float32 and selects with
``qsort``. On inputs whose every product and sum is exact (small multiples of
1/4, power-of-two weights) the two must agree bit for bit.

Equations from the PIVOT paper summary page (picx.dev): eq. (1) indexer score,
eq. (4) mean-pool proxy, eq. (5) proxy scan, eq. (6) Reuse, eq. (7) candidate
set, eqs. (8)-(9) Refine; section "Ablation Studies" for the first / last
query proxies, and eq. (6) with each member's own bound for member-causal
Reuse.
"""
from __future__ import annotations

import numpy as np

from workloads import BF16, bf16_bits_to_f32, f32_to_bf16_bits


def _f64(a, dtype):
    return bf16_bits_to_f32(a).astype(np.float64) if dtype == BF16 else np.asarray(a, np.float64)


def score_matrix(qv, wv, kv):
    """I[t, s] = sum_j w[t, j] * max(q[t, j] . k[s], 0) for all t, s (float64).
    qv [T, H, d], wv [T, H], kv [S, d]."""
    dots = np.einsum("thd,sd->ths", qv, kv)
    return np.einsum("th,ths->ts", wv, np.maximum(dots, 0.0))


def select(scores, positions, kk):
    """Best kk by (score desc, position asc); returned in ascending position."""
    order = np.lexsort((positions, -scores))[:kk]
    chosen = positions[order]
    sc = scores[order]
    o = np.argsort(chosen, kind="stable")
    return chosen[o], sc[o]


def _emit(out_i, out_s, row, chosen, sc, topk):
    n = len(chosen)
    out_i[row, :n] = chosen
    out_i[row, n:] = -1
    out_s[row, :n] = sc
    out_s[row, n:] = -np.inf


def proxy(q, w, g, dtype, agg="mean"):
    """eq. (4) per sequence: float64 mean, then rounded like the q storage;
    agg "first" / "last" takes that member's q and w as they are."""
    B, Lq, H, d = q.shape
    G = -(-Lq // g)
    qf, wf = _f64(q, dtype), np.asarray(w, np.float64)
    qbar = np.empty((B, G, H, d))
    wbar = np.empty((B, G, H))
    for m in range(G):
        sl = slice(m * g, min((m + 1) * g, Lq))
        if agg in ("first", "last"):
            r = sl.start if agg == "first" else sl.stop - 1
            qbar[:, m] = qf[:, r]
            wbar[:, m] = wf[:, r]
            continue
        qm = qf[:, sl].sum(axis=1) / (sl.stop - sl.start)
        qm32 = qm.astype(np.float32)
        if dtype == BF16:
            qm32 = bf16_bits_to_f32(f32_to_bf16_bits(qm32))
        qbar[:, m] = qm32
        wbar[:, m] = (wf[:, sl].sum(axis=1) / (sl.stop - sl.start)).astype(np.float32)
    return qbar, wbar


def dense(q, w, k, topk, dtype):
    B, Lq, H, d = q.shape
    Lk = k.shape[1]
    qf, wf, kf = _f64(q, dtype), np.asarray(w, np.float64), _f64(k, dtype)
    idx = np.empty((B, Lq, topk), np.int64)
    sco = np.empty((B, Lq, topk))
    pos = np.arange(Lk)
    for b in range(B):
        I = score_matrix(qf[b], wf[b], kf[b])
        for r in range(Lq):
            t = Lk - Lq + r
            ch, sc = select(I[r, :t + 1], pos[:t + 1], topk)
            _emit(idx[b], sco[b], r, ch, sc, topk)
    return idx, sco


def reuse(q, w, k, g, topk, dtype, agg="mean", member_causal=False):
    B, Lq, H, d = q.shape
    Lk = k.shape[1]
    qbar, wbar = proxy(q, w, g, dtype, agg)
    kf = _f64(k, dtype)
    idx = np.empty((B, Lq, topk), np.int64)
    sco = np.empty((B, Lq, topk))
    pos = np.arange(Lk)
    for b in range(B):
        Ibar = score_matrix(qbar[b], wbar[b], kf[b])
        for m in range(qbar.shape[1]):
            rows = range(m * g, min((m + 1) * g, Lq))
            t_last = Lk - Lq + rows[-1]
            ch, sc = select(Ibar[m, :t_last + 1], pos[:t_last + 1], topk)
            for r in rows:
                if member_causal:
                    t = Lk - Lq + r
                    ch, sc = select(Ibar[m, :t + 1], pos[:t + 1], topk)
                _emit(idx[b], sco[b], r, ch, sc, topk)
    return idx, sco


def refine(q, w, k, g, topk, c, dtype, agg="mean"):
    """Returns (indices, scores, candidate sets as a list of arrays)."""
    B, Lq, H, d = q.shape
    Lk = k.shape[1]
    qbar, wbar = proxy(q, w, g, dtype, agg)
    qf, wf, kf = _f64(q, dtype), np.asarray(w, np.float64), _f64(k, dtype)
    idx = np.empty((B, Lq, topk), np.int64)
    sco = np.empty((B, Lq, topk))
    pos = np.arange(Lk)
    cands = []
    for b in range(B):
        Ibar = score_matrix(qbar[b], wbar[b], kf[b])
        I = score_matrix(qf[b], wf[b], kf[b])
        for m in range(qbar.shape[1]):
            rows = range(m * g, min((m + 1) * g, Lq))
            t_last = Lk - Lq + rows[-1]
            C, _ = select(Ibar[m, :t_last + 1], pos[:t_last + 1], c)
            cands.append(C)
            for r in rows:
                t = Lk - Lq + r
                keep = C[C <= t]
                ch, sc = select(I[r, keep], keep, topk)
                _emit(idx[b], sco[b], r, ch, sc, topk)
    return idx, sco, cands
