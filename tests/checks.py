"""Shared checks for indexer outputs (used by the oracle pins and GPU parity).

Row layout everywhere: the selected set in ascending position, then -1
(scores: the matching values, then -inf).
"""
from __future__ import annotations

import numpy as np


def positions(Lq: int, Lk: int) -> np.ndarray:
    return np.arange(Lq) + (Lk - Lq)


def group_last_pos(Lq: int, Lk: int, g: int) -> np.ndarray:
    G = -(-Lq // g)
    last_row = np.minimum((np.arange(G) + 1) * g, Lq) - 1
    return Lk - Lq + last_row


def valid_counts(indices: np.ndarray) -> np.ndarray:
    return (indices >= 0).sum(axis=-1)


def check_structure(indices, scores, Lq, Lk, counts=None, rows=None, g=None):
    """Ascending, duplicate-free, causal rows with -1 only in the tail.
    ``rows``: optional flat (b*Lq + r) row ids to restrict the check to.
    ``g``: Reuse group size; a Reuse row may hold positions up to its group's
    last position (one proxy row is shared by the whole group)."""
    B, _, K = indices.shape
    flat_i = indices.reshape(-1, K)
    flat_s = None if scores is None else scores.reshape(-1, K)
    if g is None:
        pos = np.tile(positions(Lq, Lk), B)
    else:
        pos = np.tile(group_last_pos(Lq, Lk, g)[np.arange(Lq) // g], B)
    sel = np.arange(flat_i.shape[0]) if rows is None else np.asarray(rows)
    for row in sel:
        ir = flat_i[row]
        n = int((ir >= 0).sum())
        assert np.all(ir[:n] >= 0) and np.all(ir[n:] == -1), f"row {row}: -1 not only in the tail"
        assert np.all(np.diff(ir[:n]) > 0), f"row {row}: not strictly ascending"
        assert n == 0 or ir[n - 1] <= pos[row], f"row {row}: index beyond its position"
        if counts is not None:
            assert n == counts[row], f"row {row}: {n} valid entries, expected {counts[row]}"
        if flat_s is not None:
            sr = flat_s[row]
            assert np.all(np.isfinite(sr[:n])), f"row {row}: non-finite score on a valid entry"
            assert np.all(np.isneginf(sr[n:])), f"row {row}: pad score is not -inf"


def dense_counts(B, Lq, Lk, topk):
    return np.tile(np.minimum(topk, positions(Lq, Lk) + 1), B)


def reuse_counts(B, Lq, Lk, g, topk):
    tl = group_last_pos(Lq, Lk, g)
    per_row = np.minimum(topk, tl[np.arange(Lq) // g] + 1)
    return np.tile(per_row, B)


def check_topk_optimal(chosen, chosen_scores, all_scores, all_pos, rtol=0.0):
    """``chosen`` must be a best set under (score desc, position asc).
    With rtol > 0 an element may be swapped with one whose score is within
    rtol of the boundary score."""
    kk = len(chosen)
    if kk == 0:
        return
    order = np.lexsort((all_pos, -all_scores))
    best = set(all_pos[order[:kk]].tolist())
    got = set(chosen.tolist())
    if rtol == 0.0:
        assert got == best, "selected set differs from the exact top-k"
        return
    boundary = all_scores[order[kk - 1]]
    tol = rtol * abs(boundary) + 1e-30
    score_of = dict(zip(all_pos.tolist(), all_scores.tolist()))
    for p in got ^ best:
        assert abs(score_of[p] - boundary) <= tol, (
            f"position {p} differs from the exact top-k with score {score_of[p]} "
            f"vs boundary {boundary}")
