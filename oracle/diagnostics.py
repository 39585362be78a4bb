"""CPU oracle of the O1-O3 diagnostics of selected index sets.

TEST INFRASTRUCTURE ONLY: called by the test-suite (and nothing on the
product path). Plain Python sets and float64 numpy, one row or group at a
time.

The pages' key observations (PIVOT paper summary, "Key observations",
Figure 2) describe the top-k sets T_t the indexer selects:
  O1 (local)     adjacent queries share most of their top-k, and a good part
                 of it even across a whole group of g queries;
  O2 (shareable) the union of a group's top-k sets stays near k, far below
                 the worst case g * k;
  O3 (sparse)    the indexer scores of a top-k set concentrate on a few
                 entries: the cumulative score mass saturates well before
                 k/2, 3k/4 and k.
Readings taken here (the pages give the plots, not formulas):
  * overlap(t, d) = |T_t ∩ T_{t+d}| for rows t and t + d of one sequence;
    d = 1 is "adjacent", d = g - 1 spans a whole group; rows without a
    partner (t + d >= Lq) get -1;
  * union_m = |∪_{t in group m} T_t|, inter_m = |∩_{t in group m} T_t|,
    groups being g consecutive rows (the last one may be short);
  * mass_f(t) = (sum of the floor(f * k) largest selected scores of row t)
    / (sum of all its selected scores), f in (1/4, 1/2, 3/4), k the row
    width; NaN when that sum is not positive.
A row is the prefix of entries that are not -1 (the indexer's padding).
"""
from __future__ import annotations

import numpy as np

FRACTIONS = (0.25, 0.5, 0.75)


def _valid(row):
    row = np.asarray(row)
    n = int(np.argmax(row < 0)) if np.any(row < 0) else row.shape[0]
    return row[:n]


def overlap(indices, d: int = 1):
    """|T_t ∩ T_{t+d}| per row; -1 where t + d is past the sequence."""
    idx = np.asarray(indices)
    B, Lq, _ = idx.shape
    out = np.full((B, Lq), -1, dtype=np.int32)
    for b in range(B):
        for t in range(Lq - d):
            out[b, t] = len(set(_valid(idx[b, t]).tolist()) & set(_valid(idx[b, t + d]).tolist()))
    return out


def group_sets(indices, g: int):
    """(union, intersection) sizes per group of g consecutive rows."""
    idx = np.asarray(indices)
    B, Lq, _ = idx.shape
    G = -(-Lq // g)
    union = np.zeros((B, G), dtype=np.int32)
    inter = np.zeros((B, G), dtype=np.int32)
    for b in range(B):
        for m in range(G):
            sets = [set(_valid(idx[b, t]).tolist()) for t in range(m * g, min((m + 1) * g, Lq))]
            u, i = set(), set(sets[0])
            for s in sets:
                u |= s
                i &= s
            union[b, m] = len(u)
            inter[b, m] = len(i)
    return union, inter


def mass(indices, scores, fractions=FRACTIONS):
    """Cumulative score mass of each row's floor(f k) best entries (float64)."""
    idx = np.asarray(indices)
    sc = np.asarray(scores, dtype=np.float64)
    B, Lq, k = idx.shape
    out = np.zeros((B, Lq, len(fractions)), dtype=np.float64)
    for b in range(B):
        for t in range(Lq):
            n = _valid(idx[b, t]).shape[0]
            s = np.sort(sc[b, t, :n])[::-1]
            total = float(np.sum(s))
            for f, frac in enumerate(fractions):
                j = int(frac * k)
                out[b, t, f] = float(np.sum(s[:j])) / total if total > 0 else np.nan
    return out
