"""Helpers for comparing the HIP library with the CPU oracle.

Float comparison rule (float workloads; the exact-arithmetic workload and the
exact-order kernels are compared bit for bit instead):
  1. every GPU score is within RTOL (relative, with a floor of ATOL_FRAC of
     the row's largest score) of the reference score of the same position;
  2. a position may be selected by one side and not the other only if its
     reference score lies within that tolerance of the reference boundary
     (the reference's K-th best score).
"""
from __future__ import annotations

import numpy as np

from workloads import to_device  # noqa: F401  (re-exported for the tests)

RTOL = 1e-3
ATOL_FRAC = 1e-6


def bf16_tensor_bits(t) -> np.ndarray:
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def tol(boundary: float, row_max: float) -> float:
    return RTOL * abs(boundary) + ATOL_FRAC * abs(row_max) + 1e-30


def compare_row(gpu_idx, gpu_sc, ref_idx, ref_sc, score_of, what=""):
    """Compare one output row. ``score_of(positions) -> float64 scores`` gives
    reference scores of arbitrary positions. Returns the number of positions
    in the symmetric difference."""
    gv = gpu_idx[gpu_idx >= 0]
    rv = ref_idx[ref_idx >= 0]
    assert len(gv) == len(rv), f"{what}: {len(gv)} valid entries vs reference {len(rv)}"
    assert np.all(gpu_idx[len(gv):] == -1), f"{what}: -1 not only in the tail"
    assert np.all(np.diff(gv) > 0), f"{what}: not strictly ascending"
    if len(rv) == 0:
        return 0
    rs = ref_sc[:len(rv)].astype(np.float64)
    boundary = rs.min()
    row_max = rs.max()
    t = tol(boundary, row_max)
    if gpu_sc is not None:
        exp = score_of(gv)
        err = np.abs(gpu_sc[:len(gv)].astype(np.float64) - exp)
        lim = RTOL * np.abs(exp) + ATOL_FRAC * abs(row_max) + 1e-30
        bad = err > lim
        assert not bad.any(), (f"{what}: score mismatch at positions {gv[bad][:5]}: "
                               f"gpu {gpu_sc[:len(gv)][bad][:5]} ref {exp[bad][:5]}")
    diff = np.setxor1d(gv, rv)
    if len(diff):
        ds = score_of(diff)
        far = np.abs(ds - boundary) > t
        assert not far.any(), (f"{what}: positions {diff[far][:5]} differ from the reference set with "
                               f"scores {ds[far][:5]} vs boundary {boundary}")
    return len(diff)


def check_candidates(gpu_C, ref_C, proxy_row, what=""):
    """Refine candidate sets: symmetric difference only at the boundary of the
    reference proxy scores (proxy_row: reference scores of s <= t_last)."""
    assert len(gpu_C) == len(ref_C), f"{what}: |C| {len(gpu_C)} vs {len(ref_C)}"
    assert np.all(np.diff(gpu_C) > 0), f"{what}: candidates not ascending"
    diff = np.setxor1d(gpu_C, ref_C)
    if len(diff) == 0:
        return 0
    rs = proxy_row[ref_C].astype(np.float64)
    boundary = rs.min()
    t = tol(boundary, rs.max())
    ds = proxy_row[diff].astype(np.float64)
    far = np.abs(ds - boundary) > t
    assert not far.any(), f"{what}: candidates {diff[far][:5]} differ away from the boundary {boundary}"
    return len(diff)


# ----------------------------------------------------------- group checks
def _f64(a):
    from workloads import bf16_bits_to_f32
    return bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def member_scores(q, w, k, b, r, positions):
    """Float64 eq. (1) scores of query row r of sequence b over ``positions``."""
    qv = _f64(q[b, r])                                   # [H, d]
    kv = _f64(k[b, positions])                           # [P, d]
    return (w[b, r].astype(np.float64)[:, None] * np.maximum(qv @ kv.T, 0.0)).sum(axis=0)


def _padded(lists, fill=-1):
    n = max([len(x) for x in lists] + [1])
    out = np.full((len(lists), n), fill, dtype=np.int32)
    for i, x in enumerate(lists):
        out[i, :len(x)] = x
    return out


def check_rows(q, w, k, units, gpu_idx, gpu_sc, ref_idx, ref_sc, what, g=None):
    """The float rule on many rows at once. Row i belongs to ``units[i]`` (a
    flat query row for eq. (1) scores, or, with g, a flat group whose proxy
    scores (eq. (5)) judge the row). gpu_* and ref_* are [n, K] (ref: the
    oracle's rows for the same units). Every GPU score must be within RTOL of
    the oracle's score of the same position (oracle.scores_at), and every
    position in the symmetric difference of the two sets within the
    tolerance of the reference boundary. Returns the total difference size."""
    import oracle
    n, K = gpu_idx.shape
    gv, rv = gpu_idx >= 0, ref_idx >= 0
    ng, nr = gv.sum(axis=1), rv.sum(axis=1)
    bad = np.flatnonzero(ng != nr)
    assert not len(bad), f"{what}: valid counts differ at rows {bad[:5]}: {ng[bad[:5]]} vs {nr[bad[:5]]}"
    assert np.array_equal(gv, np.arange(K)[None, :] < ng[:, None]), f"{what}: -1 not only in the tail"
    assert np.all(np.diff(gpu_idx, axis=1)[gv[:, 1:]] > 0), f"{what}: valid entries not strictly ascending"
    rs = np.where(rv, ref_sc, np.nan).astype(np.float64)
    has = nr > 0
    boundary = np.where(has, np.nanmin(np.where(has[:, None], rs, 0.0), axis=1), 0.0)
    row_max = np.where(has, np.nanmax(np.where(has[:, None], rs, 0.0), axis=1), 0.0)
    t = RTOL * np.abs(boundary) + ATOL_FRAC * np.abs(row_max) + 1e-30
    if gpu_sc is not None:
        exp = oracle.scores_at(q, w, k, units, np.where(gv, gpu_idx, -1), g=g).astype(np.float64)
        err = np.abs(gpu_sc.astype(np.float64) - exp)
        lim = RTOL * np.abs(exp) + ATOL_FRAC * np.abs(row_max)[:, None] + 1e-30
        badm = gv & ~(err <= lim)
        if badm.any():
            i, j = np.argwhere(badm)[0]
            raise AssertionError(f"{what}: score mismatch in row {i} (unit {units[i]}) at position "
                                 f"{gpu_idx[i, j]}: gpu {gpu_sc[i, j]} oracle {exp[i, j]}")
    diffs = [np.setxor1d(gpu_idx[i, :ng[i]], ref_idx[i, :nr[i]]) for i in range(n)]
    total = int(sum(len(d) for d in diffs))
    if total:
        D = _padded(diffs)
        ds = oracle.scores_at(q, w, k, units, D, g=g).astype(np.float64)
        far = (D >= 0) & (np.abs(ds - boundary[:, None]) > t[:, None])
        if far.any():
            i, j = np.argwhere(far)[0]
            raise AssertionError(f"{what}: row {i} (unit {units[i]}) position {D[i, j]} differs from the oracle's "
                                 f"set with score {ds[i, j]} vs boundary {boundary[i]}")
    return total


def check_refine_groups(q, w, k, g, topk, c, gpu_idx, gpu_sc, gpu_C, gpu_n, groups=None):
    """The float rule on Refine groups (all of them when ``groups`` is None):
    candidate sets against the oracle's proxy scores (eq. (7) at the
    boundary only), member rows against the oracle's member step (eqs.
    (8)-(9)) run on the GPU's own candidate sets. Returns the total
    symmetric-difference size."""
    import oracle
    B, Lq = q.shape[:2]
    G = -(-Lq // g)
    groups = np.arange(B * G) if groups is None else np.asarray(groups, dtype=np.int64)
    ref = oracle.refine(q, w, k, g, topk, c, groups=groups, want_scores=False)
    given = oracle.refine(q, w, k, g, topk, c, groups=groups, cand_in=gpu_C, cand_in_n=gpu_n)
    b_, m_ = np.divmod(groups, G)
    gC, rC = gpu_C[b_, m_], ref["cand"][b_, m_]
    # eq. (7): the candidate sets as top-c sets of the proxy scores (the
    # oracle's own proxy scores of its C give the boundary)
    rsc = oracle.scores_at(q, w, k, groups, np.where(rC >= 0, rC, -1), g=g)
    diffs = check_rows(q, w, k, groups, gC, None, rC, rsc, "C", g=g)
    # eqs. (8)-(9): member rows on the GPU's C
    rows = np.concatenate([b * Lq + np.arange(m * g, min((m + 1) * g, Lq)) for b, m in zip(b_, m_)])
    rb, rr = np.divmod(rows, Lq)
    diffs += check_rows(q, w, k, rows, gpu_idx[rb, rr], None if gpu_sc is None else gpu_sc[rb, rr],
                        given["indices"][rb, rr], given["scores"][rb, rr], "refine rows")
    return diffs


def check_reuse_groups(q, w, k, g, topk, gpu_idx, gpu_sc, groups=None):
    """The float rule on Reuse groups (all when ``groups`` is None): each
    group's row against the oracle's eq. (6) row by the proxy scores; every
    member row must equal its group's first."""
    import oracle
    B, Lq = q.shape[:2]
    G = -(-Lq // g)
    groups = np.arange(B * G) if groups is None else np.asarray(groups, dtype=np.int64)
    ref = oracle.reuse(q, w, k, g, topk, groups=groups)
    b_, m_ = np.divmod(groups, G)
    r0 = m_ * g
    for j in range(1, g):
        r = np.minimum(r0 + j, Lq - 1)
        assert np.array_equal(gpu_idx[b_, r], gpu_idx[b_, r0]), "reuse: member rows differ within a group"
    return check_rows(q, w, k, groups, gpu_idx[b_, r0], None if gpu_sc is None else gpu_sc[b_, r0],
                      ref["indices"][b_, r0], ref["scores"][b_, r0], "reuse groups", g=g)


def check_dense_rows(q, w, k, topk, gpu_idx, gpu_sc, rows=None):
    """The float rule on dense rows (all when ``rows`` is None; flat b*Lq+r)."""
    import oracle
    B, Lq = q.shape[:2]
    rows = np.arange(B * Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    ref = oracle.dense(q, w, k, topk, rows=rows)
    rb, rr = np.divmod(rows, Lq)
    return check_rows(q, w, k, rows, gpu_idx[rb, rr], None if gpu_sc is None else gpu_sc[rb, rr],
                      ref["indices"][rb, rr], ref["scores"][rb, rr], "dense rows")


def structure_all_rows(idx, Lq, Lk, topk, g=None, counts=None):
    """Vectorised structural checks over every row: -1 only in the tail,
    strictly ascending valid entries, each <= its bound (t, or t_last for
    Reuse), and the valid count where it has a closed form."""
    B, _, K = idx.shape
    valid = idx >= 0
    n = valid.sum(axis=-1)
    ar = np.arange(K)
    assert np.array_equal(valid, ar[None, None, :] < n[..., None]), "-1 entries not confined to the tail"
    d = np.diff(idx, axis=-1)
    both = valid[..., 1:]
    assert np.all(d[both] > 0), "valid entries not strictly ascending"
    pos = np.arange(Lq) + (Lk - Lq)
    if g is not None:
        pos = np.minimum((pos - (Lk - Lq)) // g * g + g, Lq) - 1 + (Lk - Lq)
    last = np.take_along_axis(idx, np.maximum(n - 1, 0)[..., None], axis=-1)[..., 0]
    assert np.all((n == 0) | (last <= pos[None, :])), "index beyond its causal bound"
    if counts is not None:
        assert np.array_equal(n, counts), "valid counts differ from the closed form"
