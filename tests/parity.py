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


def check_refine_groups(q, w, k, g, topk, c, gpu_idx, gpu_sc, gpu_C, gpu_n, groups):
    """Float rule on sampled Refine groups: candidate sets against the oracle's
    proxy scores, member rows against the oracle's member step run on the
    GPU's own candidate sets. Returns the total symmetric-difference size."""
    import oracle
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    G = -(-Lq // g)
    ref = oracle.refine(q, w, k, g, topk, c, groups=groups)
    given = oracle.refine(q, w, k, g, topk, c, groups=groups, cand_in=gpu_C, cand_in_n=gpu_n)
    diffs = 0
    for u in groups:
        b, m = divmod(int(u), G)
        prow = oracle.proxy_row(q, w, k, g, b, m)
        n = gpu_n[b, m]
        diffs += check_candidates(gpu_C[b, m, :n], ref["cand"][b, m, :ref["cand_n"][b, m]], prow,
                                  f"C of group {b}/{m}")
        for r in range(m * g, min((m + 1) * g, Lq)):
            diffs += compare_row(gpu_idx[b, r], None if gpu_sc is None else gpu_sc[b, r],
                                 given["indices"][b, r], given["scores"][b, r],
                                 lambda p, b=b, r=r: member_scores(q, w, k, b, r, p), f"refine row {b}/{r}")
    return diffs


def check_reuse_groups(q, w, k, g, topk, gpu_idx, gpu_sc, groups):
    import oracle
    B, Lq = q.shape[:2]
    G = -(-Lq // g)
    ref = oracle.reuse(q, w, k, g, topk, groups=groups)
    diffs = 0
    for u in groups:
        b, m = divmod(int(u), G)
        prow = oracle.proxy_row(q, w, k, g, b, m).astype(np.float64)
        r0 = m * g
        diffs += compare_row(gpu_idx[b, r0], None if gpu_sc is None else gpu_sc[b, r0], ref["indices"][b, r0],
                             ref["scores"][b, r0], lambda p: prow[p], f"reuse group {b}/{m}")
        rows = gpu_idx[b, r0:min(r0 + g, Lq)]
        assert np.all(rows == rows[0]), f"reuse group {b}/{m}: member rows differ"
    return diffs


def check_dense_rows(q, w, k, topk, gpu_idx, gpu_sc, rows):
    import oracle
    B, Lq = q.shape[:2]
    Lk = k.shape[1]
    ref = oracle.dense(q, w, k, topk, rows=rows)
    diffs = 0
    for u in rows:
        b, r = divmod(int(u), Lq)
        t = Lk - Lq + r
        diffs += compare_row(gpu_idx[b, r], None if gpu_sc is None else gpu_sc[b, r], ref["indices"][b, r],
                             ref["scores"][b, r], lambda p, b=b, r=r: member_scores(q, w, k, b, r, p),
                             f"dense row {b}/{r}")
    return diffs


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
