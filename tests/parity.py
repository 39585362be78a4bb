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
