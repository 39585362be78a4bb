"""Float-rule parity of the 128K PIVOT-Refine g=8 workload on every group.

A long check, run by hand on a GPU host (the test suite samples 512 groups of
this workload; this script covers all 16384 in chunks, printing a line per
chunk):

    python tests/full_parity_128k.py [--first M] [--last M] [--chunk N]

It makes one library call on the whole workload (prefill L = 131072, H = 64,
d = 128, bf16, k = 2048, c = 4096), then, chunk by chunk, runs the CPU oracle
on those groups and applies the float rule of ``tests/parity.py``: every
candidate set C against the oracle's top-c of the proxy scores (eq. (7)),
every member row against the oracle's eqs. (8)-(9) run on the library's own
C, scores within 1e-3 relative, and every position in which the sets differ
within the tolerance of the oracle's boundary score. Exit status 0 when every
checked group passes.
"""
import argparse
import os
import sys
import time

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from tests import parity  # noqa: E402
from workloads import LONG_128K, generate, to_device  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--first", type=int, default=0, help="first group")
    ap.add_argument("--last", type=int, default=None, help="last group (inclusive)")
    ap.add_argument("--chunk", type=int, default=1024, help="groups per oracle call")
    args = ap.parse_args()

    import torch
    import sparse_attention_indexer_proxy_amd as pv

    W = LONG_128K
    G = -(-W.Lq // W.g)
    last = G - 1 if args.last is None else min(args.last, G - 1)
    t0 = time.perf_counter()
    q, w, k = generate(W)
    tq, tw, tk = to_device(q, w, k)
    f_i, f_s, f_c, f_n = pv.index_refine(tq, tw, tk, W.g, W.topk, W.c, return_scores=True, return_candidates=True)
    torch.cuda.synchronize()
    f_i, f_s, f_c, f_n = (t.cpu().numpy() for t in (f_i, f_s, f_c, f_n))
    del tq, tw, tk
    print(f"[full parity] library call done ({time.perf_counter() - t0:.0f} s); groups {args.first}..{last}",
          flush=True)
    tl = np.minimum((np.arange(G) + 1) * W.g, W.Lq) - 1
    assert np.array_equal(f_n[0], np.minimum(W.c, tl + 1)), "candidate counts"
    parity.structure_all_rows(f_i, W.Lq, W.Lk, W.topk)
    swaps = checked = 0
    for lo in range(args.first, last + 1, args.chunk):
        hi = min(lo + args.chunk, last + 1)
        groups = np.arange(lo, hi)
        d = parity.check_refine_groups(q, w, k, W.g, W.topk, W.c, f_i, f_s, f_c, f_n, groups)
        swaps += d
        checked += len(groups)
        print(f"[full parity] groups {lo}..{hi - 1} pass ({d} boundary swaps); {checked} checked, "
              f"{time.perf_counter() - t0:.0f} s", flush=True)
    print(f"[full parity] PASS: {checked} groups of {W.name} Refine g={W.g}, {swaps} boundary swaps in total",
          flush=True)


if __name__ == "__main__":
    main()
