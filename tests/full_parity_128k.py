"""Float-rule parity of the 128K workload on every group (Refine, Reuse) or on
many evenly spaced rows (dense).

A long check, run by hand on a GPU host (the test suite samples 512 Refine
groups of this workload; this script covers all 16384 in chunks, printing a
line per chunk):

    python tests/full_parity_128k.py [--variant refine|reuse|dense] [--g 8]
                                     [--first M] [--last M] [--chunk N] [--dense-rows R]

It makes one library call on the whole workload (prefill L = 131072, H = 64,
d = 128, bf16, k = 2048, c = 4096), then, chunk by chunk, runs the CPU oracle
on those groups and applies the float rule of ``tests/parity.py``: Refine:
every candidate set C against the oracle's top-c of the proxy scores (eq.
(7)), every member row against the oracle's eqs. (8)-(9) run on the
library's own C; Reuse: every group row against the oracle's eq. (6) row;
dense: rows against eq. (1). Scores must agree within 1e-3 relative, and
every position in which the sets differ must lie within the tolerance of the
oracle's boundary score. Exit status 0 when every checked unit passes.
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
    ap.add_argument("--variant", default="refine", choices=["refine", "reuse", "dense"])
    ap.add_argument("--g", type=int, default=None, help="group size (default: the workload's 8)")
    ap.add_argument("--dense-rows", type=int, default=4096, help="dense: evenly spaced rows checked")
    ap.add_argument("--first", type=int, default=0, help="first group")
    ap.add_argument("--last", type=int, default=None, help="last group (inclusive)")
    ap.add_argument("--chunk", type=int, default=1024, help="groups per oracle call")
    args = ap.parse_args()

    import torch
    import sparse_attention_indexer_proxy_amd as pv

    W = LONG_128K
    g = 1 if args.variant == "dense" else (args.g or W.g)
    G = -(-W.Lq // g)
    t0 = time.perf_counter()
    q, w, k = generate(W)
    tq, tw, tk = to_device(q, w, k)
    if args.variant == "refine":
        outs = pv.index_refine(tq, tw, tk, g, W.topk, W.c, return_scores=True, return_candidates=True)
    elif args.variant == "reuse":
        outs = pv.index_reuse(tq, tw, tk, g, W.topk, return_scores=True)
    else:
        outs = pv.index_dense(tq, tw, tk, W.topk, return_scores=True)
    torch.cuda.synchronize()
    outs = [t.cpu().numpy() for t in outs]
    del tq, tw, tk
    if args.variant == "dense":
        units = np.unique(np.linspace(0, W.Lq - 1, args.dense_rows).astype(np.int64))
    else:
        last = G - 1 if args.last is None else min(args.last, G - 1)
        units = np.arange(args.first, last + 1)
    print(f"[full parity] library call done ({time.perf_counter() - t0:.0f} s); {args.variant} g={g}, "
          f"{len(units)} units from {units[0]} to {units[-1]}", flush=True)
    parity.structure_all_rows(outs[0], W.Lq, W.Lk, W.topk, g=g if args.variant == "reuse" else None)
    if args.variant == "refine":
        tl = np.minimum((np.arange(G) + 1) * g, W.Lq) - 1
        assert np.array_equal(outs[3][0], np.minimum(W.c, tl + 1)), "candidate counts"
    swaps = checked = 0
    for at in range(0, len(units), args.chunk):
        chunk = units[at:at + args.chunk]
        if args.variant == "refine":
            d = parity.check_refine_groups(q, w, k, g, W.topk, W.c, *outs, chunk)
        elif args.variant == "reuse":
            d = parity.check_reuse_groups(q, w, k, g, W.topk, outs[0], outs[1], chunk)
        else:
            d = parity.check_dense_rows(q, w, k, W.topk, outs[0], outs[1], chunk)
        swaps += d
        checked += len(chunk)
        print(f"[full parity] units {chunk[0]}..{chunk[-1]} pass ({d} boundary swaps); {checked} checked, "
              f"{time.perf_counter() - t0:.0f} s", flush=True)
    print(f"[full parity] PASS: {checked} {'rows' if args.variant == 'dense' else 'groups'} of {W.name} "
          f"{args.variant} g={g}, {swaps} boundary swaps in total", flush=True)


if __name__ == "__main__":
    main()
