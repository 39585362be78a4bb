#!/usr/bin/env python3
"""Throughput of the PIVOT indexer on one MI355X.

One step = one full indexer call over the workload (Refine: pool -> fused
proxy scan with top-c selection -> per-member re-score and top-k), inputs
resident in HBM. Prints one JSON line:

  value        query positions per second (B * Lq / step time)
  roofline     the fused proxy-scan kernel alone against the bf16 MFMA peak:
               algorithmic FLOPs per launch (2 d H sum_groups (t_last + 1))
               over its average launch time from hipEvents on its stream;
               roofline_scan_select counts the group select kernel's time too
  cpu_baseline the CPU oracle on a stratified sample of the same groups

    python bench.py [--steps K] [--warmup W] [--variant refine|reuse|dense] [--g G]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import ALL, LONG_128K  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
HBM_PEAK_GBS = 8000.0
HEADLINE_METRIC = "indexer query-positions/sec (Refine g=8, L=128K) + % of bf16 MFMA peak"
SCAN_SRC = os.path.join(ROOT, "sparse_attention_indexer_proxy_amd", "csrc", "pivot_kernels.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "scan_counters.json")


def metric_name(W, variant, g):
    """The headline metric string for its own configuration (128K Refine
    g=8); the same form, naming the workload, for every other run."""
    if W.name == "prefill_L131072" and variant == "refine" and g == 8:
        return HEADLINE_METRIC
    peak = "HBM bandwidth" if W.kind.startswith("decode") else "bf16 MFMA peak"
    return f"indexer query-positions/sec ({variant.capitalize()} g={g}, {W.name}) + % of {peak}"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def group_last_positions(Lq, Lk, g):
    G = -(-Lq // g)
    return Lk - Lq + np.minimum((np.arange(G) + 1) * g, Lq) - 1


def scan_flops(W, g):
    from workloads import seq_lens
    return sum(2.0 * W.d * W.H * float((group_last_positions(W.Lq, int(n), g) + 1).sum()) for n in seq_lens(W))


def refine_flops(W, g, c):
    from workloads import seq_lens
    total = 0.0
    for n in seq_lens(W):
        tl = group_last_positions(W.Lq, int(n), g)
        G = len(tl)
        gm = np.minimum((np.arange(G) + 1) * g, W.Lq) - np.arange(G) * g
        total += 2.0 * W.d * W.H * float((gm * np.minimum(c, tl + 1)).sum())
    return total


def scan_key_bytes(W):
    """Keys each group's scan must read once: every key s <= t_last."""
    from workloads import seq_lens
    return float(sum(int(n) for n in seq_lens(W))) * W.d * (2 if W.dtype == "bf16" else 4)


def kernel_source_hash():
    with open(SCAN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_counters(workload_name, variant, g):
    """Figures from committed rocprofv3 counter runs of this workload (HBM
    bytes per scan launch from FETCH_SIZE / WRITE_SIZE; the shader clock
    from SQ_CYCLES over the scan's duration), if they were taken on the
    current kernel source; else {}."""
    try:
        with open(COUNTERS_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return {}
    ent = rec.get(f"{workload_name}/{variant}/g{g}")
    if not ent or ent.get("kernel_source_sha256_16") != kernel_source_hash():
        return {}
    return ent


def practical_peaks():
    """Run the in-tree probe (dense bf16 MFMA loop with random and with zero
    operands, and a 2 GiB device copy); None if it is not built."""
    import subprocess
    probe = os.path.join(ROOT, "sparse_attention_indexer_proxy_amd", "mfma_probe")
    if not os.path.exists(probe):
        return None
    try:
        res = subprocess.run([probe, "0.5"], capture_output=True, text=True, timeout=120)
        return json.loads(res.stdout.strip().splitlines()[-1]) if res.returncode == 0 else None
    except (subprocess.SubprocessError, ValueError, IndexError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(q, w, k, W, variant, g, budget_s):
    """The oracle on a stratified sample of groups (rows for dense), sized to
    about budget_s seconds; returns the metric-unit rate."""
    import oracle
    threads = oracle.num_threads()
    if W.kind == "decode_ragged":
        from workloads import seq_lens
        lens = seq_lens(W)
        fn = {"dense": lambda b: oracle.dense(q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]], W.topk, want_scores=False),
              "reuse": lambda b: oracle.reuse(q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]], g, W.topk,
                                              want_scores=False),
              "refine": lambda b: oracle.refine(q[b:b + 1], w[b:b + 1], k[b:b + 1, :lens[b]], g, W.topk, W.c,
                                                want_scores=False, want_cand=False)}[variant]
        t0 = time.perf_counter()
        done = 0
        for b in range(W.B):
            fn(b)
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": done * W.Lq / dt, "unit": "query positions/s", "cores": threads, "kind": "oracle",
                "cpu_model": cpu_model(), "nproc": os.cpu_count(),
                "sample": f"{done} of {W.B} sequences (each on its own key prefix), {dt:.1f} s on {threads} threads"}
    per_seq = W.Lq if variant == "dense" else -(-W.Lq // g)
    rows_per_unit = 1 if variant == "dense" else g
    run = {"dense": lambda u: oracle.dense(q, w, k, W.topk, rows=u, want_scores=False),
           "reuse": lambda u: oracle.reuse(q, w, k, g, W.topk, groups=u, want_scores=False),
           "refine": lambda u: oracle.refine(q, w, k, g, W.topk, W.c, groups=u, want_scores=False,
                                             want_cand=False)}[variant]
    # probe: one thread-batch of mid-sequence units gives the time per unit
    probe = np.linspace(per_seq // 2, per_seq // 2 + threads - 1, threads).astype(np.int64) % per_seq
    run(probe)  # untimed: thread start-up and first touches would inflate the estimate
    t0 = time.perf_counter()
    run(probe)
    per_unit = max((time.perf_counter() - t0) / len(probe), 1e-6)
    n = int(max(threads, min(per_seq * W.B, budget_s / per_unit)))
    n = max(threads, n // threads * threads)
    units = np.unique(np.linspace(0, per_seq * W.B - 1, n).astype(np.int64))
    # in at most four chunks (each call also allocates the workload's output
    # rows), with a progress line each: a long budget runs for minutes
    chunk = max(threads * 64, -(-len(units) // 4))
    t0 = time.perf_counter()
    for i in range(0, len(units), chunk):
        run(units[i:i + chunk])
        if len(units) > chunk:
            log(f"[bench] cpu baseline: {min(i + chunk, len(units))} of {len(units)} units, "
                f"{time.perf_counter() - t0:.0f} s")
    dt = time.perf_counter() - t0
    return {"value": len(units) * rows_per_unit / dt, "unit": "query positions/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": (f"{len(units)} of {per_seq * W.B} {'rows' if variant == 'dense' else 'groups'} "
                       f"evenly spaced over the sequence (same mean prefix as the full workload), "
                       f"{dt:.1f} s on {threads} threads")}


def oracle_one_thread():
    """The oracle on one thread for the two small workloads: the tiny f32
    workload in full (Refine), and the exact 8K workload's Refine on 64
    evenly spaced groups. Query positions/s each."""
    import oracle
    from workloads import EXACT, TINY, generate
    before = oracle.num_threads()
    oracle.set_threads(1)
    out = {}
    try:
        for W, n in ((TINY, None), (EXACT, 64)):
            q, w, k = generate(W)
            G = -(-W.Lq // W.g)
            groups = None if n is None else np.unique(np.linspace(0, G - 1, n).astype(np.int64))
            oracle.refine(q, w, k, W.g, W.topk, W.c, groups=groups[:1] if groups is not None else [0],
                          want_scores=False, want_cand=False)
            t0 = time.perf_counter()
            oracle.refine(q, w, k, W.g, W.topk, W.c, groups=groups, want_scores=False, want_cand=False)
            dt = time.perf_counter() - t0
            rows = W.Lq if groups is None else len(groups) * W.g
            out[W.name] = {"value": rows / dt, "unit": "query positions/s", "cores": 1,
                           "sample": "all groups" if groups is None else f"{len(groups)} of {G} groups evenly spaced"}
    finally:
        oracle.set_threads(before)
    return out


def copy_calibration(torch, mib):
    """A plain device-to-device copy of known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch against mib MiB gives the factor that
    turns those counters into HBM bytes."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "dispatches": 3}), flush=True)


def bench_stats(torch, pv, W, args, g, tq, tw, tk, ws):
    """The O1-O3 diagnostics on this workload's rows: one JSON line with the
    time per call and the statistics' means. Algorithmic bytes: the index and
    score rows read once (mass reads both)."""
    if args.variant == "refine":
        idx, sc = pv.index_refine(tq, tw, tk, g, W.topk, W.c, workspace=ws, return_scores=True)
    elif args.variant == "reuse":
        idx, sc = pv.index_reuse(tq, tw, tk, g, W.topk, workspace=ws, return_scores=True)
    else:
        idx, sc = pv.index_dense(tq, tw, tk, W.topk, workspace=ws, return_scores=True)
    torch.cuda.synchronize()
    sg = max(g, W.g)
    out = pv.index_stats(idx, sc, d=1, g=sg)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        out = pv.index_stats(idx, sc, d=1, g=sg)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = 2.0 * idx.numel() * 4
    ov = out["overlap"]
    res = {"metric": "index-row diagnostics (O1-O3) per call", "value": ms, "unit": "ms", "higher_is_better": False,
           "config": {"workload": f"{W.name} PIVOT-{args.variant} rows", "g": g, "group_g": sg, "topk": W.topk},
           "roofline": {"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
           "adjacent_overlap_over_k": float(ov[ov >= 0].float().mean()) / W.topk,
           "group_union_over_k": float(out["union"].float().mean()) / W.topk,
           "group_inter_over_k": float(out["inter"].float().mean()) / W.topk,
           "mass_at_k4_k2_3k4": [float(x) for x in out["mass"].nanmean(dim=(0, 1)).cpu()]}
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=LONG_128K.name, choices=sorted(ALL))
    ap.add_argument("--variant", default="refine", choices=["refine", "reuse", "dense"])
    ap.add_argument("--g", type=int, default=None, help="group size (default: the workload's)")
    ap.add_argument("--heads", type=int, default=None,
                    help="indexer heads (default: the workload's 64; 32 runs the 32-head MFMA kernels)")
    ap.add_argument("--order", default="position", choices=["position", "score"],
                    help="row order: ascending position (default) or rank order (adds the rank pass)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--stats", action="store_true",
                    help="time the O1-O3 diagnostics (pivot_index_stats) on the variant's rows instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB a few times (scales HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the indexer's groups "
              "would be split across GPUs; see the sharding notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        return copy_calibration(torch, args.copy_calibration)
    import sparse_attention_indexer_proxy_amd as pv

    W = ALL[args.workload]
    if args.heads:
        W = W.replace(H=args.heads, name=f"{W.name}_H{args.heads}")
    g = 1 if args.variant == "dense" else (args.g or W.g)
    t0 = time.perf_counter()
    from workloads import generate, to_device, seq_lens, paged_layout
    q, w, k = generate(W)
    log(f"[bench] generated {W.name} in {time.perf_counter() - t0:.1f} s")
    tq, tw, tk = to_device(q, w, k)
    dev = tq.device
    variant_id = {"dense": pv.DENSE, "reuse": pv.REUSE, "refine": pv.REFINE}[args.variant]
    ragged = W.kind == "decode_ragged"
    if ragged:
        # ragged lengths, keys in a shuffled pool of 64-key pages
        lens = seq_lens(W)
        pool, table = paged_layout(k, lens, 64, W.seed)
        tpool = to_device(q[:1], w[:1], pool)[2]
        ttable, tlens = torch.from_numpy(table).to(dev), torch.from_numpy(lens).to(dev)
        kcfg = pv.make_config(variant=variant_id, g=g, topk=W.topk, c=W.c, order=args.order)
        ws = None
        log(f"[bench] ragged: lengths {int(lens.min())}..{int(lens.max())}, {pool.shape[0]} pages of 64 keys")
    else:
        ws = torch.empty(pv.workspace_size(variant_id, W.B, W.Lq, W.Lk, W.H, W.d, tq.dtype, g, W.topk, W.c),
                         dtype=torch.uint8, device=dev)
        log(f"[bench] workspace {ws.numel() / 2**30:.2f} GiB")

    ocfg = pv.make_config(variant=variant_id, g=g, topk=W.topk, c=W.c, order=args.order)

    def step():
        if ragged:
            return pv.index_kv(tq, tw, tpool, tlens, ttable, page_size=64, lk=W.Lk, cfg=kcfg)
        if args.order != "position":
            return pv.index(tq, tw, tk, ocfg, workspace=ws)
        if args.variant == "refine":
            return pv.index_refine(tq, tw, tk, g, W.topk, W.c, workspace=ws)
        if args.variant == "reuse":
            return pv.index_reuse(tq, tw, tk, g, W.topk, workspace=ws)
        return pv.index_dense(tq, tw, tk, W.topk, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    if args.stats:
        return bench_stats(torch, pv, W, args, g, tq, tw, tk, ws)

    # timed region: plain calls, as a caller would make them
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    del out
    # per-kernel durations: the same steps again with every launch bracketed
    # by hipEvents on its stream
    pv.timing_enable(True)
    for _ in range(args.steps):
        out = step()
    torch.cuda.synchronize()
    stages = pv.timing_read()
    pv.timing_enable(False)
    del out

    # per-call durations from hipEvents around each ABI call on its stream
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record(stream)
        out = step()
        e1.record(stream)
    torch.cuda.synchronize()
    call_ms = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    median_call_ms = call_ms[len(call_ms) // 2]
    del out
    practical = practical_peaks()

    ms_per_step = 1e3 * wall / args.steps
    qpos = W.B * W.Lq
    value = qpos / (wall / args.steps)
    scan_ms, scan_n = stages["scan"]
    scan_avg_s = scan_ms / max(scan_n, 1) / 1e3
    sflops = scan_flops(W, g)
    achieved = sflops / scan_avg_s / 1e12
    total_flops = sflops + (refine_flops(W, g, W.c) if args.variant == "refine" else 0.0)
    kernels = {name: round(ms / max(n, 1), 4) for name, (ms, n) in stages.items() if n}
    log(f"[bench] {args.variant} g={g}: {ms_per_step:.3f} ms/step, kernels (ms/launch) {kernels}")

    counters = recorded_counters(W.name, args.variant, g)
    roofline_scan_select = None
    if W.kind.startswith("decode"):
        # one group per sequence: the split-key scan reads every key once and
        # meets it with only H rows, so HBM bounds it
        kbytes = scan_key_bytes(W)
        gbs = kbytes / scan_avg_s / 1e9
        roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                    "traffic": None, "kernel": "split-key proxy scan, eq. (5) score rows (k_scan_split)",
                    "bytes_per_launch": kbytes}
    else:
        roofline = {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": counters.get("hbm_bytes_per_launch"),
                    "kernel": "fused proxy scan, eq. (5) with its streaming top-K filter (k_scan_mfma alone)",
                    "flops_per_launch": sflops}
        sel_ms, sel_n = stages["scan_select"]
        if sel_n:
            both_s = scan_avg_s + sel_ms / sel_n / 1e3
            a2 = sflops / both_s / 1e12
            roofline_scan_select = {
                "bound": "mfma", "achieved": a2, "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": a2 / MFMA_BF16_PEAK_TFLOPS,
                "kernel": "proxy scan + its final top-K / top-c select, eqs. (5)-(7) (k_scan_mfma + k_select_groups)",
                "flops_per_launch": sflops}

    cpu = None
    one_thread = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(q, w, k, W, args.variant, g, args.cpu_seconds)
        log(f"[bench] cpu baseline: {cpu}")
        one_thread = oracle_one_thread()
        log(f"[bench] oracle on one thread: {one_thread}")

    res = {
        "metric": metric_name(W, args.variant, g),
        "value": value,
        "unit": "query positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if W.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{W.name} PIVOT-{args.variant}", "batch": W.B, "seq_len": W.Lk,
                   "query_rows": W.Lq, "heads": W.H, "dim": W.d, "g": g, "topk": W.topk,
                   "c": W.c if args.variant == "refine" else None, "parallelism": "single GPU",
                   **({"order": args.order} if args.order != "position" else {})},
        "roofline": roofline,
        "roofline_scan_select": roofline_scan_select,
        "cpu_baseline": cpu,
        "oracle_one_thread": one_thread,
        "sclk_ghz_observed": counters.get("sclk_ghz"),
        "sclk_source": ("SQ_CYCLES per shader engine over the scan's traced duration, from the rocprofv3 counter run "
                        "of this kernel source (profiles/scan_counters.json); not measured in this run"
                        if counters.get("sclk_ghz") else None),
        "median_call_ms": median_call_ms,
        "practical_peak": practical,
        "scan_frac_of_practical_mfma": (achieved / practical["mfma_bf16_random_tflops"]
                                        if practical and practical.get("mfma_bf16_random_tflops") else None),
        "kernels_ms_per_launch": kernels,
        "whole_call_mfma_frac": total_flops / (wall / args.steps) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
