"""Writes tests/golden/input_manifest.json: the SHA-256 of every array the
seeded generators produce for the measured workloads (q, w, k and, for the
ragged decode, the sequence lengths and the paged layout of the benchmark).
It calls only the generators in workloads/ (no indexer arithmetic). Any change
to a generator, a seed or a reading of the input recipe changes a digest, and
tests/test_input_manifest.py fails until this script is re-run and the change
is committed with its reason.

    python tests/golden/make_input_manifest.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from workloads import ALL, generate, paged_layout, seq_lens  # noqa: E402

OUT = os.path.join(HERE, "input_manifest.json")


def digest(a: np.ndarray) -> dict:
    a = np.ascontiguousarray(a)
    return {"shape": list(a.shape), "dtype": str(a.dtype), "sha256": hashlib.sha256(a.tobytes()).hexdigest()}


def workload_digests(name: str) -> dict:
    W = ALL[name]
    q, w, k = generate(W)
    out = {"q": digest(q), "w": digest(w), "k": digest(k)}
    if W.kind == "decode_ragged":
        lens = seq_lens(W)
        pool, table = paged_layout(k, lens, 64, W.seed)
        out.update({"seq_lens": digest(lens), "page_pool_64": digest(pool), "page_table_64": digest(table)})
    return out


def main():
    manifest = {name: workload_digests(name) for name in sorted(ALL)}
    with open(OUT, "w") as f:
        json.dump(manifest, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
