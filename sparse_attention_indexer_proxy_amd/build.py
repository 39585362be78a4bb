"""Build libpivot.so (HIP, gfx950) in-tree with hipcc.

    python -m sparse_attention_indexer_proxy_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, "pivot_kernels.hip"), os.path.join(CSRC, "pivot_diag.hip"),
           os.path.join(CSRC, "pivot_order.hip"), os.path.join(CSRC, "pivot_api.hip")]
LIB = os.path.join(PKG, "libpivot.so")
PROBE_SRC = os.path.join(CSRC, "mfma_probe.hip")
PROBE = os.path.join(PKG, "mfma_probe")  # practical MFMA / copy ceilings (measurement only)
ARCH = os.environ.get("PIVOT_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU ops stay off: plain fp32 instructions only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the ReLU/weight reduction reads them directly
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libpivot.so)")


def _run_hipcc(cmd, verbose):
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in res.stderr.splitlines() if noise not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build_probe(verbose: bool = False) -> str:
    tmp = PROBE + ".tmp"
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    _run_hipcc([hipcc(), *flags, PROBE_SRC, "-o", tmp], verbose)
    os.replace(tmp, PROBE)
    return PROBE


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    _run_hipcc([hipcc(), *HIPCC_FLAGS, *extra_flags, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    build_probe(verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
