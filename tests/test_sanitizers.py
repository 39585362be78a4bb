"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The oracle (plain C, gcc) and the C ABI library's host side (hipcc, with
-fsanitize applied to the host pass only) are built with ASan + UBSan
(-fno-sanitize-recover: the first report aborts the process) and exercised
in a subprocess that preloads the sanitizer runtime: every oracle entry point
on ragged f32/bf16 inputs (results compared with the normal build), and
every argument check, workspace computation and refusal path of the ABI that
runs without a GPU."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_indexer_proxy_amd", "csrc")

pytestmark = pytest.mark.slow


def _run(code, preload, tmp):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1",
               LD_PRELOAD=preload, PYTHONPATH=ROOT)
    res = subprocess.run([sys.executable, "-c", textwrap.dedent(code)], env=env, cwd=str(tmp),
                         capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, f"sanitized run failed:\n{res.stdout[-3000:]}\n{res.stderr[-6000:]}"
    return res.stdout


def test_oracle_under_asan_and_ubsan(tmp_path):
    lib = tmp_path / "oracle_san.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(ROOT, "oracle", "pivot_oracle.c"), "-o", str(lib), "-lm"], check=True)
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    ubsan = subprocess.run(["gcc", "-print-file-name=libubsan.so"], capture_output=True, text=True).stdout.strip()
    out = _run(f"""
        import numpy as np, oracle
        from workloads import gauss_random, BF16, F32
        san = {str(lib)!r}
        for dt in (F32, BF16):
            q, w, k = gauss_random(1, 2, 37, 50, 3, 8, dt)
            for v, kw in ((0, {{}}), (1, {{}}), (2, {{}}), (1, dict(member_causal=True)), (2, dict(agg="first")),
                          (1, dict(agg="last"))):
                a = oracle.run(v, q, w, k, 5, 4, 9, lib_path=san, **kw)
                b = oracle.run(v, q, w, k, 5, 4, 9, **kw)
                np.testing.assert_array_equal(a["indices"], b["indices"])
                np.testing.assert_array_equal(a["scores"], b["scores"])
            r = oracle.refine(q, w, k, 4, 5, 9)
            a = oracle.refine(q, w, k, 4, 5, 9, groups=[1, 12], cand_in=r["cand"], cand_in_n=r["cand_n"], lib_path=san)
            np.testing.assert_array_equal(oracle.pool(q, w, 4, lib_path=san)[0], oracle.pool(q, w, 4)[0])
            np.testing.assert_array_equal(oracle.proxy_row(q, w, k, 4, 1, 9, lib_path=san),
                                          oracle.proxy_row(q, w, k, 4, 1, 9))
            pos = np.array([[0, 49, -1, 60], [5, 7, 2, 0]])
            np.testing.assert_array_equal(oracle.scores_at(q, w, k, [0, 73], pos, lib_path=san),
                                          oracle.scores_at(q, w, k, [0, 73], pos))
            np.testing.assert_array_equal(oracle.scores_at(q, w, k, [0, 19], pos, g=4, lib_path=san),
                                          oracle.scores_at(q, w, k, [0, 19], pos, g=4))
        print("oracle sanitized ok")
        """, f"{asan}:{ubsan}", tmp_path)
    assert "oracle sanitized ok" in out


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    rts = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's ASan runtime is not installed")
    lib = tmp_path / "libpivot_san.so"
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    from sparse_attention_indexer_proxy_amd import build as b
    flags = [f for f in b.HIPCC_FLAGS if f not in ("-O3",)]
    res = subprocess.run([b.hipcc(), *flags, "-O1", "-g", *san, "-I", os.path.join(ROOT, "include"), *b.SOURCES,
                          "-o", str(lib)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    out = _run(f"""
        import ctypes
        import sparse_attention_indexer_proxy_amd as pv
        lib = pv.load_library({str(lib)!r})
        sz = ctypes.c_size_t(0)
        P = lambda B=1, Lq=64, Lk=64, H=64, D=128, dt=1: pv.Problem(B, Lq, Lk, H, D, dt)
        cases = [(P(), 2, 8, 16, 32), (P(Lq=65), 1, 8, 16, 0), (P(B=0), 0, 1, 16, 0), (P(), 1, 0, 16, 0),
                 (P(), 2, 8, 16, 8), (P(dt=7), 0, 1, 16, 0), (P(D=12), 0, 1, 16, 0),
                 (P(Lk=2 ** 31, Lq=4), 0, 1, 16, 0), (P(), 9, 1, 16, 0), (P(H=48, Lq=131072, Lk=131072), 2, 8, 2048, 4096),
                 (P(Lq=131072, Lk=131072), 2, 8, 2048, 4096), (P(B=32, Lq=4, Lk=65536), 2, 4, 2048, 4096)]
        got = [lib.pivot_workspace_size(ctypes.byref(p), v, g, k, c, ctypes.byref(sz)) for p, v, g, k, c in cases]
        assert got == [0, 1, 1, 1, 1, 1, 2, 1, 1, 2, 0, 0], got
        for v in range(4):
            cfg = pv.make_config(variant=v, g=8, topk=16, c=32, member_causal=(v == 1))
            for path in range(3):
                cfg.scan_path = path
                assert lib.pivot_index_workspace_size(ctypes.byref(P()), ctypes.byref(cfg), ctypes.byref(sz)) == 0
                out = ctypes.c_int32(0)
                assert lib.pivot_resolve_variant(ctypes.byref(P()), ctypes.byref(cfg), ctypes.byref(out)) == 0
        keys = pv.Keys()
        keys.k, keys.page_table, keys.page_size, keys.num_pages, keys.max_pages = 1 << 20, 1 << 21, 16, 8, 4
        cfg = pv.make_config(variant=2, g=8, topk=16, c=32)
        assert lib.pivot_index_kv_workspace_size(ctypes.byref(P()), ctypes.byref(cfg), ctypes.byref(keys),
                                                 ctypes.byref(sz)) == 0
        keys.max_pages = 2
        assert lib.pivot_index_kv_workspace_size(ctypes.byref(P()), ctypes.byref(cfg), ctypes.byref(keys),
                                                 ctypes.byref(sz)) == 1
        fake, idx = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
        assert lib.pivot_index_dense(ctypes.byref(P()), None, fake, fake, 16, idx, None, fake, 1 << 30, None) == 1
        assert lib.pivot_index_refine(ctypes.byref(P()), fake, fake, fake, 8, 16, 32, idx, None, None, None, fake, 16,
                                      None) == 3
        big = pv.make_config(variant=2, g=8, topk=2048, c=4096)
        assert lib.pivot_index_static(ctypes.byref(P(Lq=32768, Lk=32768)), ctypes.byref(big), fake, fake, fake, idx,
                                      None, None, None, None) == 3
        assert lib.pivot_index_stats(1, 4, 0, idx, None, 1, 1, idx, None, None, None, None) == 2
        for s in range(6):
            lib.pivot_status_str(s)
        assert lib.pivot_last_error()
        print("abi sanitized ok")
        """, rts[-1], tmp_path)
    assert "abi sanitized ok" in out
