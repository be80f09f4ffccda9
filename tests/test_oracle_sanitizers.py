"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only) and run over every entry point on small inputs with the
edge cases its callers reach: empty and one-position contexts, fewer
candidates than K, ties, padding (-1) entries, rows outside the cache, partial
pool blocks, a zero FP8 key row, a query with no valid key.  Any invalid
memory access, overflow or other undefined behaviour aborts the driver."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "oracle_sanitize_driver")
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "oracle"),
           "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.cpp"), os.path.join(ROOT, "oracle", "csa2_ref.cpp")]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-2000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert "oracle sanitizer driver: ok" in r.stdout
