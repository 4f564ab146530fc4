"""The CPU oracle built with the address and undefined-behaviour sanitizers.

oracle/oracle.c is compiled with gcc -fsanitize=address,undefined
(-fno-sanitize-recover, so any report aborts) together with
tests/oracle_sanitized_main.c, a driver that calls every oracle function on
exactly-sized heap buffers and checks each result against a closed form or a
brute-force recomputation.  A plain executable needs no preloaded sanitizer
runtime.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fno-fast-math",
           "-ffp-contract=off", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-Wextra",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_sanitized_main.c"),
           "-o", exe, "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitized run: OK" in r.stdout
