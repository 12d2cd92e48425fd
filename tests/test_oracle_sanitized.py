"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

A C driver (oracle_sanitize_driver.c) calls every oracle function on small
and degenerate inputs; built with both sanitizers and no recovery, any
out-of-bounds access, leak or undefined operation fails the run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_sanitized"
    cmd = [gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "oracle sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr
