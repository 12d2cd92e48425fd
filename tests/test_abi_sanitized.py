"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

api.hip's host code is compiled with both sanitizers (host side only:
-Xarch_host before each sanitizer flag) and linked with the library's other
objects and a C driver (abi_sanitize_driver.c) that goes through context
create/destroy, workspace sizing and every entry point's argument checks.
None of those calls reaches a GPU.
"""
import glob
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "mxfp4_expert_ffn_amd", "csrc")
BUILD = os.path.join(ROOT, "mxfp4_expert_ffn_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"


def test_abi_host_code_runs_clean_under_asan_and_ubsan(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANG)):
        pytest.skip("no ROCm compilers")
    objs = [o for o in glob.glob(os.path.join(BUILD, "*.o")) if os.path.basename(o) != "api.o"]
    if len(objs) < 5:
        pytest.skip("library objects not built (run the build first)")
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = tmp_path / "api_asan.o"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-Xclang", "-target-feature",
                    "-Xclang", "-packed-fp32-ops", *inc,
                    "-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all",
                    "-c", os.path.join(CSRC, "api.hip"), "-o", str(api)],
                   check=True, capture_output=True, text=True, timeout=600)
    drv = tmp_path / "driver.o"
    subprocess.run([CLANG, "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", *inc,
                    "-c", os.path.join(HERE, "abi_sanitize_driver.c"), "-o", str(drv)],
                   check=True, capture_output=True, text=True, timeout=300)
    exe = tmp_path / "abi_sanitized"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address,undefined",
                    str(drv), str(api), *objs, "-o", str(exe)],
                   check=True, capture_output=True, text=True, timeout=600)
    # leak checking stays off: the HIP runtime's own start-up allocations are not ours
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "abi sanitizer run: ok" in r.stdout
    assert "runtime error" not in r.stderr
