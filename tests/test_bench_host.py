"""Host-side logic of bench.py (CPU only: nothing here touches a GPU)."""
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "multi-GPU" in r.stderr
    assert r.stdout == ""                              # no JSON line


@pytest.mark.parametrize("workload,mx8", [("verify_32seq", False), ("chunk_8192", True)])
def test_traffic_comes_from_the_committed_counter_summary(workload, mx8):
    # the summary's own figure while the kernel source is the one it was
    # taken on; null otherwise (a kernel edited after its counters were read)
    t = bench.measured_traffic(workload, mx8)
    text = open(os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")).read()
    assert t is None or (t > 0 and f"traffic bytes per launch: {t:.0f}" in text)


def test_traffic_is_dropped_once_the_kernel_source_changes(tmp_path):
    # a copy of the tree's profile next to a kernel source with other bytes
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "mxfp4_expert_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    prof = open(os.path.join(ROOT, "profiles", "hbm_traffic_verify_32seq.md")).read()
    (tmp_path / "profiles" / "hbm_traffic_verify_32seq.md").write_text(prof)
    src = open(os.path.join(ROOT, "mxfp4_expert_ffn_amd", "csrc", "expert_gemm.hip")).read()
    (csrc / "expert_gemm.hip").write_text(src)
    root = str(tmp_path)
    assert bench.measured_traffic("verify_32seq", False, root) is not None      # same bytes: kept
    (csrc / "expert_gemm.hip").write_text(src + "\n// edited\n")
    assert bench.measured_traffic("verify_32seq", False, root) is None          # changed: null
    assert bench.measured_traffic("share_64seq", False, root) is None           # no summary: null


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()
