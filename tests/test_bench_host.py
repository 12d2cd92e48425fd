"""Host-side logic of bench.py (CPU only: nothing here touches a GPU)."""
import hashlib
import os
import re
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
    text = open(os.path.join(ROOT, "profiles", f"beyond_l2_bytes_{workload}.md")).read()
    assert t is None or (t > 0 and f"traffic bytes per launch: {t:.0f}" in text)


def test_traffic_is_dropped_once_the_kernel_source_changes(tmp_path):
    # a copy of the tree's profile next to a kernel source with other bytes
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "mxfp4_expert_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    prof = open(os.path.join(ROOT, "profiles", "beyond_l2_bytes_verify_32seq.md")).read()
    src = "// a kernel source\n"
    digest = hashlib.sha256(src.encode()).hexdigest()
    prof = re.sub(r"kernel source sha256: `[0-9a-f]+`", f"kernel source sha256: `{digest}`", prof)
    prof = re.sub(r"kernel source: .*", "kernel source: `mxfp4_expert_ffn_amd/csrc/expert_gemm.hip`", prof)
    (tmp_path / "profiles" / "beyond_l2_bytes_verify_32seq.md").write_text(prof)
    (csrc / "expert_gemm.hip").write_text(src)
    root = str(tmp_path)
    assert bench.measured_traffic("verify_32seq", False, root) is not None      # same bytes: kept
    (csrc / "expert_gemm.hip").write_text(src + "\n// edited\n")
    assert bench.measured_traffic("verify_32seq", False, root) is None          # changed: null
    assert bench.measured_traffic("share_64seq", False, root) is None           # no summary: null


def test_traffic_is_dropped_once_a_header_of_the_kernel_changes(tmp_path):
    # a kernel built from several sources: the summary hashes them in order,
    # so editing any of them (here the shared pipeline header) drops the figure
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "mxfp4_expert_ffn_amd" / "csrc"
    csrc.mkdir(parents=True)
    files = {"expert_gemm.hip": "// kernel\n", "stream_pipe.hpp": "// pipeline\n", "common.hpp": "// common\n"}
    for n, t in files.items():
        (csrc / n).write_text(t)
    digest = hashlib.sha256("".join(files.values()).encode()).hexdigest()
    listed = ", ".join(f"`mxfp4_expert_ffn_amd/csrc/{n}`" for n in files)
    prof = open(os.path.join(ROOT, "profiles", "beyond_l2_bytes_verify_32seq.md")).read()
    prof = re.sub(r"kernel source sha256: `[0-9a-f]+`", f"kernel source sha256: `{digest}`", prof)
    prof = re.sub(r"kernel source: .*", f"kernel source: {listed}", prof)
    (tmp_path / "profiles" / "beyond_l2_bytes_verify_32seq.md").write_text(prof)
    root = str(tmp_path)
    assert bench.measured_traffic("verify_32seq", False, root) is not None
    (csrc / "stream_pipe.hpp").write_text("// pipeline, edited\n")
    assert bench.measured_traffic("verify_32seq", False, root) is None


def test_cpu_model_is_a_string():
    assert isinstance(bench.cpu_model(), str) and bench.cpu_model()


def test_every_bench_command_in_the_profiles_parses():
    # each summary under profiles/ names the command that produced it; the
    # bench arguments of every such command must still be accepted as written
    import glob
    import shlex
    n = 0
    for p in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(p):
            if "bench.py" not in line or not line.startswith("    "):
                continue
            words = shlex.split(line.strip())
            i = next(j for j, w in enumerate(words) if w.endswith("bench.py"))
            rest = []
            for w in words[i + 1:]:
                if w in (">", "2>", "&&", "|") or w.startswith(">"):
                    break
                rest.append(w)
            args = bench.parse_args(rest)
            assert args.gpus == 1, (p, line)
            n += 1
    assert n >= 20
