"""Build libmoe_mxfp4.so (HIP, gfx950 only) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe_mxfp4.so")
SOURCES = ["api.hip", "router.hip", "dflash.hip", "probes.hip", "route_sort.hip", "expert_gemm.hip", "fused.hip", "dense_gemm.hip", "combine.hip",
           "quant_act.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 VALU forms are disabled for all device code (see DESIGN notes on
# this machine class); -O3 for gfx950 only.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
# fused.hip: one lane takes the next work unit with an atomic whose result is
# only needed at the end of the current unit; the compiler's atomic optimizer
# would rewrite it into a wave-wide form that waits for the result at once.
EXTRA = {"fused.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        if verbose:
            noise = "is not a recognized feature for this target"
            err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
            if err.strip():
                print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
