"""Build libbigemm.so (hipcc, gfx950) in-tree.

    python -m invariant_gemm_amd.build          # or __graft_entry__.build()

Every .hip file under csrc/ is compiled to an object in parallel, then linked
into invariant_gemm_amd/libbigemm.so next to the Python binding.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbigemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CXXFLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",        # every fp32 operation rounds as written
    "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


# Kernels whose K loop feeds MFMA results to the VALU (a block product scaled
# and added by an FMA) keep those results in ordinary VGPRs instead of
# accumulation registers, which saves one v_accvgpr_read per element.  The
# instructions and their order are otherwise unchanged (same bits); measured
# 3-16 % faster for these files and neutral or slower for the others.
PER_FILE_FLAGS = {
    name: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
    for name in ("gemm_fp8_packed.hip", "gemm_fp4.hip", "gemm_fp4_packed.hip",
                 "gemm_w4a8_packed.hip")
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    extra = PER_FILE_FLAGS.get(os.path.basename(src), [])
    cmd = [HIPCC, *CXXFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if noise not in l and l.strip()]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
