"""Build libbitgemm.so in-tree with hipcc for gfx950.

Usage: ``python -m bit_gemm_w4_amd.build`` (or ``__graft_entry__.build()``).
Each HIP source is compiled to an object in parallel, then linked into
``bit_gemm_w4_amd/libbitgemm.so``.  Packed-FP32 instructions are disabled
(``-packed-fp32-ops``): the kernels never rely on them.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libbitgemm.so")
OBJDIR = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


# Per-source extra flags.  Kernels whose MFMA accumulators are read by VALU
# code inside the K loop keep MFMA results in VGPRs: the AGPR form adds a
# v_accvgpr_read per value (the W4A16 decode kernels: 2 % on the widest
# layer; the block-scaled FP8 GEMM, which scales and adds its accumulators
# every 128-wide K block: 6-10 % at M = 2048; the other W8A8 tile kernels
# in the same file measured unchanged).
FILE_FLAGS = {
    "k_w4a16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_w8a8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build()
