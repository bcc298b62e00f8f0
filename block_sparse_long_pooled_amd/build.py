"""Builds libbslp.so in-tree with hipcc for gfx950.

    python -m block_sparse_long_pooled_amd.build

Every source is compiled as HIP (one object per file, in parallel) and linked
into one shared library next to this file.  Packed fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbslp.so")

SOURCES = ["api.cpp", "pool_scores.hip", "select.hip", "attn_valu.hip", "attn_mfma.hip", "scores_mfma.hip", "quant.hip", "noalloc.hip", "attn_fp8.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE, "-I" + CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


# The fp8 attention keeps every matrix-core accumulator in VGPRs: its 2- and
# 4-wave instantiations would otherwise be given AGPR accumulators for the
# fp8 MFMA, a form whose results read back wrong in an earlier version of
# that kernel.
FILE_FLAGS = {"attn_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
