"""Builds libattn_bwd.so (HIP, gfx950) in-tree, next to this file.

    python -m scaled_dot_product_bwd_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instructions disabled (-packed-fp32-ops) and MFMA results kept in VGPRs.  The sources compile in parallel and
link into one shared library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["abi.cpp", "paged_plan.cpp", "dense_kernels.hip", "paged_kernels.hip",
           "paged_q_kernels.hip", "noalloc.hip"]


def library_path() -> str:
    return os.path.join(HERE, "libattn_bwd.so")


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build")


# -amdgpu-mfma-vgpr-form: MFMA results in VGPRs, so the softmax reads them
# without accumulator-register moves.
# -pragma-unroll-threshold: the fused statistics + dQ step is large; below this
# the compiler leaves some of its `#pragma unroll` loops rolled and indexes the
# fragment and score arrays in scratch memory.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-pragma-unroll-threshold=1000000",
          "-I", INCLUDE, "-I", CSRC]


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(extra=(), verbose=False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    out = library_path()
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(out)
    return out


if __name__ == "__main__":
    build(verbose=True)
