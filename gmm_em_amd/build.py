"""Build the HIP library libgmm_em.so in-tree for gfx950.

Usage: python -m gmm_em_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgmm_em.so")
SOURCES = ["gmm_api.hip", "gmm_kernels.hip", "gmm_wide.hip", "gmm_ivf.hip", "gmm_i8.hip",
           "gmm_b16.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops stay off: ordinary float code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: long-lived MFMA operands (the statistics passes'
    # resident coefficient digits) go to the accumulator registers instead,
    # so the VALU reads the products without v_accvgpr_read copies
    "-mllvm", "--amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then link."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    cflags = [f for f in FLAGS if f != "-shared"]

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *cflags, *inc, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        return obj

    jobs = int(os.environ.get("MAX_JOBS", "0") or 0) or min(len(SOURCES), os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as pool:
        objs = list(pool.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
