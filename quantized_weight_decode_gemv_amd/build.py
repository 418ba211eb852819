"""Build libqwg.so (gfx950 HIP kernels + C ABI) in-tree with hipcc.

Every HIP translation unit is compiled with FP contraction off and with packed
fp32 instructions disabled (-packed-fp32-ops); the kernels issue their FMAs
explicitly.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqwg.so")
SOURCES = ["qwg_api.cpp", "q4k.hip", "short.hip", "chain.hip", "iq3.hip", "codebook.hip", "encode.hip"]
ARCH = os.environ.get("QWG_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core results in ordinary VGPRs (no copies out of AGPRs)
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]


def build(verbose: bool = False) -> str:
    """Compile every translation unit (in parallel, one hipcc per source) and
    link libqwg.so in-tree; raises CalledProcessError on a compile error."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, "-x", "hip", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        jobs.append((cmd, obj))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(subprocess.check_call, cmd) for cmd, _ in jobs]:
            f.result()
    objs = [obj for _, obj in jobs]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
