"""Build libfp8z1.so (HIP kernels for gfx950 + host C++) in-tree.

    python blockwise_fp8_zero_fold_amd/build.py

(run as a script: importing the package loads the library, which a fresh
checkout does not have yet).

Objects go to <repo>/_build/, the library next to this file.  Every call
compiles from scratch.
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
OUT = os.path.join(PKG, "libfp8z1.so")
OBJ = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", shutil.which("g++") or "g++")

# Device code: no fused multiply-add contraction (every float32 operation of the
# update is one IEEE rounding), correctly rounded division and square root
# (hipcc's default), and no packed-FP32 instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]
CXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def sources():
    hip = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    cpp = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".cpp"))
    return hip, cpp


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    hip, cpp = sources()
    jobs = []
    for src in hip:
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        jobs.append([HIPCC, *HIP_FLAGS, "-c", src, "-o", obj])
    for src in cpp:
        obj = os.path.join(OBJ, os.path.basename(src) + ".o")
        jobs.append([CXX, *CXX_FLAGS, "-c", src, "-o", obj])
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [j[-1] for j in jobs]
    tmp = OUT + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, OUT)
    # a C-ABI consumer without Python or torch, used by the GPU tests
    example = os.path.join(ROOT, "tests", "native", "abi_c_step.cpp")
    if os.path.exists(example):
        exe = os.path.join(ROOT, "tests", "native", "abi_c_step")
        _run([HIPCC, "-O2", "-std=c++17", example, "-L" + PKG, "-lfp8z1",
              "-Wl,-rpath,$ORIGIN/../../blockwise_fp8_zero_fold_amd", "-o", exe + ".tmp"])
        os.replace(exe + ".tmp", exe)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
