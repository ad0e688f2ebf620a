"""Build libmoe.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage:  python sparsely_gated_mixture_amd/build.py
(run by path: importing the package loads the library this script builds).
Every call recompiles (objects go to _build/ at the repository root).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

HIP_SOURCES = ["gemm_f32.hip", "gemm_gate.hip", "gate.hip", "dispatch.hip", "ggemm_bf16.hip", "combine.hip",
               "fp8.hip", "backward.hip", "ggemm_bwd.hip", "ggemm_bwd_f32.hip", "probe.hip",
               "ggemm_big.hip", "static_ws.hip"]
HOST_SOURCES = ["api.cpp", "profile.cpp"]

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-I", CSRC, "-I", os.path.join(ROOT, "include")]
# Packed fp32 arithmetic stays off in every device compilation.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def _compile(args):
    src, obj, device = args
    cmd = [_hipcc()] + COMMON + (DEVICE if device else []) + ["-c", src, "-o", obj]
    if not device:
        cmd[1:1] = ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(_rocm(), "include")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{out}")
    return out


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    work = []
    for s in HIP_SOURCES:
        work.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o"), True))
    for s in HOST_SOURCES:
        work.append((os.path.join(CSRC, s), os.path.join(BUILD, s + ".o"), False))
    jobs = jobs or min(len(work), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_compile, work):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + \
          [w[1] for w in work]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
