"""Build libpsk_fused.so in-tree (hipcc for the gfx950 kernels, g++ for host code).

    python -m elementwise_reduction_groups_amd.build

Device code is compiled for gfx950 with -ffp-contract=off, correctly rounded
f32 division and square root, no denormal flush and packed-FP32 instructions
disabled; emitted kernels get the same flags through hipRTC at run time.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpsk_fused.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HOST_SOURCES = ["api.cpp", "validate.cpp", "plan.cpp", "emit.cpp", "jit.cpp", "partition.cpp"]
HIP_SOURCES = ["adamw.hip"]

DEVICE_FLAGS = ["--offload-arch=gfx950", "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                "-fno-gpu-flush-denormals-to-zero", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HOST_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append(["g++", *COMMON, "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", "-c",
                     os.path.join(CSRC, s), "-o", obj])
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD, s + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, s), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [os.path.join(BUILD, s + ".o") for s in HOST_SOURCES + HIP_SOURCES]
    tmp = LIB + f".tmp{os.getpid()}"
    _run([HIPCC, "-shared", "-fPIC", "-o", tmp, *objs, f"-L{ROCM}/lib", "-lamdhip64", "-lhiprtc",
          f"-Wl,-rpath,{ROCM}/lib"])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
