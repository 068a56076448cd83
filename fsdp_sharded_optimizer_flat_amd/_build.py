"""Build libzero.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python fsdp_sharded_optimizer_flat_amd/_build.py

(run as a file: importing it through the package would load the library it
is about to rebuild).

Floating-point flags are part of the contract: -ffp-contract=off (no FMA
contraction), IEEE binary32 denormals (-fno-gpu-flush-denormals-to-zero),
correctly rounded division and square root, and no packed-fp32 instructions.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libzero.so")

SOURCES = ["layout.cpp", "scalars.cpp", "ledger.cpp", "capi.cpp", "caps.cpp", "offload.cpp", "reshard.cpp",
           "step_kernels.hip", "norm_kernels.hip", "stage_kernels.hip", "pack_kernels.hip",
           "reshard_kernels.hip"]
# Host-only C++ built with g++: the offload step's AVX2 code (no FMA, no
# fast-math, so every operation rounds once, as on the GPU) and the
# checkpoint files (the SSE4.2 crc32 instruction, which -mavx2 includes).
HOST_SOURCES = ["host_step.cpp", "checkpoint.cpp"]
HOST_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-mavx2", "-mno-fma", "-ffp-contract=off",
              "-fno-fast-math", "-pthread", "-Wall"]

# Test support built with the same flags: bare sqrt / division kernels the GPU
# tests check exhaustively against the host's IEEE operations.
PROBE_SRC = os.path.join(ROOT, "tests", "support", "fp_probe.hip")
PROBE_LIB = os.path.join(ROOT, "tests", "support", "libfp_probe.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found; the library needs ROCm's hipcc to build")
    return p


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src + ".o")
    if src in HOST_SOURCES:
        cmd = ["g++", *HOST_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, src),
               "-o", obj]
    else:
        cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr}")
    return obj


def build(jobs: int | None = None) -> str:
    """Compile every source and link libzero.so next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + HOST_SOURCES
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    build_probe()
    return LIB


def build_probe() -> str:
    """The test-support probe library (tests/support/libfp_probe.so)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc(), *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def device_ir(src: str = "step_kernels.hip") -> str:
    """Device LLVM IR of one source, for the flag checks in the tests."""
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, src + ".ll")
    cmd = [hipcc(), *FLAGS, "--cuda-device-only", "-S", "-emit-llvm",
           os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


def device_asm(src: str = "step_kernels.hip") -> str:
    """gfx950 assembly of one source (resource usage, instruction checks)."""
    os.makedirs(BUILD, exist_ok=True)
    out = os.path.join(BUILD, src + ".s")
    cmd = [hipcc(), *FLAGS, "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    with open(out) as f:
        return f.read()


if __name__ == "__main__":
    print(build())
    sys.exit(0)
