"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).  A copy of libzero.so is built from the same sources and flags as
the real one, with the sanitizers on its host code (each flag behind
-Xarch_host: the device code is built exactly as usual and never runs here),
and tests/c/host_sanitize_check.c drives every host-only entry point, the host
step and the host reshard against the oracle's C library, and the validation
paths of the device entry points.  The sanitizer runtime comes from the
driver, which ROCm's clang links with the same -Xarch_host flags."""
import concurrent.futures as cf
import importlib.util
import os
import shutil
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _builder():
    path = os.path.join(ROOT, "fsdp_sharded_optimizer_flat_amd", "_build.py")
    spec = importlib.util.spec_from_file_location("zero_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _clang(name):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    p = os.path.join(rocm, "llvm", "bin", name)
    return p if os.path.exists(p) else shutil.which(name)


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stderr[-3000:]


def test_host_code_under_asan_and_ubsan(tmp_path):
    b = _builder()
    clang, clangxx = _clang("clang"), _clang("clang++")
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")) or not clang or not clangxx:
        pytest.skip("needs hipcc and ROCm's clang")
    flags = [f for f in b.FLAGS if f != "-O3"] + ["-O1", "-g"]
    host_flags = [f for f in b.HOST_FLAGS if f != "-O3"] + ["-O1", "-g"]

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        path = os.path.join(b.CSRC, src)
        if src in b.HOST_SOURCES:
            _run([clangxx, *host_flags, *SAN, f"-I{b.INCLUDE}", f"-I{b.CSRC}", "-c", path, "-o", obj])
        else:
            _run([b.hipcc(), *flags, *SAN, "-c", path, "-o", obj])
        return obj

    srcs = b.SOURCES + b.HOST_SOURCES
    with cf.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4, 8)) as ex:
        objs = list(ex.map(compile_one, srcs))
    lib = str(tmp_path / "libzero_san.so")
    _run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-pthread", *objs, "-o", lib])

    oracle.load()  # builds oracle/liboracle.so when it is missing or stale
    orc_dir = os.path.dirname(oracle.LIB)
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    exe = str(tmp_path / "host_sanitize_check")
    _run([clang, "-std=c11", "-O1", "-g", "-Wall", "-Werror", *SAN, f"-I{b.INCLUDE}",
          os.path.join(ROOT, "tests", "c", "host_sanitize_check.c"), "-o", exe,
          f"-L{tmp_path}", "-lzero_san", f"-L{orc_dir}", "-loracle",
          f"-Wl,-rpath,{tmp_path}:{orc_dir}:{rocm_lib}", "-lm"])
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout[-2000:] + res.stderr[-4000:]
