"""The boundary from plain C: compile tests/c/abi_host_check.c with gcc
against include/zero.h, link libzero.so, run it (host-only calls; no GPU)."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "fsdp_sharded_optimizer_flat_amd")


def test_c_program_against_header(tmp_path):
    if not os.path.exists(os.path.join(LIBDIR, "libzero.so")):
        pytest.skip("libzero.so not built")
    exe = tmp_path / "abi_host_check"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-o", str(exe),
                    "-L", LIBDIR, "-lzero", f"-Wl,-rpath,{LIBDIR}", "-lm"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
