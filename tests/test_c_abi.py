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


@pytest.mark.gpu
def test_c_program_on_the_gpu():
    """tests/c/gpu_step_check.c (built by __graft_entry__.build()): the step,
    the norm, the clipped step with no host synchronization and the staged
    step at 40 ranks driven from plain C with HIP's C runtime API, checked
    against the oracle's C library, with no Python in the process."""
    import torch
    if torch.cuda.device_count() == 0:
        pytest.skip("needs a GPU")
    exe = os.path.join(ROOT, "tests", "c", "gpu_step_check.bin")
    if not os.path.exists(exe):
        pytest.fail(f"{exe} is missing: run __graft_entry__.build()")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
