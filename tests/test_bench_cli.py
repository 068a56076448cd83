"""bench.py on the CPU: more than one GPU is refused in every mode before
anything touches a device, the help text lists the modes, and the oracle
baseline leg runs on one thread and on all of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


@pytest.mark.parametrize("mode", [[], ["--workload", "llama8b_z3_clip"], ["--reshard", "llama8b_reshard"],
                                  ["--offload"], ["--host-step"]])
def test_more_than_one_gpu_is_refused(mode):
    res = subprocess.run([sys.executable, BENCH, "--gpus", "8", *mode], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2 and "one GPU only" in res.stderr, res.stderr
    assert res.stdout == ""


def test_help_lists_the_modes():
    res = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0
    for flag in ("--workload", "--reshard", "--offload", "--host-step", "--no-box-copy", "--copy-calibration"):
        assert flag in res.stdout


def test_fp32_gradient_variant_needs_no_cpu_leg():
    """The fp32-gradient variant has no oracle leg of its own: it must be
    asked for without one (refused before any device work)."""
    res = subprocess.run([sys.executable, BENCH, "--grad-dtype", "f32"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode != 0 and "--no-cpu-baseline" in res.stderr, res.stderr
    assert res.stdout == ""


def test_cpu_baseline_one_thread_and_all_cores():
    """The oracle leg of bench.py on CPU: one thread, then every available
    thread on its own copy of the sample; the clipped workload's sample runs
    the norm pass too."""
    sys.path.insert(0, ROOT)
    import bench
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS

    for name in ("llama8b_z3_clip", "llama8b_z3"):
        res = bench.cpu_baseline(WORKLOADS[name], 0.3)
        assert res["kind"] == "oracle" and res["cores"] == 1 and res["value"] > 0
        assert ("norm passes" in res["sample"]) == (name == "llama8b_z3_clip")
        avail = len(os.sched_getaffinity(0))
        if avail > 1:
            allc = res["all_cores"]
            assert allc["cores"] == min(16, avail) and allc["value"] > 0
        else:
            assert "all_cores" not in res


def test_stagger_plan_reproduces_the_arena_plan():
    """bench.py --stagger-kib 256 places the buffers exactly as the library's
    zero_arena_plan (which --stagger-kib sweeps around)."""
    import numpy as np
    z = pytest.importorskip("fsdp_sharded_optimizer_flat_amd")
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench
    rng = np.random.default_rng(4)
    for _ in range(50):
        sizes = [int(x) for x in rng.integers(0, 40 << 20, int(rng.integers(1, 70)))]
        offs, total = bench.stagger_plan(sizes, 256 << 10, alias_fix=True)
        lib_offs, lib_total = z.zero_arena_plan(sizes)
        assert list(offs) == list(lib_offs) and total == lib_total
        offs, total = bench.stagger_plan(sizes, 0)
        assert all(o % (2 << 20) == 0 for o in offs) and total == offs[-1] + sizes[-1]
    # runs of equal sizes (gradient buffers of the 8B model's shard at N ranks):
    # more than 32 whose stagger leaves them 32 MiB apart modulo 64 MiB (plus
    # whole pages and the stagger) start one 2 MiB page later; shorter runs
    # and other spacings are the plain stagger
    page, mib = 2 << 20, 1 << 20
    for n, size, moved in ((160, 100_378_268, True), (96, 167_297_110, True),
                           (64, 501_891_328, True), (32, 501_891_328, False),
                           (64, 250_945_664, False), (256, 62_736_416, False)):
        sizes = [size] * n + [size * 2] * 3 + [size // 2]
        offs, total = bench.stagger_plan(sizes, 256 << 10, alias_fix=True)
        lib_offs, lib_total = z.zero_arena_plan(sizes)
        assert list(offs) == list(lib_offs) and total == lib_total
        plain, _ = bench.stagger_plan(sizes, 256 << 10)
        assert (list(offs) != list(plain)) == moved, (n, size)
        def spacings(o):
            return {((o[i] - o[i - 1]) // page * page) % (64 * mib) for i in range(1, n)}
        assert (n > 32 and 32 * mib in spacings(plain)) == moved, (n, size, spacings(plain))
        assert 32 * mib not in spacings(offs) or n <= 32, (n, size, spacings(offs))
        assert all(o % page == (i * (256 << 10)) % page for i, o in enumerate(offs))
