"""The benchmark's own path against the oracle.  bench.setup_step builds the
inputs exactly as bench.py times them -- one allocation placed by
zero_arena_plan, gradient pointers marshalled once, the staged step with its
workspace above 32 ranks, the device-side norm -> coefficient -> step chain
for the clipped workload -- and two steps run through its one_step.  Sampled
elements (random positions plus the first, middle and last element of every
unit) are then compared with the oracle, which recomputes them one by one;
for the clipped workload the sum of squares of the reduced gradient the norm
pass wrote is compared with an accurate binary64 sum (and the oracle's serial
sum with its error bound), and the coefficient with the oracle's."""
import os
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS  # noqa: E402
from gpu_common import (DEV, assert_same_bf16, assert_same_f32, gather_np,  # noqa: E402
                        oracle_on_samples, sampled_indices, to_np)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["gpt2l", "llama8b_z3", "llama8b_z3_clip"])
def test_bench_path_matches_oracle(name):
    S = bench.setup_step(WORKLOADS[name])
    log(f"{name}: N={S.n}, staged={S.staged}, clip={S.clip}, {S.se} elements")
    assert S.staged == (name == "llama8b_z3")
    # identity index maps: every rank's shards GLOBAL, or one rank all LOCAL
    assert S.gidx == S.sidx == S.oidx
    assert (S.sidx == z.ZERO_LOCAL) == (S.wl.rank >= 0)
    rng = np.random.default_rng(11)
    idx = sampled_indices(S.se, S.L.unit_table(), S.sidx, rng, k=8192)
    idx_t = torch.from_numpy(idx).to(DEV)
    master0 = gather_np(S.master, idx_t)
    gs = [np.ascontiguousarray(gather_np(g, idx_t)) for g in S.grads]  # the same every step
    clips = [] if S.clip else None
    for t in (1, 2):
        S.one_step(t)
        if S.clip:
            torch.cuda.synchronize()
            og = oracle.reduced_grad(S.n, [idx.size * S.n], 0, gs, grad_local=True,
                                     divisor=float(S.n))
            assert_same_f32(gather_np(S.g_red, idx_t), og, f"{name} reduced gradient, step {t}")
            # the sum of squares of the g the norm pass wrote: numpy's pairwise
            # binary64 sum (error ~ log2(n) ulps) is the accurate reference;
            # the oracle's serial binary64 sum is held to its own bound,
            # n * 2^-53 relative (1.4e-8 at 125M terms)
            gh = to_np(S.g_red).astype(np.float64)
            accurate = float(np.sum(gh * gh))
            serial = oracle.sumsq(to_np(S.g_red))
            del gh
            dev_total = float(S.ss_dev.item())
            assert abs(dev_total - accurate) <= 1e-12 * accurate, (dev_total, accurate)
            assert abs(serial - accurate) <= S.se * 2.0 ** -53 * accurate, (serial, accurate)
            coef = float(S.coef_dev.item())
            assert coef == np.float32(oracle.clip_coef(accurate, S.wl.clip_max_norm)), coef
            assert 0.0 < coef < 1.0
            clips.append(coef)
    torch.cuda.synchronize()
    w, mm, vv, oo = oracle_on_samples(S.n, [gs, gs], master0, 2, S.h, clips=clips)
    assert_same_f32(gather_np(S.master, idx_t), w, f"{name} master")
    assert_same_f32(gather_np(S.m, idx_t), mm, f"{name} m")
    assert_same_f32(gather_np(S.v, idx_t), vv, f"{name} v")
    assert_same_bf16(gather_np(S.out, idx_t), oo, f"{name} out")
    log(f"{name}: {idx.size} sampled elements bit-exact after 2 steps of the benchmark's path")
