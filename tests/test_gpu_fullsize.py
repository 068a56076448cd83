"""Full workload sizes, in the launch configuration the benchmark times.
The GPT-2-Large-sized model (774M elements, N = 8) and the 8B Llama shard
(125M elements, N = 64) are compared with the oracle element by element over
two steps, and so is the clipped workload (the norm pass's reduced gradient,
its sum of squares and coefficient, and the clipped step, through the
benchmark's sync-free chain).  A step of 2^32 + 17 elements (more than one
dispatch) is checked on sampled elements the oracle recomputes one by one,
which is exact because the step is elementwise; so is the staged step on a
shard past 2^31 elements, whose norm pass is compared on every element."""
import concurrent.futures as cf
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd import synth  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS  # noqa: E402
from gpu_common import (DEV, assert_same_bf16, assert_same_f32, gather_np,  # noqa: E402
                        hyper_args, oracle_on_samples, scalars, to_np)

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _run_full(name, steps=2, staged=False):
    """Every element of the workload after `steps` steps, against the oracle.
    The oracle runs unit by unit on the unit's slices of the host copies, in
    a thread pool: a unit's elements map only to its own range in every index
    space, so this is exactly the oracle's step of the whole layout."""
    wl = WORKLOADS[name]
    n, h = wl.n_ranks, wl.hyper
    L = z.zero_pack(n, wl.unit_numel)
    all_ranks = wl.rank < 0
    idx = G if all_ranks else Lc
    assert (wl.grad_index == "global") == all_ranks and (wl.out_index == "global") == all_ranks
    E = L.padded if all_ranks else L.shard
    log(f"{name} full compare: N={n}, {E} elements, {steps} steps")
    master = torch.empty(E, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(E, dtype=torch.int16, device=DEV)
    grads = torch.empty(n, E, dtype=torch.bfloat16, device=DEV)
    wh, mh, vh = to_np(master).copy(), np.zeros(E, np.float32), np.zeros(E, np.float32)
    oh = np.zeros(E, np.uint16)
    units = [(int(nu), int(off if all_ranks else loff), int(pad if all_ranks else sh))
             for nu, pad, sh, off, loff in L.unit_table()]
    ha = hyper_args(h)

    def oracle_unit(u, gh, t):
        numel, a, ln = u
        gs = [g[a:a + ln] for g in gh]
        st = dict(master=wh[a:a + ln], m=mh[a:a + ln], v=vh[a:a + ln], t=t, **ha)
        if all_ranks:
            oracle.zero_step_all(n, [numel], gs, divisor=float(n), clip=1.0, out=oh[a:a + ln], **st)
        else:
            oracle.zero_step_rank(n, [numel], wl.rank, gs, grad_local=True, divisor=float(n),
                                  clip=1.0, state_global=False, out=oh[a:a + ln],
                                  out_gather=False, **st)

    workers = min(16, os.cpu_count() or 1)
    ws = None
    if staged:  # the launch configuration bench.py times at this N
        ws = torch.empty(z.zero_step_staged_workspace_bytes(L, wl.rank, n) // 4, dtype=torch.float32,
                         device=DEV)
    for t in range(1, steps + 1):
        for r in range(n):
            synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, t, r))
        if staged:
            z.zero_step_staged(L, wl.rank, list(grads), idx, float(n), master, m, v, idx, out, idx,
                               scalars(t, h), ws)
        else:
            z.zero_step(L, wl.rank, list(grads), idx, float(n), master, m, v, idx, out, idx, scalars(t, h))
        gh = [to_np(grads[r]) for r in range(n)]
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda u: oracle_unit(u, gh, t), units))
        del gh
        log(f"{name}: step {t} done on the GPU and in the oracle")
    torch.cuda.synchronize()
    assert_same_f32(to_np(master), wh, f"{name} master")
    assert_same_f32(to_np(m), mh, f"{name} m")
    assert_same_f32(to_np(v), vh, f"{name} v")
    assert_same_bf16(to_np(out), oh, f"{name} out")
    log(f"{name}: all {E} elements bit-exact after {steps} steps (staged={staged})")


def test_gpt2l_full_size_every_element():
    _run_full("gpt2l")


def test_llama8b_z3_shard_full_size_every_element():
    _run_full("llama8b_z3")


def test_llama8b_z3_shard_staged_full_size_every_element():
    _run_full("llama8b_z3", staged=True)


def test_llama8b_z3_clip_full_size_every_element():
    """The clipped workload at full size (N = 64, the 125,472,832-element
    shard, Student-t(3) x 1e-3 gradients), two steps of the benchmark's
    sync-free chain -- zero_gradnorm_async (writing the reduced gradient g) ->
    zero_clip_coef_async -> zero_step_device_clip on g -- against the oracle
    on every element: g bit for bit against orc_reduced_grad; the device's
    binary64 sum of squares within n 2^-53 of the oracle's serial sum over its
    own g (that sum's error bound) and within 1e-12 of a pairwise binary64 sum;
    the device coefficient equal to the oracle's; master, m, v and the bf16
    shard bit for bit against the oracle's clipped step on the 64 gradients
    with the oracle's own coefficient."""
    wl = WORKLOADS["llama8b_z3_clip"]
    n, h, rank = wl.n_ranks, wl.hyper, wl.rank
    L = z.zero_pack(n, wl.unit_numel)
    E = L.shard
    log(f"clip full compare: N={n}, S={E}")
    master = torch.empty(E, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(E, dtype=torch.int16, device=DEV)
    grads = torch.empty(n, E, dtype=torch.bfloat16, device=DEV)
    g_out = torch.empty(E, dtype=torch.float32, device=DEV)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
    sumsq = torch.zeros(1, dtype=torch.float64, device=DEV)
    coef = torch.zeros(1, dtype=torch.float32, device=DEV)
    wh, mh, vh = to_np(master).copy(), np.zeros(E, np.float32), np.zeros(E, np.float32)
    oh = np.zeros(E, np.uint16)
    og = np.zeros(E, np.float32)
    units = [(int(nu), int(loff), int(sh)) for nu, pad, sh, off, loff in L.unit_table()]
    ha = hyper_args(h)
    workers = min(16, os.cpu_count() or 1)
    for t in range(1, 3):
        for r in range(n):
            synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, t, r))
        z.zero_gradnorm_async(L, rank, list(grads), Lc, float(n), g_out, Lc, ws, sumsq)
        z.zero_clip_coef_async(sumsq, wl.clip_max_norm, coef)
        z.zero_step_device_clip(L, rank, [g_out], Lc, 1.0, master, m, v, Lc, out, Lc, scalars(t, h), coef)
        torch.cuda.synchronize()
        dev_sum, dev_coef = float(sumsq.item()), float(coef.item())
        gh = [to_np(grads[r]) for r in range(n)]

        def reduce_unit(u):
            numel, a, ln = u
            og[a:a + ln] = oracle.reduced_grad(n, [numel], rank, [g[a:a + ln] for g in gh],
                                               grad_local=True, divisor=float(n))
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(reduce_unit, units))
        assert_same_f32(to_np(g_out), og, f"step {t}: reduced gradient")
        orc_sum = oracle.sumsq(og)
        pair = float(np.sum(og.astype(np.float64) ** 2))
        assert abs(dev_sum - orc_sum) <= E * 2.0 ** -53 * orc_sum, (dev_sum, orc_sum)
        assert abs(dev_sum - pair) <= 1e-12 * pair, (dev_sum, pair)
        orc_coef = oracle.clip_coef(orc_sum, wl.clip_max_norm)
        assert dev_coef == orc_coef, (dev_coef, orc_coef)
        assert 0.0 < orc_coef < 1.0, "Student-t(3) x 1e-3 gradients over 125M elements must clip"
        log(f"step {t}: sumsq device {dev_sum:.9e} oracle {orc_sum:.9e}, coef {orc_coef:.7f}")

        def step_unit(u):
            numel, a, ln = u
            oracle.zero_step_rank(n, [numel], rank, [g[a:a + ln] for g in gh], grad_local=True,
                                  divisor=float(n), clip=orc_coef, master=wh[a:a + ln], m=mh[a:a + ln],
                                  v=vh[a:a + ln], state_global=False, out=oh[a:a + ln],
                                  out_gather=False, t=t, **ha)
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(step_unit, units))
        del gh
        # the norm is reproducible and independent of writing g
        z.zero_gradnorm_async(L, rank, list(grads), Lc, float(n), None, Lc, ws, sumsq)
        torch.cuda.synchronize()
        assert float(sumsq.item()) == dev_sum
        log(f"clip: step {t} done on the GPU and in the oracle")
    assert_same_f32(to_np(master), wh, "clip master")
    assert_same_f32(to_np(m), mh, "clip m")
    assert_same_f32(to_np(v), vh, "clip v")
    assert_same_bf16(to_np(out), oh, "clip out")
    log(f"clip: all {E} elements bit-exact after 2 steps")


def test_step_beyond_one_launch():
    """2^32 + 17 elements at N = 1: more quads than one dispatch addresses
    (2^30), so the step runs as two vector launches plus a scalar tail.  The
    oracle checks elements around both launch boundaries and random ones."""
    n, P = 1, (1 << 32) + 17
    h = WORKLOADS["gpt2l"].hyper
    L = z.zero_pack(n, [P])
    log(f"max-size: P={P} ({P * 18 / 1e9:.1f} GB of device buffers)")
    g = torch.empty(P, dtype=torch.bfloat16, device=DEV)
    synth.fill_normal_(g, 1e-3, 99)
    master = torch.empty(P, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, 0.02, 98)
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(P, dtype=torch.int16, device=DEV)
    rng = np.random.default_rng(5)
    edge = (1 << 30) * 4                   # first element of the second launch
    picks = set(int(x) for x in rng.integers(0, P, 4096))
    picks.update(range(0, 8))
    picks.update(range(edge - 8, edge + 8))
    picks.update(range(P - 24, P))
    idx = np.array(sorted(picks), np.int64)
    idx_t = torch.from_numpy(idx).to(DEV)
    master0 = gather_np(master, idx_t)
    gs = [[gather_np(g, idx_t)]]
    z.zero_step(L, -1, [g], G, 1.0, master, m, v, G, out, G, scalars(1, h))
    torch.cuda.synchronize()
    w, mm, vv, oo = oracle_on_samples(1, gs, master0, 1, h, divisor=1.0)
    assert_same_f32(gather_np(master, idx_t), w, "max-size master")
    assert_same_f32(gather_np(v, idx_t), vv, "max-size v")
    assert_same_bf16(gather_np(out, idx_t), oo, "max-size out")
    del g, master, m, v, out


def test_norm_and_staged_step_past_2_31_elements():
    """One rank's shard of 2^31 + 3 * 2^20 + 17 elements (element indices past
    int32, byte offsets past 2^33, a ragged last tile) under 33 gradients that
    alternate between two buffers.  The norm pass: its reduced gradient on
    every element bit for bit against orc_reduced_grad (in chunks, on host
    threads) and its binary64 sum of squares within n 2^-53 of the oracle's
    (the chunks' sums added in order) and within 1e-12 of a pairwise binary64
    sum of the oracle's gradient.  The staged step (many workspace
    chunks): two steps on sampled elements around 2^31, the chunk boundaries
    and the tail, recomputed by the oracle one by one."""
    n, E = 33, (1 << 31) + 3 * (1 << 20) + 17
    h = WORKLOADS["llama8b_z3"].hyper
    L = z.zero_pack(n, [E * n])
    assert L.shard == E
    log(f"past 2^31: N={n}, S={E}")
    g0 = torch.empty(E, dtype=torch.bfloat16, device=DEV)
    g1 = torch.empty(E, dtype=torch.bfloat16, device=DEV)
    synth.fill_normal_(g0, 1e-3, 71)
    synth.fill_normal_(g1, 3e-3, 72)
    grads = [g0 if q % 2 == 0 else g1 for q in range(n)]

    # the norm pass
    g_out = torch.empty(E, dtype=torch.float32, device=DEV)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, 0) // 8, dtype=torch.float64, device=DEV)
    sumsq = torch.zeros(1, dtype=torch.float64, device=DEV)
    z.zero_gradnorm_async(L, 0, grads, Lc, float(n), g_out, Lc, ws, sumsq)
    torch.cuda.synchronize()
    dev_sum = float(sumsq.item())
    del ws
    h0, h1, gh = to_np(g0), to_np(g1), to_np(g_out)
    del g_out
    log("past 2^31: norm pass done, host copies taken")
    CH = 1 << 26
    bounds = [(a, min(a + CH, E)) for a in range(0, E, CH)]

    def chunk(b):
        a, e = b
        gs = [h0[a:e] if q % 2 == 0 else h1[a:e] for q in range(n)]
        og = oracle.reduced_grad(n, [(e - a) * n], 0, gs, grad_local=True, divisor=float(n))
        same = bool(np.array_equal(og.view(np.uint32), gh[a:e].view(np.uint32)))
        return same, oracle.sumsq(og), float(np.sum(og.astype(np.float64) ** 2))

    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        res = list(ex.map(chunk, bounds))
    bad = [b for b, (same, _, _) in zip(bounds, res) if not same]
    assert not bad, f"reduced gradient differs from the oracle in chunks {bad[:4]}"
    orc_sum = pair = 0.0
    for _, s, p in res:
        orc_sum += s
        pair += p
    assert abs(dev_sum - orc_sum) <= E * 2.0 ** -53 * orc_sum, (dev_sum, orc_sum)
    assert abs(dev_sum - pair) <= 1e-12 * pair, (dev_sum, pair)
    log(f"past 2^31: g bit-exact on all {E} elements; sumsq device {dev_sum:.12e} oracle {orc_sum:.12e} "
        f"pairwise {pair:.12e}")
    del gh

    # the staged step, two steps on the same gradients
    master = torch.empty(E, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, 0.02, 73)
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(E, dtype=torch.int16, device=DEV)
    wsb = z.zero_step_staged_workspace_bytes(L, 0, n)
    stage_ws = torch.empty(wsb // 4, dtype=torch.float32, device=DEV)
    chunk_elems = wsb // 4 - 4
    rng = np.random.default_rng(6)
    picks = set(int(x) for x in rng.integers(0, E, 4096))
    picks.update(range(0, 8))
    picks.update(range((1 << 31) - 8, (1 << 31) + 8))
    for k in (1, 2, E // chunk_elems):
        picks.update(x for x in range(k * chunk_elems - 8, k * chunk_elems + 8) if 0 <= x < E)
    picks.update(range(E - 24, E))
    idx = np.array(sorted(picks), np.int64)
    idx_t = torch.from_numpy(idx).to(DEV)
    master0 = gather_np(master, idx_t)
    s0, s1 = h0[idx], h1[idx]
    gs = [s0 if q % 2 == 0 else s1 for q in range(n)]
    del h0, h1
    for t in (1, 2):
        z.zero_step_staged(L, 0, grads, Lc, float(n), master, m, v, Lc, out, Lc, scalars(t, h), stage_ws)
    torch.cuda.synchronize()
    w, mm, vv, oo = oracle_on_samples(n, [gs, gs], master0, 2, h, divisor=float(n))
    assert_same_f32(gather_np(master, idx_t), w, "past 2^31 staged master")
    assert_same_f32(gather_np(m, idx_t), mm, "past 2^31 staged m")
    assert_same_f32(gather_np(v, idx_t), vv, "past 2^31 staged v")
    assert_same_bf16(gather_np(out, idx_t), oo, "past 2^31 staged out")
    log(f"past 2^31: staged step bit-exact on {idx.size} sampled elements after 2 steps "
        f"({-(-E // chunk_elems)} chunks of {chunk_elems})")
