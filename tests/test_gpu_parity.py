"""GPU parity: the HIP step and norm, called through the C ABI, against the
oracle, element by element.  Floating-point state (master, m, v) and the bf16
output must match bit for bit (NaN compared as NaN-ness); the binary64 sum of
squares must match to a relative 1e-12 (its summation order differs).

Sizes: small enough for the oracle to finish in seconds yet spanning many
workgroup tiles and ragged tails, plus the full workload sizes with sampled
elements the oracle computes one by one."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd import synth  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS, GPT_HYPER, TOY_HYPER  # noqa: E402
from gpu_common import (DEV, assert_same_bf16, assert_same_f32, dev_buffer,  # noqa: E402
                        dev_buffer_guarded, extent, gather_np, hyper_args, oracle_on_samples,
                        sampled_indices, scalars, to_np)

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL


def log(msg):
    print(msg, flush=True)


def test_one_hip_runtime():
    """The library and torch share one HIP runtime in the process."""
    torch.zeros(1, device=DEV)
    maps = z.hip_runtimes_mapped()
    assert len(maps) == 1, maps


# ---------------------------------------------------------------------------
# The pages' toy, 50 steps, bit-exact (fp32 gradients w - t_r).
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,P", [(4, 1000), (4, 1001), (3, 1000), (8, 13)])
def test_toy_bitexact(n, P):
    log(f"toy n={n} P={P}")
    h = TOY_HYPER
    L = z.zero_pack(n, [P])
    Ph = L.padded
    tgt = torch.tensor([[(i * 7 + r * 13) % 11 for i in range(P)] for r in range(n)],
                       dtype=torch.float32, device=DEV)
    w = torch.zeros(Ph, dtype=torch.float32, device=DEV)
    m = torch.zeros_like(w)
    v = torch.zeros_like(w)
    out = torch.zeros(Ph, dtype=torch.int16, device=DEV)
    grads = [torch.zeros(Ph, dtype=torch.float32, device=DEV) for _ in range(n)]
    steps = 50
    for t in range(1, steps + 1):
        for r in range(n):
            torch.sub(w[:P], tgt[r], out=grads[r][:P])   # rank r's local gradient; padding stays 0
        z.zero_step(L, -1, grads, G, float(n), w, m, v, G, out, G, scalars(t, h))
    torch.cuda.synchronize()
    ws, wu, ob, _ = oracle.toy(n, P, steps, h["lr"])
    assert_same_f32(to_np(w)[:P], ws, "toy master vs oracle")
    assert_same_f32(to_np(w)[:P], wu, "toy master vs unsharded AdamW")
    assert_same_bf16(to_np(out)[:P], ob, "toy bf16 out")
    assert np.all(to_np(w)[P:].view(np.uint32) == 0), "padding must stay +0"


# ---------------------------------------------------------------------------
# One GPT-2 Large block, N = 8, all shards, 10 steps: full comparison.
# ---------------------------------------------------------------------------

def test_gpt2l_block_full_10_steps():
    wl = WORKLOADS["gpt2l_block"]
    log(f"gpt2l_block P={sum(wl.unit_numel)}")
    n, h = wl.n_ranks, wl.hyper
    L = z.zero_pack(n, wl.unit_numel)
    Ph = L.padded
    master = torch.empty(Ph, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(Ph, dtype=torch.int16, device=DEV)
    grads = torch.empty(n, Ph, dtype=torch.bfloat16, device=DEV)
    om = to_np(master).copy()
    omm, ov = np.zeros_like(om), np.zeros_like(om)
    oout = np.zeros(Ph, np.uint16)
    for t in range(1, wl.steps + 1):
        for r in range(n):
            synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, t, r))
        z.zero_step(L, -1, list(grads), G, float(n), master, m, v, G, out, G, scalars(t, h))
        gnp = [np.ascontiguousarray(to_np(grads[r])) for r in range(n)]
        oracle.zero_step_all(n, list(wl.unit_numel), gnp, divisor=float(n), clip=1.0, master=om,
                             m=omm, v=ov, out=oout, t=t, **hyper_args(h))
    torch.cuda.synchronize()
    assert_same_f32(to_np(master), om, "master")
    assert_same_f32(to_np(m), omm, "m")
    assert_same_f32(to_np(v), ov, "v")
    assert_same_bf16(to_np(out), oout, "bf16 out")


# ---------------------------------------------------------------------------
# Every index mode, rank, dtype, rank count and pointer alignment on tiny
# layouts (brute force), against the oracle's rank step.
# ---------------------------------------------------------------------------

def _order_sensitive(gnp, gdt):
    """True if summing the ranks' values in reverse order gives other binary32
    bits than in rank order for some element (numpy, test-side check only)."""
    vals = [g.astype(np.uint32) << 16 if gdt == z.ZERO_BF16 else g for g in gnp]
    vals = [np.asarray(x).view(np.float32) for x in vals]
    fwd, rev = vals[0].copy(), vals[-1].copy()
    for x in vals[1:]:
        fwd = fwd + x
    for x in vals[-2::-1]:
        rev = rev + x
    return bool(np.any(fwd.view(np.uint32) != rev.view(np.uint32)))


def _run_case(rng, n, numel, rank, gdt, gidx, sidx, oidx, shift, steps=2, with_out=True, n_grads=None,
              dist="normal", check_order=False, staged=None):
    """staged: None for zero_step; otherwise zero_step_staged with a
    workspace of that many fp32 elements (0: the size the library asks for),
    followed by sentinels the call must leave untouched."""
    h = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    L = z.zero_pack(n, numel)
    O = oracle.Layout(n, numel)
    ng = n if n_grads is None else n_grads
    tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
    ge, se, oe = extent(L, gidx), extent(L, sidx), extent(L, oidx)
    grads = [dev_buffer(ge, tdt, shift=(shift * (q + 1)) % 8) for q in range(ng)]
    # the written buffers carry sentinels before and after them
    master, cw = dev_buffer_guarded(se, torch.float32, shift=shift)
    m, cm = dev_buffer_guarded(se, torch.float32, shift=shift)
    v, cv = dev_buffer_guarded(se, torch.float32, shift=shift)
    out, co = dev_buffer_guarded(oe, torch.int16, shift=(shift * 3) % 8) if with_out else (None, None)
    init = rng.normal(0, 0.02, se).astype(np.float32)
    master.copy_(torch.from_numpy(init))
    om, omm, ov = init.copy(), np.zeros(se, np.float32), np.zeros(se, np.float32)
    oout = np.zeros(oe, np.uint16)
    ws = ws_guard = None
    if staged is not None:
        want = z.zero_step_staged_workspace_bytes(L, rank, ng) // 4
        elems = want if staged == 0 else staged
        if want:   # a guard of 64 sentinels past the workspace, which the call must not touch
            ws_full = torch.full((max(elems, 1) + 64,), -99.0, dtype=torch.float32, device=DEV)
            ws, ws_guard = ws_full[:max(elems, 1)], ws_full[max(elems, 1):]
    for t in range(1, steps + 1):
        for g in grads:
            vals = rng.standard_normal(ge) * 1e-3
            if dist == "wide":   # magnitudes over 48 binades: rank sums round often
                vals = vals * np.exp2(rng.integers(-24, 25, ge))
            g.copy_(torch.from_numpy(vals.astype(np.float32)).to(tdt))
        gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
        if check_order:   # (with 1 or 2 ranks no order can show: a + b == b + a)
            assert _order_sensitive(gnp, gdt), "test data cannot see the rank order"
        if staged is None:
            z.zero_step(L, rank, grads, gidx, float(n), master, m, v, sidx, out, oidx, scalars(t, h))
        else:
            z.zero_step_staged(L, rank, grads, gidx, float(n), master, m, v, sidx, out, oidx,
                               scalars(t, h), ws)
        if rank < 0:
            oracle.zero_step_all(n, numel, gnp, divisor=float(n), clip=1.0, master=om, m=omm, v=ov,
                                 out=oout if with_out else None, t=t, **hyper_args(h))
        else:
            oracle.zero_step_rank(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n),
                                  clip=1.0, master=om, m=omm, v=ov, state_global=(sidx == G),
                                  out=oout if with_out else None, out_gather=(oidx == G), t=t,
                                  **hyper_args(h))
    torch.cuda.synchronize()
    tag = f"n={n} numel={numel} rank={rank} gdt={gdt} idx={gidx}{sidx}{oidx} shift={shift} staged={staged}"
    if ws_guard is not None:
        assert bool((ws_guard == -99.0).all()), f"{tag}: the staged step wrote past its workspace"
    # compare only the elements the selection owns (others stay as initialised)
    if rank < 0:
        sel_s = np.arange(se)
        sel_o = np.arange(oe)
    else:
        ks = np.arange(L.shard)
        js = np.array([O.global_of_local(rank, int(k)) for k in ks], np.int64)
        sel_s = js if sidx == G else ks
        sel_o = js if oidx == G else ks
    assert_same_f32(to_np(master)[sel_s], om[sel_s], "master " + tag)
    assert_same_f32(to_np(m)[sel_s], omm[sel_s], "m " + tag)
    assert_same_f32(to_np(v)[sel_s], ov[sel_s], "v " + tag)
    rest = np.setdiff1d(np.arange(se), sel_s)   # state outside the selection: as initialised
    assert_same_f32(to_np(master)[rest], init[rest], "master outside the selection " + tag)
    assert np.all(to_np(m)[rest] == 0) and np.all(to_np(v)[rest] == 0), \
        "m / v outside the selection were written " + tag
    for check, what in ((cw, "master"), (cm, "m"), (cv, "v")):
        check(f"{what} {tag}")
    if with_out:
        assert_same_bf16(to_np(out)[sel_o], oout[sel_o], "out " + tag)
        untouched = np.setdiff1d(np.arange(oe), sel_o)
        assert np.all(to_np(out)[untouched] == 0), "elements outside the selection were written"
        co(f"out {tag}")


def test_index_modes_bruteforce():
    rng = np.random.default_rng(11)
    cases = 0
    for n in (1, 2, 3, 4, 8):
        for numel in ([37], [64, 5, 0, 19], [8 * n + 3, 16 * n]):
            for gdt in (z.ZERO_BF16, z.ZERO_F32):
                ranks = [-1] + sorted(set([0, n - 1, n // 2]))
                for rank in ranks:
                    modes = [(G, G, G)] if rank < 0 else [(gi, si, oi) for gi in (G, Lc) for si in (G, Lc) for oi in (G, Lc)]
                    for gidx, sidx, oidx in modes:
                        shift = int(rng.integers(0, 8))
                        _run_case(rng, n, numel, rank, gdt, gidx, sidx, oidx, shift)
                        cases += 1
    log(f"index-mode cases: {cases}")


@pytest.mark.parametrize("n", [5, 7, 16, 32, 64, 100, 256])
def test_rank_counts(n):
    """Compile-time and runtime rank-count kernels, power-of-two and other
    divisors, multi-tile sizes with ragged tails."""
    rng = np.random.default_rng(n)
    numel = [n * 2048 + 11, 3 * n + 1] if n <= 64 else [n * 64 + 5]
    _run_case(rng, n, numel, -1, z.ZERO_BF16, G, G, G, shift=0)
    _run_case(rng, n, numel, n - 1, z.ZERO_BF16, Lc, Lc, Lc, shift=0)
    _run_case(rng, n, numel, 0, z.ZERO_BF16, G, Lc, G, shift=2)


@pytest.mark.parametrize("n,gdt,dist", [(8, z.ZERO_BF16, "wide"), (8, z.ZERO_F32, "normal"),
                                          (64, z.ZERO_BF16, "wide"), (5, z.ZERO_BF16, "wide"),
                                          (256, z.ZERO_F32, "normal")])
def test_rank_order_visible(n, gdt, dist):
    """Data on which another summation order changes bits (checked before
    the step): bf16 gradients whose magnitudes span 48 binades, or fp32
    gradients.  Eight bf16 values of one magnitude usually add exactly in
    binary32 whatever the order, so these cases are what proves the kernel
    sums in rank order."""
    rng = np.random.default_rng(100 + n)
    numel = [n * 4096 + 13] if n <= 64 else [n * 64 + 5]
    _run_case(rng, n, numel, -1, gdt, G, G, G, shift=0, dist=dist, check_order=True)
    _run_case(rng, n, numel, n // 2, gdt, Lc, Lc, Lc, shift=1, dist=dist, check_order=True)


@pytest.mark.parametrize("n", [33, 48, 64, 100, 256, 32, 25, 24, 8])
def test_staged_step(n):
    """zero_step_staged against the oracle, bit for bit: the workspace size
    sets the chunk, so small workspaces give many chunks with ragged ends
    inside every contiguous run; every index mode, both gradient types (each
    on aligned pointers, where the reduction loads whole spans, and on
    pointers that are not 16-byte aligned: the element path of the
    reduction, scalar heads of the step).  The fused step runs up to 32 bf16
    and 24 fp32 ranks."""
    log(f"staged n={n}")
    rng = np.random.default_rng(300 + n)
    numel = [n * 512 * 3 + 11, 3 * n + 1] if n <= 64 else [n * 64 * 9 + 5]
    for ws in (0, 512, 512 * 3, 4096):
        _run_case(rng, n, numel, -1, z.ZERO_BF16, G, G, G, shift=0, staged=ws)
        _run_case(rng, n, numel, n - 1, z.ZERO_BF16, Lc, Lc, Lc, shift=0, staged=ws)
        _run_case(rng, n, numel, 0, z.ZERO_F32, G, Lc, G, shift=2, staged=ws)
        _run_case(rng, n, numel, n - 1, z.ZERO_F32, Lc, Lc, Lc, shift=0, staged=ws)
        _run_case(rng, n, numel, n // 2, z.ZERO_BF16, Lc, G, Lc, shift=1, staged=ws, with_out=False)


def _staged_shifted(n, rank, numel, shift, rng, ws_elems, h, check, time_calls=0):
    L = z.zero_pack(n, numel)
    grads = [dev_buffer(L.shard, torch.bfloat16, shift=shift) for _ in range(n)]
    for g in grads:
        synth.fill_normal_(g, 1e-3, int(rng.integers(1 << 30)))
    w0 = rng.normal(0, 0.02, L.shard).astype(np.float32)
    master = dev_buffer(L.shard, torch.float32, shift=shift)
    master.copy_(torch.from_numpy(w0))
    m = dev_buffer(L.shard, torch.float32, shift=shift)
    v = dev_buffer(L.shard, torch.float32, shift=shift)
    out = dev_buffer(L.shard, torch.int16, shift=shift)
    ws = torch.empty(ws_elems, dtype=torch.float32, device=DEV)
    z.zero_step_staged(L, rank, grads, Lc, float(n), master, m, v, Lc, out, Lc, scalars(1, h), ws)
    torch.cuda.synchronize()
    if check:
        gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
        ow, om, ov = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
        oo = np.zeros(L.shard, np.uint16)
        oracle.zero_step_rank(n, numel, rank, gnp, grad_local=True, divisor=float(n), clip=1.0,
                              master=ow, m=om, v=ov, state_global=False, out=oo, out_gather=False, t=1,
                              **hyper_args(h))
        assert_same_f32(to_np(master), ow, f"master shift={shift}")
        assert_same_f32(to_np(v), ov, f"v shift={shift}")
        assert_same_bf16(to_np(out), oo, f"out shift={shift}")
    if not time_calls:
        return None

    def timed(staged):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        call = (lambda: z.zero_step_staged(L, rank, grads, Lc, float(n), master, m, v, Lc, out, Lc,
                                           scalars(2, h), ws)) if staged else \
            (lambda: z.zero_step(L, rank, grads, Lc, float(n), master, m, v, Lc, out, Lc, scalars(2, h)))
        for _ in range(3):
            call()
        a.record()
        for _ in range(time_calls):
            call()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / time_calls
    # interleaved, twice each
    t = [timed(True), timed(False), timed(True), timed(False)]
    return min(t[0], t[2]), min(t[1], t[3])


def test_staged_step_vectorizes_with_shifted_buffers():
    """Every buffer shifted by 1-3 elements (the gradients and the state then
    share a nonzero quad phase, which the fused step handles with a short
    element-wise head): the staged step places each chunk's reduced gradient
    at the state's phase, so both of its kernels still take their vector
    paths.  Bit for bit against the oracle at 1M elements per rank (two
    chunks); timed at 16M elements per rank against the fused step on the
    same shifted buffers (both pay the same for spans that straddle cache
    lines): no slower than 1.25 x the fused step (measured 0.93-1.05 x; the
    bound leaves room for timing noise), which it beats at 64 ranks when both
    run vector bodies (the element-wise kernels the unmatched phases used to
    fall back to are several times slower)."""
    n, rank, h = 64, 5, GPT_HYPER
    rng = np.random.default_rng(61)
    for shift in (0, 1, 2, 3):
        _staged_shifted(n, rank, [n * (1 << 20) + 3 * n], shift, rng, (1 << 20) + 4, h, check=True)
    big = [n * (1 << 24) + 3 * n]
    times = {shift: _staged_shifted(n, rank, big, shift, rng, (1 << 24) + 4, h, check=False,
                                    time_calls=10) for shift in (0, 1, 3)}
    log(f"(staged, fused) step ms by buffer shift (16M elements per rank): {times}")
    for shift in (0, 1, 3):
        staged, fused = times[shift]
        assert staged < 1.25 * fused, times


def test_staged_step_rank_order_visible():
    """The staged reduction sums in rank order: data on which another order
    changes bits (checked before the step), N = 64 and a runtime N."""
    for n in (64, 77):
        rng = np.random.default_rng(400 + n)
        _run_case(rng, n, [n * 4096 + 13], -1, z.ZERO_BF16, G, G, G, shift=0, dist="wide",
                  check_order=True, staged=2048)
        _run_case(rng, n, [n * 4096 + 13], n // 3, z.ZERO_F32, Lc, Lc, Lc, shift=0, check_order=True,
                  staged=0)


def test_ragged_multitile_and_no_out():
    rng = np.random.default_rng(5)
    numel = [1_000_003, 77, 12_293, 0, 4096 * 8 + 3]
    _run_case(rng, 8, numel, -1, z.ZERO_BF16, G, G, G, shift=0)
    _run_case(rng, 8, numel, 3, z.ZERO_BF16, G, Lc, G, shift=0)
    _run_case(rng, 8, numel, 5, z.ZERO_BF16, Lc, Lc, Lc, shift=1, with_out=False)


def test_reduced_gradient_input():
    """n_grads = 1: the step on an already-reduced fp32 gradient, the way the
    clipped step consumes the norm pass's output."""
    rng = np.random.default_rng(6)
    _run_case(rng, 8, [4096 + 3], 2, z.ZERO_F32, Lc, Lc, Lc, shift=0, n_grads=1)


@pytest.mark.parametrize("n,gdt", [(8, z.ZERO_BF16), (5, z.ZERO_BF16), (64, z.ZERO_BF16),
                                   (48, z.ZERO_BF16), (8, z.ZERO_F32), (3, z.ZERO_F32)])
def test_many_units_one_rank(n, gdt):
    """One rank's slice of 81 units with quad-aligned bases: the vector
    pieces go out several per launch (more than one launch carries), the
    heads and tails one by one; rank counts with a compiled kernel and
    without (48, fp32 at 3: one launch per piece)."""
    rng = np.random.default_rng(600 + n)
    numel = [1000 + 37 * k for k in range(80)] + [4096 * n + 5]
    for rank, (gidx, sidx, oidx) in ((n - 1, (G, Lc, G)), (n // 2, (G, G, Lc)), (0, (Lc, Lc, Lc))):
        _run_case(rng, n, numel, rank, gdt, gidx, sidx, oidx, shift=0)


def test_one_rank_piece_longer_than_a_launch():
    """A rank slice of more than 2^24 quads (2^18 workgroups) is cut across
    launches of the batched step: rank 1 of N = 2 over a 134M-element unit
    and a small one, GLOBAL gradients, LOCAL state and output."""
    rng = np.random.default_rng(601)
    n, numel, rank = 2, [2 * (1 << 26) + 24, 1000], 1
    h = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    L = z.zero_pack(n, numel)
    log(f"one rank, long piece: {L.shard} elements of rank {rank}")
    gnp = [(rng.standard_normal(L.padded, dtype=np.float32) * 1e-3) for _ in range(n)]
    grads = [torch.from_numpy(g).to(DEV).to(torch.bfloat16) for g in gnp]
    gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
    init = rng.normal(0, 0.02, L.shard).astype(np.float32)
    master = torch.from_numpy(init).to(DEV)
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(L.shard, dtype=torch.int16, device=DEV)
    z.zero_step(L, rank, grads, G, float(n), master, m, v, Lc, out, Lc, scalars(1, h))
    om, omm, ov = init.copy(), np.zeros(L.shard, np.float32), np.zeros(L.shard, np.float32)
    oout = np.zeros(L.shard, np.uint16)
    oracle.zero_step_rank(n, numel, rank, gnp, grad_local=False, divisor=float(n), clip=1.0,
                          master=om, m=omm, v=ov, state_global=False, out=oout, out_gather=False,
                          t=1, **hyper_args(h))
    torch.cuda.synchronize()
    assert_same_f32(to_np(master), om, "master")
    assert_same_f32(to_np(m), omm, "m")
    assert_same_f32(to_np(v), ov, "v")
    assert_same_bf16(to_np(out), oout, "bf16 out")


def test_rank_by_rank_equals_all_at_once_and_unsharded():
    """The pages' invariant on the GPU: every rank stepping its own shard
    (LOCAL state) reproduces the all-ranks step and plain AdamW."""
    n, numel = 8, [100_003, 4097]
    h = GPT_HYPER
    L = z.zero_pack(n, numel)
    O = oracle.Layout(n, numel)
    rng = np.random.default_rng(7)
    w0 = rng.normal(0, 0.02, L.padded).astype(np.float32)
    for u in range(len(numel)):
        w0[O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
    g = (rng.standard_normal((n, L.padded)) * 1e-3).astype(np.float32)
    for u in range(len(numel)):
        g[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
    grads = torch.from_numpy(g).to(DEV).to(torch.bfloat16)
    W = torch.from_numpy(w0).to(DEV)
    M, V = torch.zeros_like(W), torch.zeros_like(W)
    out_all = torch.zeros(L.padded, dtype=torch.int16, device=DEV)
    out_rank = torch.zeros(L.padded, dtype=torch.int16, device=DEV)
    idx = [torch.tensor([O.global_of_local(r, k) for k in range(L.shard)], device=DEV) for r in range(n)]
    ws = [W.index_select(0, idx[r]).contiguous() for r in range(n)]
    ms = [torch.zeros(L.shard, device=DEV) for _ in range(n)]
    vs = [torch.zeros(L.shard, device=DEV) for _ in range(n)]
    for t in (1, 2, 3):
        sc = scalars(t, h)
        z.zero_step(L, -1, list(grads), G, float(n), W, M, V, G, out_all, G, sc)
        for r in range(n):
            z.zero_step(L, r, list(grads), G, float(n), ws[r], ms[r], vs[r], Lc, out_rank, G, sc)
    torch.cuda.synchronize()
    Wr = torch.zeros_like(W)
    for r in range(n):
        Wr.index_copy_(0, idx[r], ws[r])
    assert_same_f32(to_np(Wr), to_np(W), "rank-by-rank vs all-at-once")
    assert_same_bf16(to_np(out_rank), to_np(out_all), "gathered bf16")
    # plain AdamW on the averaged gradient, unpadded
    gu = [np.ascontiguousarray(np.concatenate([to_np(grads[q])[O.offset[u]:O.offset[u] + numel[u]]
                                               for u in range(len(numel))])) for q in range(n)]
    wu = np.concatenate([w0[O.offset[u]:O.offset[u] + numel[u]] for u in range(len(numel))])
    mu, vu = np.zeros_like(wu), np.zeros_like(wu)
    for t in (1, 2, 3):
        oracle.adamw_unsharded(gu, divisor=float(n), clip=1.0, w=wu, m=mu, v=vu, t=t, **hyper_args(h))
    Wn = to_np(W)
    got = np.concatenate([Wn[O.offset[u]:O.offset[u] + numel[u]] for u in range(len(numel))])
    assert_same_f32(got, wu, "sharded GPU vs unsharded AdamW")


# ---------------------------------------------------------------------------
# Edge cases.
# ---------------------------------------------------------------------------

def test_empty_layouts_are_noops():
    for numel in ([], [0], [0, 0]):
        L = z.zero_pack(4, numel)
        dummy = torch.zeros(8, device=DEV)
        g = torch.zeros(8, dtype=torch.bfloat16, device=DEV)
        z.zero_step(L, -1, [g], G, 4.0, dummy, dummy.clone(), dummy.clone(), G, None, G,
                    scalars(1, GPT_HYPER))
        ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, -1) // 8, dtype=torch.float64, device=DEV)
        assert z.zero_gradnorm(L, -1, [g], G, 4.0, None, G, ws) == 0.0
    torch.cuda.synchronize()


def test_all_padding_shards():
    """P = 1 over N = 8: ranks 1..7 own nothing but padding; it stays +0."""
    rng = np.random.default_rng(8)
    for rank in range(8):
        _run_case(rng, 8, [1], rank, z.ZERO_BF16, G, Lc, G, shift=0)


def test_nan_and_inf_propagate_like_the_oracle():
    n, P = 4, 4096 + 5
    h = GPT_HYPER
    L = z.zero_pack(n, [P])
    rng = np.random.default_rng(9)
    g = (rng.standard_normal((n, L.padded)) * 1e-3).astype(np.float32)
    g[0, 10] = np.nan
    g[1, 20] = np.inf
    g[2, 20] = -np.inf          # inf + -inf = NaN
    g[3, 30] = np.inf
    g[0, 4000] = 3e38
    g[1, 4000] = 3e38           # overflow in the sum
    w0 = rng.normal(0, 0.02, L.padded).astype(np.float32)
    w0[40] = np.nan
    w0[41] = np.inf
    gb = torch.from_numpy(g).to(torch.bfloat16).to(DEV)
    W = torch.from_numpy(w0).to(DEV)
    M, V = torch.zeros_like(W), torch.zeros_like(W)
    out = torch.zeros(L.padded, dtype=torch.int16, device=DEV)
    gnp = [np.ascontiguousarray(to_np(gb[q])) for q in range(n)]
    om, omm, ov, oo = w0.copy(), np.zeros_like(w0), np.zeros_like(w0), np.zeros(L.padded, np.uint16)
    for t in (1, 2):
        z.zero_step(L, -1, list(gb), G, float(n), W, M, V, G, out, G, scalars(t, h))
        oracle.zero_step_all(n, [P], gnp, divisor=float(n), clip=1.0, master=om, m=omm, v=ov, out=oo,
                             t=t, **hyper_args(h))
    torch.cuda.synchronize()
    assert_same_f32(to_np(W), om, "master with NaN/Inf")
    assert_same_f32(to_np(M), omm, "m with NaN/Inf")
    assert_same_f32(to_np(V), ov, "v with NaN/Inf")
    assert_same_bf16(to_np(out), oo, "out with NaN/Inf")


def test_resume_equals_uninterrupted():
    """10 steps == 5 steps, copy the state out and back, 5 more steps."""
    n, numel = 8, [50_001]
    h = GPT_HYPER
    L = z.zero_pack(n, numel)
    rng = np.random.default_rng(10)
    w0 = rng.normal(0, 0.02, L.padded).astype(np.float32)
    w0[numel[0]:] = 0
    gsteps = []
    for _ in range(10):
        g = (rng.standard_normal((n, L.padded)) * 1e-3).astype(np.float32)
        g[:, numel[0]:] = 0
        gsteps.append(torch.from_numpy(g).to(torch.bfloat16).to(DEV))

    def run(W, M, V, t0, t1):
        for t in range(t0, t1):
            z.zero_step(L, -1, list(gsteps[t - 1]), G, float(n), W, M, V, G, None, G, scalars(t, h))

    A = [torch.from_numpy(w0).to(DEV), torch.zeros(L.padded, device=DEV), torch.zeros(L.padded, device=DEV)]
    run(*A, 1, 11)
    B = [torch.from_numpy(w0).to(DEV), torch.zeros(L.padded, device=DEV), torch.zeros(L.padded, device=DEV)]
    run(*B, 1, 6)
    saved = [to_np(x).copy() for x in B]
    C = [torch.from_numpy(s).to(DEV) for s in saved]
    run(*C, 6, 11)
    torch.cuda.synchronize()
    for a, c, name in zip(A, C, "wmv"):
        assert_same_f32(to_np(c), to_np(a), "resume " + name)


def test_bf16_cast_on_all_exponents():
    """With lr = 0 the update is exactly zero and decay exactly one, so the
    step writes bf16(master): every upper half-word with the low half-words
    that decide rounding, plus random patterns, against the oracle's cast."""
    import pins
    pats = pins.bf16_probe_patterns(seed=1, n_random=1 << 22)
    P = pats.size
    L = z.zero_pack(1, [P])
    W = torch.from_numpy(pats.view(np.float32).copy()).to(DEV)
    M, V = torch.zeros_like(W), torch.zeros_like(W)
    g = torch.zeros(P, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(P, dtype=torch.int16, device=DEV)
    sc = z.zero_adamw_scalars_for(1, 0.0, 0.9, 0.95, 1e-8, 0.1)
    assert sc.step_size == 0.0 and sc.decay == 1.0
    z.zero_step(L, -1, [g], G, 1.0, W, M, V, G, out, G, sc)
    torch.cuda.synchronize()
    x = pats.view(np.float32)
    assert_same_f32(to_np(W), x, "master unchanged at lr = 0")
    assert_same_bf16(to_np(out), oracle.bf16(x), "bf16 cast")


# ---------------------------------------------------------------------------
# Norm: full oracle comparison at moderate size, closed form, determinism.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n,numel,rank,gidx,gdt", [
    (64, [64 * 30_000 + 64, 64 * 777], 0, Lc, z.ZERO_BF16),
    (8, [1_000_003, 77], -1, G, z.ZERO_BF16),
    (8, [1_000_003, 77], 5, G, z.ZERO_BF16),
    (3, [10_001], 1, Lc, z.ZERO_F32),
])
def test_norm_and_clipped_step_vs_oracle(n, numel, rank, gidx, gdt):
    log(f"norm n={n} numel={numel} rank={rank}")
    rng = np.random.default_rng(12)
    L = z.zero_pack(n, numel)
    O = oracle.Layout(n, numel)
    ge = extent(L, gidx)
    gidx_state = G if rank < 0 else Lc
    se = extent(L, gidx_state)
    tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
    vals = (rng.standard_t(3, (n, ge)) * 1e-3 * 40).astype(np.float32)
    if gidx == G:
        for u in range(len(numel)):
            vals[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
    grads = torch.from_numpy(vals).to(tdt).to(DEV)
    gnp = [np.ascontiguousarray(to_np(grads[q])) for q in range(n)]
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
    g_out = torch.zeros(se, dtype=torch.float32, device=DEV)
    s1 = z.zero_gradnorm(L, rank, list(grads), gidx, float(n), g_out, gidx_state, ws)
    s2 = z.zero_gradnorm(L, rank, list(grads), gidx, float(n), None, gidx_state, ws)
    assert s1 == s2, "norm must be bitwise reproducible"
    # oracle: reduced gradient over the selection, then sum of squares
    if rank < 0:
        og = np.zeros(se, np.float32)
        for r in range(n):
            ks = oracle.reduced_grad(n, numel, r, gnp, grad_local=False, divisor=float(n))
            js = [O.global_of_local(r, k) for k in range(L.shard)]
            og[js] = ks
        sel = np.arange(se)
    else:
        og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n))
        sel = np.arange(se)
    assert_same_f32(to_np(g_out)[sel], og[sel], "reduced gradient written by the norm pass")
    osum = oracle.sumsq(og)
    assert abs(s1 - osum) <= 1e-12 * osum, (s1, osum)
    coef_gpu = z.zero_clip_coef(s1, 1.0)
    coef_orc = oracle.clip_coef(osum, 1.0)
    assert coef_gpu == coef_orc
    assert coef_gpu < 1.0, "the test data should make clipping active"
    # the clipped step reading the reduced gradient (n_grads = 1, divisor 1)
    h = GPT_HYPER
    w0 = rng.normal(0, 0.02, se).astype(np.float32)
    W = torch.from_numpy(w0).to(DEV)
    M, V = torch.zeros_like(W), torch.zeros_like(W)
    out = torch.zeros(se, dtype=torch.int16, device=DEV)
    sc = scalars(1, h, clip=coef_gpu)
    if rank < 0:
        z.zero_step(L, -1, [g_out], G, 1.0, W, M, V, G, out, G, sc)
    else:
        z.zero_step(L, rank, [g_out], Lc, 1.0, W, M, V, Lc, out, Lc, sc)
    # and the same step straight from the N gradients
    W2 = torch.from_numpy(w0).to(DEV)
    M2, V2 = torch.zeros_like(W2), torch.zeros_like(W2)
    z.zero_step(L, rank, list(grads), gidx, float(n), W2, M2, V2, gidx_state, None, gidx_state, sc)
    torch.cuda.synchronize()
    om, omm, ov, oo = w0.copy(), np.zeros(se, np.float32), np.zeros(se, np.float32), np.zeros(se, np.uint16)
    oracle.zero_step_rank(1, [se], 0, [og], grad_local=True, divisor=1.0, clip=coef_orc, master=om,
                          m=omm, v=ov, state_global=False, out=oo, out_gather=False, t=1, **hyper_args(h))
    assert_same_f32(to_np(W), om, "clipped master")
    assert_same_f32(to_np(V), ov, "clipped v")
    assert_same_bf16(to_np(out), oo, "clipped out")
    assert_same_f32(to_np(W2), om, "clipped master from N gradients")


def test_norm_async_equals_sync():
    """The async pass leaves the same bits on the device as the synchronous
    call returns, for vector and unaligned pieces and an empty selection."""
    rng = np.random.default_rng(14)
    for n, numel, rank, gidx in [(8, [100_003, 5], -1, G), (8, [100_003, 5], 3, G), (16, [16 * 999], 2, Lc)]:
        L = z.zero_pack(n, numel)
        ge = extent(L, gidx)
        se = extent(L, G if rank < 0 else Lc)
        grads = [dev_buffer(ge, torch.bfloat16, shift=q % 3) for q in range(n)]
        for g in grads:
            g.copy_(torch.from_numpy((rng.standard_normal(ge) * 1e-2).astype(np.float32)).to(torch.bfloat16))
        ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
        sidx = G if rank < 0 else Lc
        want = z.zero_gradnorm(L, rank, grads, gidx, float(n), None, sidx, ws)
        res = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        z.zero_gradnorm_async(L, rank, grads, gidx, float(n), None, sidx, ws, res)
        torch.cuda.synchronize()
        assert res.item() == want
    L = z.zero_pack(4, [0])
    g = torch.zeros(8, dtype=torch.bfloat16, device=DEV)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, -1) // 8, dtype=torch.float64, device=DEV)
    res = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    z.zero_gradnorm_async(L, -1, [g], G, 4.0, None, G, ws, res)
    torch.cuda.synchronize()
    assert res.item() == 0.0 and not torch.signbit(res).item()


@pytest.mark.parametrize("n,gdt", [(8, z.ZERO_BF16), (64, z.ZERO_BF16), (5, z.ZERO_BF16), (8, z.ZERO_F32)])
def test_norm_partition_independent_of_alignment(n, gdt):
    """The same gradients in 16-byte-aligned buffers (whole tiles on the
    vector path) and shifted by 1..7 elements (every tile element by element)
    give the same sum of squares and the same reduced gradient, bit for bit:
    the partition into tiles and lanes depends only on the layout."""
    log(f"norm alignment n={n} gdt={gdt}")
    rng = np.random.default_rng(15 + n)
    numel = [n * (512 * 9 + 77), n * 300 + n]      # several tiles, ragged tails, two segments
    L = z.zero_pack(n, numel)
    rank = 1
    tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
    vals = (rng.standard_t(3, (n, L.shard)) * 1e-3).astype(np.float32)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
    res = {}
    for shift in (0, 1, 3, 7):
        grads = [dev_buffer(L.shard, tdt, shift=shift) for _ in range(n)]
        for q in range(n):
            grads[q].copy_(torch.from_numpy(vals[q]).to(tdt))
        g_out = dev_buffer(L.shard, torch.float32, shift=shift)
        s = z.zero_gradnorm(L, rank, grads, Lc, float(n), g_out, Lc, ws)
        res[shift] = (s, to_np(g_out).copy())
    s0, g0 = res[0]
    for shift in (1, 3, 7):
        s, g = res[shift]
        assert s == s0, (shift, s, s0)
        assert_same_f32(g, g0, f"reduced gradient, shift {shift}")
    # and the oracle's value
    gnp = [np.ascontiguousarray(to_np(torch.from_numpy(vals[q]).to(tdt))) for q in range(n)]
    og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=True, divisor=float(n))
    assert_same_f32(g0, og, "reduced gradient vs oracle")
    osum = oracle.sumsq(og)
    assert abs(s0 - osum) <= 1e-12 * osum


@pytest.mark.parametrize("tdt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_norm_phased_tiles_shared_launch_cut(tdt):
    """One rank's slice of two units from full (GLOBAL) gradient buffers, each
    starting off a 128-byte line (bf16: 40 and 16 elements past one; fp32: 8
    and 16), so the norm's first tile of each starts that far before its
    segment; the first slice
    is longer than one shared launch holds (2^18 tiles), so it is cut.  The
    reduced gradient and the sum equal the same pass on buffers shifted by
    one element (every tile element by element, one launch per segment) bit
    for bit, g_out's neighbours stay untouched, and both match the oracle."""
    n, rank = 2, 1
    numel = [2 * ((1 << 27) + 40), 2 * 1024]
    L = z.zero_pack(n, numel)
    log(f"norm phased tiles: rank {rank} slice of {L.shard} elements, {tdt}")
    gen = torch.Generator(device=DEV).manual_seed(616)
    vals = [(torch.randn(L.padded, device=DEV, generator=gen) * 2e-3).to(tdt) for _ in range(n)]
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
    guard = 96
    res = {}
    for shift in (0, 1):
        grads = [dev_buffer(L.padded, tdt, shift=shift) for _ in range(n)]
        for q in range(n):
            grads[q].copy_(vals[q])
        base = torch.full((L.shard + 2 * guard + shift,), float("nan"), device=DEV)
        g_out = base[guard + shift:guard + shift + L.shard]
        s = z.zero_gradnorm(L, rank, grads, G, float(n), g_out, Lc, ws)
        torch.cuda.synchronize()
        assert torch.isnan(base[:guard + shift]).all() and torch.isnan(base[guard + shift + L.shard:]).all(), \
            f"shift {shift}: the pass wrote outside g_out"
        res[shift] = (s, to_np(g_out).copy())
        del grads, base, g_out
    (s0, g0), (s1, g1) = res[0], res[1]
    assert s0 == s1, (s0, s1)
    assert_same_f32(g1, g0, "reduced gradient, shifted buffers")
    gnp = [np.ascontiguousarray(to_np(v)) for v in vals]
    og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=False, divisor=float(n))
    assert_same_f32(g0, og, "reduced gradient vs oracle")
    serial = oracle.sumsq(og)
    pair = float(np.sum(og.astype(np.float64) ** 2))
    assert abs(s0 - serial) <= og.size * 2.0 ** -53 * serial, (s0, serial)
    assert abs(s0 - pair) <= 1e-12 * pair, (s0, pair)


def test_norm_closed_form():
    """Every rank's gradient equal to c: the average is c exactly and the sum
    of squares is (elements) * c^2 exactly in binary64."""
    n, P = 64, 64 * 100_000
    L = z.zero_pack(n, [P])
    c = 0.375
    grads = [torch.full((L.shard,), c, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, 3) // 8, dtype=torch.float64, device=DEV)
    s = z.zero_gradnorm(L, 3, grads, Lc, float(n), None, Lc, ws)
    assert s == L.shard * c * c


# ---------------------------------------------------------------------------
# Packer copies.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("src_dt,dst_dt", [(torch.float32, torch.float32), (torch.float32, torch.bfloat16),
                                           (torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16)])
def test_pack_and_unpack(src_dt, dst_dt):
    from fsdp_sharded_optimizer_flat_amd.workloads import gpt2_block, numel_of
    rng = np.random.default_rng(13)
    n = 8
    shapes = [s for _, s in gpt2_block(64)] + [(13,), (5, 3)]
    units = [0] * 12 + [1, 1]
    params = [torch.from_numpy(rng.standard_normal(numel_of(s)).astype(np.float32)).to(src_dt).to(DEV)
              for s in shapes]
    unit_numel = [sum(numel_of(s) for s, u in zip(shapes, units) if u == k) for k in (0, 1)]
    L = z.zero_pack(n, unit_numel)
    O = oracle.Layout(n, unit_numel)
    flat = torch.full((L.padded,), 7, dtype=dst_dt, device=DEV)
    z.zero_pack_copy(L, -1, params, units, flat)
    # expected flat buffer, built on the host from the oracle's layout
    exp = np.zeros(L.padded, np.float32)
    pos = [0, 0]
    for p, u in zip(params, units):
        a = O.offset[u] + pos[u]
        exp[a:a + p.numel()] = p.float().cpu().numpy()
        pos[u] += p.numel()
    got = flat.float().cpu().numpy()
    want = torch.from_numpy(exp).to(dst_dt).float().numpy()
    assert_same_f32(got, want, "packed flat buffer (padding zero)")
    for r in (0, 5, n - 1):
        shard = torch.full((L.shard,), 7, dtype=dst_dt, device=DEV)
        z.zero_pack_copy(L, r, params, units, shard)
        js = [O.global_of_local(r, k) for k in range(L.shard)]
        assert_same_f32(shard.float().cpu().numpy(), want[js], f"rank {r} shard")
    back = [torch.zeros_like(p) for p in params]
    z.zero_unpack_copy(L, -1, flat, back, units)
    torch.cuda.synchronize()
    for p, b in zip(params, back):
        assert_same_f32(b.float().cpu().numpy(), p.to(dst_dt).to(src_dt).float().cpu().numpy(), "unpack")


def test_host_step_equals_gpu_step():
    """The offload (host) step and the GPU step give the same bits."""
    rng = np.random.default_rng(31)
    n, numel = 8, [200_003, 4097]
    L = z.zero_pack(n, numel)
    h = GPT_HYPER
    g = (rng.standard_normal((n, L.shard)) * 1e-3).astype(np.float32)
    gb = torch.from_numpy(g).to(torch.bfloat16)
    w0 = rng.normal(0, 0.02, L.shard).astype(np.float32)
    W, M, V = torch.from_numpy(w0).to(DEV), torch.zeros(L.shard, device=DEV), torch.zeros(L.shard, device=DEV)
    O = torch.zeros(L.shard, dtype=torch.int16, device=DEV)
    gd = gb.to(DEV)
    hw, hm, hv = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    ho = np.zeros(L.shard, np.uint16)
    hg = [np.ascontiguousarray(gb[q].view(torch.int16).numpy().view(np.uint16)) for q in range(n)]
    for t in (1, 2, 3):
        z.zero_step(L, 4, list(gd), Lc, float(n), W, M, V, Lc, O, Lc, scalars(t, h))
        z.zero_step_host(L, 4, hg, Lc, float(n), hw, hm, hv, Lc, ho, Lc, scalars(t, h), 0)
    torch.cuda.synchronize()
    assert_same_f32(to_np(W), hw, "host vs GPU master")
    assert_same_f32(to_np(V), hv, "host vs GPU v")
    assert_same_bf16(to_np(O), ho, "host vs GPU out")


@pytest.mark.parametrize("chunk", [1 << 16, 100_003, 1 << 22])
def test_offload_step_equals_gpu_step(chunk):
    """The pipelined offload step (reduced gradient down over PCIe, host step,
    bf16 parameters up) against the GPU step on the same reduced gradient."""
    rng = np.random.default_rng(32)
    n, numel = 8, [8 * 300_007, 8 * 77]
    L = z.zero_pack(n, numel)
    h = GPT_HYPER
    S = L.shard
    g = torch.from_numpy((rng.standard_normal(S) * 1e-3).astype(np.float32)).to(DEV)
    w0 = rng.normal(0, 0.02, S).astype(np.float32)
    W, M, V = torch.from_numpy(w0).to(DEV), torch.zeros(S, device=DEV), torch.zeros(S, device=DEV)
    O = torch.zeros(S, dtype=torch.int16, device=DEV)
    hw = torch.from_numpy(w0.copy())
    hm, hv = torch.zeros(S), torch.zeros(S)
    gst = torch.zeros(2 * chunk, dtype=torch.float32, pin_memory=True)
    ost = torch.zeros(2 * chunk, dtype=torch.int16, pin_memory=True)
    dO = torch.zeros(S, dtype=torch.int16, device=DEV)
    s_down, s_up = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    for t in (1, 2):
        sc = scalars(t, h, clip=0.75)
        z.zero_step(L, 2, [g], Lc, 1.0, W, M, V, Lc, O, Lc, sc)
        torch.cuda.synchronize()
        z.zero_offload_step(L, 2, g, gst, hw, hm, hv, ost, dO, chunk, sc, 0, s_down, s_up)
    torch.cuda.synchronize()
    assert_same_f32(hw.numpy(), to_np(W), "offload master")
    assert_same_f32(hv.numpy(), to_np(V), "offload v")
    assert_same_bf16(to_np(dO), to_np(O), "offload bf16 params on the device")


def test_device_clip_coefficient_equals_host():
    """zero_clip_coef_async forms the same binary32 coefficient as the host."""
    rng = np.random.default_rng(33)
    vals = np.concatenate([10.0 ** rng.uniform(-14, 10, 20000), [0.0, 1.0, 0.999999e0, 4.0, 1e-12]])
    res = torch.empty(1, dtype=torch.float32, device=DEV)
    d = torch.from_numpy(vals).to(DEV)
    for i in range(0, vals.size, 997):   # spread over the range; one launch per value
        for mx in (1.0, 0.5):
            z.zero_clip_coef_async(d[i:i + 1], mx, res)
            assert res.item() == z.zero_clip_coef(float(vals[i]), mx), (vals[i], mx)


def test_nonfinite_norm_skips_the_device_clip_step():
    """The sync-free chain on a gradient with an infinite or NaN element: the
    norm pass's sum is not finite, zero_clip_coef_async writes NaN (where the
    host refuses the sum), and zero_step_device_clip leaves master, m, v and
    the bf16 output bit for bit as they were -- on the quad path and on the
    one-element path (shifted pointers).  The same chain on the repaired
    gradient then steps, equal to the oracle's clipped step."""
    coef = torch.empty(1, dtype=torch.float32, device=DEV)
    for sums in ([np.inf], [np.nan], [-1.0], [1.0, np.inf], [1.7e308, 1.7e308]):
        d = torch.tensor(sums, dtype=torch.float64, device=DEV)
        if len(sums) == 1:
            z.zero_clip_coef_async(d, 1.0, coef)
        else:
            z.zero_clip_coef_ranks_async(d, 1.0, coef)
        assert np.isnan(coef.item()), sums
    n, numel, rank = 8, [4096 * 3 + 5, 77], 3
    L = z.zero_pack(n, numel)
    h = GPT_HYPER
    rng = np.random.default_rng(51)
    for bad in (np.inf, -np.inf, np.nan):
        for shift in (0, 1):
            grads = [dev_buffer(L.shard, torch.bfloat16, shift=shift) for _ in range(n)]
            for g in grads:
                g.copy_(torch.from_numpy((rng.standard_normal(L.shard) * 1e-3).astype(np.float32)))
            master = dev_buffer(L.shard, torch.float32, shift=shift)
            m = dev_buffer(L.shard, torch.float32, shift=shift)
            v = dev_buffer(L.shard, torch.float32, shift=shift)
            for t_ in (master, m, v):
                t_.copy_(torch.from_numpy(np.abs(rng.normal(0, 0.02, L.shard)).astype(np.float32)))
            out = dev_buffer(L.shard, torch.int16, shift=shift, fill=0x1234)
            g_red = dev_buffer(L.shard, torch.float32, shift=shift)
            ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
            ss = torch.zeros(1, dtype=torch.float64, device=DEV)
            before = [to_np(x).copy() for x in (master, m, v, out)]
            good = grads[2][100].item()
            grads[2][100] = float(bad)
            z.zero_gradnorm_async(L, rank, grads, Lc, float(n), g_red, Lc, ws, ss)
            z.zero_clip_coef_async(ss, 1.0, coef)
            z.zero_step_device_clip(L, rank, [g_red], Lc, 1.0, master, m, v, Lc, out, Lc, scalars(2, h), coef)
            torch.cuda.synchronize()
            assert not np.isfinite(ss.item()) and np.isnan(coef.item()), (bad, ss.item())
            for got, want, name in zip((master, m, v, out), before, ("master", "m", "v", "out")):
                assert np.array_equal(to_np(got).view(np.uint32 if want.dtype == np.float32 else np.uint16),
                                      want.view(np.uint32 if want.dtype == np.float32 else np.uint16)), \
                    f"{name} changed by a skipped step (bad={bad}, shift={shift})"
            # repaired: the chain steps, as the oracle does with its own coefficient
            grads[2][100] = good
            z.zero_gradnorm_async(L, rank, grads, Lc, float(n), g_red, Lc, ws, ss)
            z.zero_clip_coef_async(ss, 1.0, coef)
            z.zero_step_device_clip(L, rank, [g_red], Lc, 1.0, master, m, v, Lc, out, Lc, scalars(2, h), coef)
            torch.cuda.synchronize()
            gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
            og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=True, divisor=float(n))
            oc = oracle.clip_coef(oracle.sumsq(og), 1.0)
            assert coef.item() == oc
            ow, om, ov = (x.copy() for x in before[:3])
            oo = before[3].copy()
            oracle.zero_step_rank(n, numel, rank, gnp, grad_local=True, divisor=float(n), clip=oc,
                                  master=ow, m=om, v=ov, state_global=False, out=oo, out_gather=False,
                                  t=2, **hyper_args(h))
            assert_same_f32(to_np(master), ow, "master after the repaired step")
            assert_same_f32(to_np(v), ov, "v after the repaired step")
            assert_same_bf16(to_np(out), oo, "out after the repaired step")


def test_clip_coefficient_across_ranks_on_the_device():
    """Every rank's sum of squares left on the device (zero_gradnorm_async
    per rank), combined in rank order on the device: bitwise equal to the host
    combination of the same sums; the total within 1e-12 of the oracle's
    rank-ordered total of its per-rank sums, the coefficient equal."""
    rng = np.random.default_rng(19)
    n, numel = 8, [8 * 20_000 + 3, 515]
    L = z.zero_pack(n, numel)
    vals = (rng.standard_t(3, (n, L.padded)) * 2e-3).astype(np.float32)
    O = oracle.Layout(n, numel)
    for u in range(len(numel)):
        vals[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
    grads = torch.from_numpy(vals).to(torch.bfloat16).to(DEV)
    gnp = [np.ascontiguousarray(to_np(grads[q])) for q in range(n)]
    sums = torch.zeros(n, dtype=torch.float64, device=DEV)
    for r in range(n):
        ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, r) // 8, dtype=torch.float64, device=DEV)
        z.zero_gradnorm_async(L, r, list(grads), G, float(n), None, Lc, ws, sums[r:r + 1])
    coef_dev = torch.zeros(1, dtype=torch.float32, device=DEV)
    total_dev = torch.zeros(1, dtype=torch.float64, device=DEV)
    z.zero_clip_coef_ranks_async(sums, 0.1, coef_dev, total_dev)
    torch.cuda.synchronize()
    host_coef, host_total = z.zero_clip_coef_ranks(sums.cpu().numpy(), 0.1)
    assert total_dev.item() == host_total and coef_dev.item() == host_coef
    orc_total = 0.0
    for r in range(n):
        og = oracle.reduced_grad(n, numel, r, gnp, grad_local=False, divisor=float(n))
        orc_total = orc_total + oracle.sumsq(og)
    assert abs(host_total - orc_total) <= 1e-12 * orc_total
    assert host_coef == oracle.clip_coef(orc_total, 0.1) and host_coef < 1.0
    # the same total as one all-shards norm pass (rank = -1), to rounding
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, -1) // 8, dtype=torch.float64, device=DEV)
    whole = z.zero_gradnorm(L, -1, list(grads), G, float(n), None, G, ws)
    assert abs(whole - host_total) <= 1e-12 * host_total


def test_clipped_step_without_host_sync_and_in_a_graph():
    """norm (async) -> coefficient (device) -> step reading it: equal to the
    host-synchronized clipped step, eagerly and replayed from a HIP graph."""
    rng = np.random.default_rng(34)
    n, numel = 16, [16 * 40_000 + 16, 16 * 77]
    L = z.zero_pack(n, numel)
    h = GPT_HYPER
    grads = torch.from_numpy((rng.standard_t(3, (n, L.shard)) * 4e-2).astype(np.float32)).to(torch.bfloat16).to(DEV)
    gl = list(grads)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, 1) // 8, dtype=torch.float64, device=DEV)
    g_red = torch.empty(L.shard, device=DEV)
    ssd = torch.zeros(1, dtype=torch.float64, device=DEV)
    coef = torch.zeros(1, dtype=torch.float32, device=DEV)
    w0 = rng.normal(0, 0.02, L.shard).astype(np.float32)

    def fresh():
        return (torch.from_numpy(w0).to(DEV), torch.zeros(L.shard, device=DEV), torch.zeros(L.shard, device=DEV),
                torch.zeros(L.shard, dtype=torch.int16, device=DEV))

    # reference: host round trip
    W, M, V, O = fresh()
    for t in (1, 2, 3):
        ss = z.zero_gradnorm(L, 1, gl, Lc, float(n), None, Lc, ws)
        z.zero_step(L, 1, gl, Lc, float(n), W, M, V, Lc, O, Lc, scalars(t, h, clip=z.zero_clip_coef(ss, 1.0)))
    torch.cuda.synchronize()
    assert z.zero_clip_coef(ss, 1.0) < 1.0

    def device_chain(t, W2, M2, V2, O2, stream=None):
        z.zero_gradnorm_async(L, 1, gl, Lc, float(n), g_red, Lc, ws, ssd, stream)
        z.zero_clip_coef_async(ssd, 1.0, coef, stream)
        z.zero_step_device_clip(L, 1, [g_red], Lc, 1.0, W2, M2, V2, Lc, O2, Lc, scalars(t, h), coef, stream)

    W2, M2, V2, O2 = fresh()
    for t in (1, 2, 3):
        device_chain(t, W2, M2, V2, O2)
    torch.cuda.synchronize()
    assert_same_f32(to_np(W2), to_np(W), "device-clip chain master")
    assert_same_bf16(to_np(O2), to_np(O), "device-clip chain out")

    # the same chain captured once per step count and replayed, with eager work
    # and synchronizations between the replays; every replay checked
    W3, M3, V3, O3 = fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for t in (1, 2, 3):
        gph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gph, stream=s):
            device_chain(t, W3, M3, V3, O3, s)
        graphs.append(gph)
    torch.cuda.synchronize()
    W3.copy_(torch.from_numpy(w0).to(DEV)); M3.zero_(); V3.zero_(); O3.zero_()
    Wr, Mr, Vr, Or = fresh()
    for t in (1, 2, 3):
        graphs[t - 1].replay()
        torch.cuda.synchronize()
        device_chain(t, Wr, Mr, Vr, Or)          # eager, between replays
        torch.cuda.synchronize()
        assert_same_f32(to_np(W3), to_np(Wr), f"graph replay {t} master")
        assert_same_f32(to_np(V3), to_np(Vr), f"graph replay {t} v")
        assert_same_bf16(to_np(O3), to_np(Or), f"graph replay {t} out")
    assert_same_f32(to_np(W3), to_np(W), "graph chain vs host-synchronized step")


def test_random_sweep():
    """A seeded sweep across the step's parameter space, each case against the
    oracle bit for bit: rank counts from 1 to 256 (compile-time and runtime
    kernels), 1-5 units of random size (padding, empty units, several tiles
    and ragged tails), every rank or one, every valid index-mode combination,
    both gradient types, pointers shifted off 16-byte alignment, the bf16
    output on or off, one or two steps, and the staged step with random
    workspace sizes."""
    rng = np.random.default_rng(2024)
    for case in range(150):
        n = int(rng.choice([1, 2, 3, 5, 8, 16, 17, 31, 32, 33, 47, 64, 65, 128, 200, 256]))
        numel = [int(rng.integers(0, 6144)) if rng.random() < 0.8 else int(rng.integers(0, 40))
                 for _ in range(int(rng.integers(1, 6)))]
        if sum(numel) == 0:
            numel[0] = 1
        rank = int(rng.integers(-1, n))
        gdt = z.ZERO_BF16 if rng.random() < 0.7 else z.ZERO_F32
        if rank < 0:
            gidx = sidx = oidx = G
        else:
            gidx, sidx, oidx = (G if rng.random() < 0.5 else Lc for _ in range(3))
        staged = None
        if rng.random() < 0.4:
            staged = int(rng.choice([0, 512, 1024, 512 * int(rng.integers(3, 40))]))
        kw = dict(steps=int(rng.integers(1, 3)), with_out=bool(rng.random() < 0.85), staged=staged)
        log(f"sweep case {case}: n={n} numel={numel} rank={rank} gdt={gdt} "
            f"idx={gidx}{sidx}{oidx} {kw}")
        _run_case(rng, n, numel, rank, gdt, gidx, sidx, oidx, int(rng.integers(0, 8)), **kw)


def test_norm_random_sweep():
    """A seeded sweep of the norm pass against the oracle: rank counts 1-256,
    random layouts, every rank or one, GLOBAL or LOCAL gradients, both
    gradient types, pointers shifted off 16-byte alignment, with and without
    writing g.  The written g must equal the oracle's reduced gradient bit
    for bit, the sum of squares must agree with the oracle's to 1e-12 and be
    the same bits with or without g, and nothing past the workspace the size
    query gives may be written."""
    rng = np.random.default_rng(77)
    for case in range(80):
        n = int(rng.choice([1, 2, 3, 7, 8, 16, 32, 33, 64, 100, 256]))
        numel = [int(rng.integers(0, 5000)) for _ in range(int(rng.integers(1, 5)))]
        if sum(numel) == 0:
            numel[0] = 3
        rank = int(rng.integers(-1, n))
        gidx = G if rank < 0 or rng.random() < 0.5 else Lc
        gdt = z.ZERO_BF16 if rng.random() < 0.7 else z.ZERO_F32
        sidx = G if rank < 0 else Lc
        log(f"norm sweep case {case}: n={n} numel={numel} rank={rank} gidx={gidx} gdt={gdt}")
        L = z.zero_pack(n, numel)
        O = oracle.Layout(n, numel)
        ge, se = extent(L, gidx), extent(L, sidx)
        tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
        vals = (rng.standard_t(3, (n, ge)) * 1e-3).astype(np.float32)
        if gidx == G:   # the padding of a flat buffer holds +0.0
            for u in range(len(numel)):
                vals[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
        grads = []
        for q in range(n):
            g = dev_buffer(ge, tdt, shift=int(rng.integers(0, 8)))
            g.copy_(torch.from_numpy(vals[q]).to(tdt))
            grads.append(g)
        gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
        need = max(z.zero_gradnorm_workspace_bytes(L, rank) // 8, 1)
        ws_full = torch.full((need + 64,), -99.0, dtype=torch.float64, device=DEV)
        ws = ws_full[:need]   # 64 sentinels past it, which the pass must not touch
        g_out, cg = dev_buffer_guarded(se, torch.float32, shift=int(rng.integers(0, 4)), fill=-7.0)
        s1 = z.zero_gradnorm(L, rank, grads, gidx, float(n), g_out, sidx, ws)
        s2 = z.zero_gradnorm(L, rank, grads, gidx, float(n), None, sidx, ws)
        assert s1 == s2, "the sum must not depend on whether g is written"
        assert bool((ws_full[need:] == -99.0).all()), f"case {case}: the norm pass wrote past its workspace"
        cg(f"g, case {case}")
        if rank < 0:
            og = np.zeros(se, np.float32)
            for r in range(n):
                ks = oracle.reduced_grad(n, numel, r, gnp, grad_local=False, divisor=float(n))
                og[[O.global_of_local(r, k) for k in range(L.shard)]] = ks
        else:
            og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n))
        assert_same_f32(to_np(g_out), og, f"g, case {case}")
        osum = oracle.sumsq(og)
        assert abs(s1 - osum) <= 1e-12 * osum, (case, s1, osum)


def test_pack_random_sweep():
    """A seeded sweep of the packer against the oracle's layout: random rank
    counts, parameter counts and sizes (empty ones included), unit groupings
    (empty units included), every rank or one, every dtype pair, shifted
    pointers.  Pack must place every element at its offset with +0.0 padding
    (bit for bit after the dtype conversion); unpack from the flat buffer
    must return every parameter, and unpack from a rank's shard exactly the
    elements that rank owns, leaving the rest untouched."""
    rng = np.random.default_rng(91)
    dts = [torch.float32, torch.bfloat16]
    for case in range(40):
        n = int(rng.choice([1, 2, 3, 5, 8, 13, 32, 64]))
        n_params = int(rng.integers(1, 13))
        numels = [int(rng.integers(0, 3000)) if rng.random() < 0.9 else 0 for _ in range(n_params)]
        n_units = int(rng.integers(1, 5))
        units = sorted(int(u) for u in rng.integers(0, n_units, n_params))
        unit_numel = [sum(k for k, u in zip(numels, units) if u == j) for j in range(n_units)]
        if sum(unit_numel) == 0:
            numels[0] = unit_numel[units[0]] = 17
        src_dt, dst_dt = dts[int(rng.integers(0, 2))], dts[int(rng.integers(0, 2))]
        rank = int(rng.integers(-1, n))
        log(f"pack sweep case {case}: n={n} numels={numels} units={units} rank={rank} "
            f"{src_dt}->{dst_dt}")
        L = z.zero_pack(n, unit_numel)
        O = oracle.Layout(n, unit_numel)
        params = []
        for k in numels:
            p = dev_buffer(k, src_dt, shift=int(rng.integers(0, 8)))
            p.copy_(torch.from_numpy(rng.standard_normal(k).astype(np.float32)).to(src_dt))
            params.append(p)
        exp = np.zeros(L.padded, np.float32)
        pos = [0] * n_units
        for p, u in zip(params, units):
            a = O.offset[u] + pos[u]
            exp[a:a + p.numel()] = p.float().cpu().numpy()
            pos[u] += p.numel()
        want = torch.from_numpy(exp).to(dst_dt).float().numpy()
        flat = dev_buffer(L.padded, dst_dt, shift=int(rng.integers(0, 8)), fill=7)
        z.zero_pack_copy(L, -1, params, units, flat)
        assert_same_f32(flat.float().cpu().numpy(), want, f"flat, case {case}")
        js = np.array([O.global_of_local(max(rank, 0), k) for k in range(L.shard)], np.int64)
        if rank >= 0:
            shard = dev_buffer(L.shard, dst_dt, shift=int(rng.integers(0, 8)), fill=7)
            z.zero_pack_copy(L, rank, params, units, shard)
            assert_same_f32(shard.float().cpu().numpy(), want[js], f"rank {rank} shard, case {case}")
        # unpack: from the flat buffer (every element), or from the rank's shard
        src = flat if rank < 0 else shard
        back = [dev_buffer(p.numel(), src_dt, shift=int(rng.integers(0, 8)), fill=-3) for p in params]
        z.zero_unpack_copy(L, rank, src, back, units)
        torch.cuda.synchronize()
        owned = np.zeros(L.padded, bool)
        owned[js if rank >= 0 else slice(None)] = True
        pos = [0] * n_units
        for p, b, u in zip(params, back, units):
            a = O.offset[u] + pos[u]
            pos[u] += p.numel()
            full = p.to(dst_dt).to(src_dt).float().cpu().numpy()
            expect = np.where(owned[a:a + p.numel()], full, np.float32(-3))
            assert_same_f32(b.float().cpu().numpy(), expect, f"unpack, case {case}")


def test_clip_chain_random_sweep():
    """A seeded sweep of the sync-free clipped step -- norm pass writing g,
    coefficient on the device, step reading g and the coefficient -- against
    the oracle's clipped step from the N gradients: random rank counts,
    layouts, ranks, gradient types and index spaces, heavy-tailed gradients
    large enough that clipping is active.  The coefficient must equal the
    oracle's (formed from the oracle's sum of squares) and master / m / v /
    bf16 out must match bit for bit."""
    rng = np.random.default_rng(123)
    h = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    for case in range(30):
        n = int(rng.choice([1, 2, 4, 8, 16, 33, 64, 100]))
        numel = [int(rng.integers(1, 6000)) for _ in range(int(rng.integers(1, 4)))]
        rank = int(rng.integers(-1, n))
        gidx = G if rank < 0 or rng.random() < 0.5 else Lc
        sidx = G if rank < 0 else Lc
        gdt = z.ZERO_BF16 if rng.random() < 0.7 else z.ZERO_F32
        log(f"clip chain case {case}: n={n} numel={numel} rank={rank} gidx={gidx} gdt={gdt}")
        L = z.zero_pack(n, numel)
        O = oracle.Layout(n, numel)
        ge, se = extent(L, gidx), extent(L, sidx)
        tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
        # the average of n Student-t(3) draws has variance 3 s^2 / n: scale so
        # that the expected norm over the selection is about 10
        s_ = np.sqrt(100.0 * n / (3.0 * se))
        vals = (rng.standard_t(3, (n, ge)) * s_).astype(np.float32)
        if gidx == G:
            for u in range(len(numel)):
                vals[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
        grads = [dev_buffer(ge, tdt, shift=int(rng.integers(0, 8))) for _ in range(n)]
        for q in range(n):
            grads[q].copy_(torch.from_numpy(vals[q]).to(tdt))
        gnp = [np.ascontiguousarray(to_np(g)) for g in grads]
        w0 = rng.normal(0, 0.02, se).astype(np.float32)
        W = dev_buffer(se, torch.float32, shift=int(rng.integers(0, 4)))
        W.copy_(torch.from_numpy(w0))
        M, V = torch.zeros(se, device=DEV), torch.zeros(se, device=DEV)
        out = torch.zeros(se, dtype=torch.int16, device=DEV)
        g_red = torch.empty(se, dtype=torch.float32, device=DEV)
        ws = torch.zeros(max(z.zero_gradnorm_workspace_bytes(L, rank) // 8, 1), dtype=torch.float64,
                         device=DEV)
        ss = torch.zeros(1, dtype=torch.float64, device=DEV)
        coef = torch.zeros(1, dtype=torch.float32, device=DEV)
        z.zero_gradnorm_async(L, rank, grads, gidx, float(n), g_red, sidx, ws, ss)
        z.zero_clip_coef_async(ss, 1.0, coef)
        z.zero_step_device_clip(L, rank, [g_red], sidx, 1.0, W, M, V, sidx, out, sidx, scalars(1, h),
                                coef)
        torch.cuda.synchronize()
        if rank < 0:
            og = np.zeros(se, np.float32)
            for r in range(n):
                ks = oracle.reduced_grad(n, numel, r, gnp, grad_local=False, divisor=float(n))
                og[[O.global_of_local(r, k) for k in range(L.shard)]] = ks
        else:
            og = oracle.reduced_grad(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n))
        ocoef = oracle.clip_coef(oracle.sumsq(og), 1.0)
        assert float(coef.item()) == ocoef, (case, float(coef.item()), ocoef)
        # clipping is active unless the selection is all padding (g = 0, c = 1)
        assert (ocoef < 1.0) == bool(og.any()), (case, ocoef)
        om, omm, ov, oo = w0.copy(), np.zeros(se, np.float32), np.zeros(se, np.float32), np.zeros(se, np.uint16)
        if rank < 0:
            oracle.zero_step_all(n, numel, gnp, divisor=float(n), clip=ocoef, master=om, m=omm, v=ov,
                                 out=oo, t=1, **hyper_args(h))
        else:
            oracle.zero_step_rank(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n),
                                  clip=ocoef, master=om, m=omm, v=ov, state_global=False, out=oo,
                                  out_gather=False, t=1, **hyper_args(h))
        tag = f"case {case}"
        assert_same_f32(to_np(W), om, "master " + tag)
        assert_same_f32(to_np(M), omm, "m " + tag)
        assert_same_f32(to_np(V), ov, "v " + tag)
        assert_same_bf16(to_np(out), oo, "out " + tag)
