"""The step streamed unit by unit from transient gradient buckets
(zero_step_units): "ZeRO and FSDP sharding", How it works -- each unit's
gradients are reduce-scattered as backward produces them and its shards can be
stepped then; "ZeRO: Three Ledgers", section 4 -- bucketed reduce-scatter frees
each bucket, so gradients are transient.

- Moderate sizes: random layouts split into random unit ranges, each range
  stepped from its own bucket (a copy of that range's gradients at another
  alignment) on one of two streams, against the oracle's step of the whole
  layout, bit for bit; every index mode, bf16 and fp32 gradients, fused and
  staged paths.
- Full size (the GPT-2 Large model, 36 units, N = 8): a producer writes each
  unit's 8 gradient buckets into one of two recycled slots on the main stream,
  in backward order (last unit first), while a side stream steps the unit
  before it; events order the slot reuse.  Two steps, every element of
  master, m, v and the bf16 gather buffer against the oracle."""
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
from gpu_common import (DEV, assert_same_bf16, assert_same_f32, dev_buffer,  # noqa: E402
                        hyper_args, scalars, to_np)

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
H = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)


def log(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _random_ranges(rng, U):
    """A random split of units 0..U-1 into consecutive ranges (empty ranges
    included now and then), in a random order."""
    cuts = sorted(set(int(x) for x in rng.integers(0, U + 1, int(rng.integers(0, U + 1)))))
    edges = [0] + cuts + [U]
    ranges = [(a, b) for a, b in zip(edges[:-1], edges[1:])]
    if rng.random() < 0.3:
        ranges.append((int(rng.integers(0, U + 1)),) * 2)      # an empty range
    order = rng.permutation(len(ranges))
    return [ranges[i] for i in order]


def _case(rng, n, numel, rank, gdt, gidx, sidx, oidx, staged_ws=None, steps=2):
    L = z.zero_pack(n, numel)
    ext = lambda i: L.padded if i == G else L.shard
    ge, se, oe = ext(gidx), ext(sidx), ext(oidx)
    tdt = torch.bfloat16 if gdt == z.ZERO_BF16 else torch.float32
    master = dev_buffer(se, torch.float32, shift=int(rng.integers(0, 4)))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(oe, dtype=torch.int16, device=DEV)
    init = rng.normal(0, 0.02, se).astype(np.float32)
    master.copy_(torch.from_numpy(init))
    om, omm, ov = init.copy(), np.zeros(se, np.float32), np.zeros(se, np.float32)
    oout = np.zeros(oe, np.uint16)
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    ws = None
    if staged_ws:
        ws = torch.empty(staged_ws, dtype=torch.float32, device=DEV)
    for t in range(1, steps + 1):
        full = [torch.from_numpy((rng.standard_normal(ge) * 1e-3).astype(np.float32)).to(DEV).to(tdt)
                for _ in range(n)]
        synth_pad = L.unit_table()
        if gidx == G:
            for g in full:
                synth.zero_padding_(g, synth_pad)
        gnp = [np.ascontiguousarray(to_np(g)) for g in full]
        ranges = _random_ranges(rng, L.n_units)
        for i, (a, b) in enumerate(ranges):
            lo, hi = (int(x) for x in (np.r_[0, np.cumsum(L.unit_table()[:, 1 if gidx == G else 2])][[a, b]]))
            shift = int(rng.integers(0, 8))
            buckets = [dev_buffer(hi - lo, tdt, shift=shift) for _ in range(n)]
            for bk, g in zip(buckets, full):
                bk.copy_(g[lo:hi])
            st = side if i % 2 else main
            ev = torch.cuda.Event()
            ev.record(main)
            st.wait_event(ev)
            z.zero_step_units(L, rank, a, b, buckets, gidx, float(n), master, m, v, sidx, out, oidx,
                              scalars(t, H), ws, stream=st)
            done = torch.cuda.Event()
            done.record(st)
            main.wait_event(done)
        torch.cuda.synchronize()
        if rank < 0:
            oracle.zero_step_all(n, numel, gnp, divisor=float(n), clip=1.0, master=om, m=omm, v=ov,
                                 out=oout, t=t, **hyper_args(H))
        else:
            oracle.zero_step_rank(n, numel, rank, gnp, grad_local=(gidx == Lc), divisor=float(n),
                                  clip=1.0, master=om, m=omm, v=ov, state_global=(sidx == G),
                                  out=oout, out_gather=(oidx == G), t=t, **hyper_args(H))
    tag = f"n={n} numel={numel} rank={rank} idx={gidx}{sidx}{oidx} staged={staged_ws}"
    assert_same_f32(to_np(master), om, "master " + tag)
    assert_same_f32(to_np(m), omm, "m " + tag)
    assert_same_f32(to_np(v), ov, "v " + tag)
    assert_same_bf16(to_np(out), oout, "out " + tag)


def test_step_units_random_splits():
    rng = np.random.default_rng(2024)
    cases = 0
    for trial in range(24):
        n = int(rng.choice([1, 3, 8, 5, 40, 64]))
        U = int(rng.integers(1, 7))
        numel = [int(x) for x in rng.integers(0, 3000, U)]
        numel[int(rng.integers(0, U))] += n * 700       # a few tiles somewhere
        gdt = z.ZERO_BF16 if rng.random() < 0.7 else z.ZERO_F32
        rank = -1 if rng.random() < 0.35 else int(rng.integers(0, n))
        modes = [(G, G, G)] if rank < 0 else [(Lc, Lc, Lc), (G, Lc, G), (Lc, G, Lc)]
        gidx, sidx, oidx = modes[int(rng.integers(0, len(modes)))]
        staged = int(rng.choice([512, 2048])) if n > 24 and rng.random() < 0.7 else None
        _case(rng, n, numel, rank, gdt, gidx, sidx, oidx, staged)
        cases += 1
    log(f"unit-range cases: {cases}")


def test_step_units_argument_checks():
    L = z.zero_pack(4, [100, 50])
    g = [torch.zeros(L.padded, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    st = [torch.zeros(L.padded, device=DEV) for _ in range(3)]
    out = torch.zeros(L.padded, dtype=torch.int16, device=DEV)
    for a, b in ((-1, 1), (1, 0), (0, 3)):
        with pytest.raises(ValueError):
            z.zero_step_units(L, -1, a, b, g, G, 4.0, *st, G, out, G, scalars(1, H))
    # a bucket shorter than the range is refused
    with pytest.raises(ValueError):
        z.zero_step_units(L, -1, 0, 1, [x[:99] for x in g], G, 4.0, *st, G, out, G, scalars(1, H))
    # the raw C call checks the range too (no launch)
    lib = z.raw_library()
    import ctypes as C
    arr = (C.c_void_p * 4)(*[x.data_ptr() for x in g])
    s = scalars(1, H)
    rc = lib.zero_step_units(C.c_void_p(L.ptr), -1, 1, 3, C.c_void_p(C.addressof(arr)), 4, z.ZERO_BF16, G,
                             C.c_float(4.0), C.c_void_p(st[0].data_ptr()), C.c_void_p(st[1].data_ptr()),
                             C.c_void_p(st[2].data_ptr()), G, C.c_void_p(out.data_ptr()), G, C.byref(s),
                             None, 0, None)
    assert rc == z.ZERO_EINVAL
    torch.cuda.synchronize()
    assert all(torch.all(x == 0) for x in st)


def test_gpt2l_streamed_every_element():
    wl = WORKLOADS["gpt2l"]
    n, h = wl.n_ranks, wl.hyper
    L = z.zero_pack(n, wl.unit_numel)
    T = L.unit_table()
    U, P = L.n_units, L.padded
    cap = int(T[:, 1].max())
    log(f"streamed gpt2l: N={n}, {U} units, P^={P}, two slots of {n} x {cap} bf16")
    master = torch.empty(P, dtype=torch.float32, device=DEV)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(P, dtype=torch.int16, device=DEV)
    slots = torch.empty(2, n, cap, dtype=torch.bfloat16, device=DEV)
    wh, mh, vh = to_np(master).copy(), np.zeros(P, np.float32), np.zeros(P, np.float32)
    oh = np.zeros(P, np.uint16)
    gh = [np.zeros(P, np.uint16) for _ in range(n)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def seed(t, r, u):
        return synth.seed_of(wl.seed * 1000 + u, synth.TAG_GRAD, t, r)

    def produce(t, u, slot):
        # backward's stand-in: the unit's N gradient buckets, written on the
        # main stream
        pad = int(T[u, 1])
        for r in range(n):
            synth.fill_grad_(slots[slot, r, :pad], wl.grad_dist, wl.grad_scale, seed(t, r, u))

    for t in (1, 2):
        order = list(range(U - 1, -1, -1))          # backward: last unit first
        stepped = [None] * U
        for i, u in enumerate(order):
            slot = i % 2
            if i >= 2:
                main.wait_event(stepped[i - 2])      # the slot's previous unit is stepped
            produce(t, u, slot)
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
            pad = int(T[u, 1])
            z.zero_step_units(L, -1, u, u + 1, [slots[slot, r, :pad] for r in range(n)], G, float(n),
                              master, m, v, G, out, G, scalars(t, h), stream=side)
            stepped[i] = torch.cuda.Event()
            stepped[i].record(side)
        main.wait_event(stepped[-1])
        torch.cuda.synchronize()
        # the same gradients, regenerated unit by unit for the oracle
        for u in range(U):
            produce(t, u, 0)
            off, pad = int(T[u, 3]), int(T[u, 1])
            for r in range(n):
                gh[r][off:off + pad] = to_np(slots[0, r, :pad])

        def oracle_unit(u):
            numel, off, pad = int(T[u, 0]), int(T[u, 3]), int(T[u, 1])
            oracle.zero_step_all(n, [numel], [g[off:off + pad] for g in gh], divisor=float(n), clip=1.0,
                                 master=wh[off:off + pad], m=mh[off:off + pad], v=vh[off:off + pad],
                                 out=oh[off:off + pad], t=t, **hyper_args(h))
        with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(oracle_unit, range(U)))
        log(f"streamed gpt2l: step {t} done on the GPU and in the oracle")
    assert_same_f32(to_np(master), wh, "streamed master")
    assert_same_f32(to_np(m), mh, "streamed m")
    assert_same_f32(to_np(v), vh, "streamed v")
    assert_same_bf16(to_np(out), oh, "streamed out")
    log(f"streamed gpt2l: all {P} elements bit-exact after 2 steps")
