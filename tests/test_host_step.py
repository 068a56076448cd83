"""The offload step on host cores (zero_step_host) against the oracle, bit
for bit: every index mode, rank, rank count, gradient dtype and thread count,
unaligned buffers, NaN / Inf, padding, empty selections.  CPU only."""
import numpy as np
import pytest

import oracle
import pins

z = pytest.importorskip("fsdp_sharded_optimizer_flat_amd")
G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
H = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)


def sc(t, clip=1.0):
    return z.zero_adamw_scalars_for(t, H["lr"], H["b1"], H["b2"], H["eps"], H["wd"], clip)


def shifted(n, dtype, shift):
    """A C-contiguous view of n elements starting `shift` elements into a
    larger array (unaligned for the 8-wide vector loop)."""
    return np.zeros(n + shift, dtype)[shift:]


def run_case(rng, n, numel, rank, bf, gidx, sidx, oidx, threads, shift=0, steps=2, clip=1.0,
             special=False, n_grads=None):
    L = z.zero_pack(n, numel)
    O = oracle.Layout(n, numel)
    ng = n if n_grads is None else n_grads
    ge = L.padded if gidx == G else L.shard
    se = L.padded if sidx == G else L.shard
    oe = L.padded if oidx == G else L.shard
    w = shifted(se, np.float32, shift)
    w[:] = rng.normal(0, 0.02, se).astype(np.float32)
    if special and se > 8:
        w[3], w[5] = np.nan, np.inf
    m, v = shifted(se, np.float32, shift), shifted(se, np.float32, shift)
    out = shifted(oe, np.uint16, (shift * 3) % 5)
    om, omm, ov, oo = w.copy(), m.copy(), v.copy(), out.copy()
    for t in range(1, steps + 1):
        gs = []
        for q in range(ng):
            vals = (rng.standard_normal(ge) * 1e-3).astype(np.float32)
            if special and ge > 8:
                vals[q % 7] = [np.nan, np.inf, -np.inf, 3e38, -0.0, 1e-45, 0.0][q % 7]
            g = shifted(ge, np.uint16 if bf else np.float32, (shift + q) % 3)
            g[:] = oracle.bf16(vals) if bf else vals
            gs.append(g)
        z.zero_step_host(L, rank, gs, gidx, float(n), w, m, v, sidx, out, oidx, sc(t, clip), threads)
        gc = [np.ascontiguousarray(g) for g in gs]
        if rank < 0:
            oracle.zero_step_all(n, numel, gc, divisor=float(n), clip=clip, master=om, m=omm, v=ov,
                                 out=oo, t=t, **H)
        else:
            oracle.zero_step_rank(n, numel, rank, gc, grad_local=(gidx == Lc), divisor=float(n),
                                  clip=clip, master=om, m=omm, v=ov, state_global=(sidx == G),
                                  out=oo, out_gather=(oidx == G), t=t, **H)
    tag = f"n={n} numel={numel} rank={rank} bf={bf} idx={gidx}{sidx}{oidx} thr={threads} shift={shift}"
    for a, b, name in ((w, om, "master"), (m, omm, "m"), (v, ov, "v")):
        an, bn = np.isnan(a), np.isnan(b)
        assert np.array_equal(an, bn), name + " NaN " + tag
        assert np.array_equal(a[~an].view(np.uint32), b[~bn].view(np.uint32)), name + " " + tag
    onan = (out & 0x7FFF) > 0x7F80
    assert np.array_equal(onan, (oo & 0x7FFF) > 0x7F80), "out NaN " + tag
    assert np.array_equal(out[~onan], oo[~onan]), "out " + tag


def test_host_step_index_modes_bruteforce():
    rng = np.random.default_rng(21)
    for n in (1, 2, 3, 4, 8):
        for numel in ([37], [64, 5, 0, 19], [8 * n + 3, 16 * n]):
            for bf in (True, False):
                for rank in [-1] + sorted({0, n - 1, n // 2}):
                    modes = [(G, G, G)] if rank < 0 else [(gi, si, oi) for gi in (G, Lc) for si in (G, Lc) for oi in (G, Lc)]
                    for gidx, sidx, oidx in modes:
                        run_case(rng, n, numel, rank, bf, gidx, sidx, oidx, threads=1,
                                 shift=int(rng.integers(0, 4)))


@pytest.mark.parametrize("threads", [1, 2, 3, 8, 0])
def test_host_step_threads_multi_chunk(threads):
    rng = np.random.default_rng(22)
    run_case(rng, 8, [300_007, 77, 4096 * 8 + 3], -1, True, G, G, G, threads)
    run_case(rng, 8, [300_007, 77, 4096 * 8 + 3], 5, True, G, Lc, G, threads, shift=1)


@pytest.mark.parametrize("n", [5, 16, 64, 256])
def test_host_step_rank_counts(n):
    rng = np.random.default_rng(n)
    run_case(rng, n, [n * 2048 + 9], 1, True, Lc, Lc, Lc, threads=4)


def test_host_step_nan_inf_and_clip():
    rng = np.random.default_rng(23)
    run_case(rng, 8, [4096 + 5], -1, True, G, G, G, threads=2, special=True)
    run_case(rng, 4, [1000], 2, False, Lc, Lc, Lc, threads=1, special=True, clip=0.4137)


def test_host_step_reduced_gradient_input():
    rng = np.random.default_rng(24)
    run_case(rng, 8, [4096 + 3], 2, False, Lc, Lc, Lc, threads=2, n_grads=1)


def test_host_step_toy():
    """The pages' toy through the host step: 50 steps, bit-exact."""
    n, P = 4, 1000
    L = z.zero_pack(n, [P])
    tgt = np.array([[(i * 7 + r * 13) % 11 for i in range(P)] for r in range(n)], np.float32)
    w = np.zeros(P, np.float32)
    m, v = np.zeros_like(w), np.zeros_like(w)
    out = np.zeros(P, np.uint16)
    for t in range(1, 51):
        gs = [np.ascontiguousarray(w - tgt[r]) for r in range(n)]
        s = z.zero_adamw_scalars_for(t, 0.01, 0.9, 0.95, 1e-8, 0.1)
        z.zero_step_host(L, -1, gs, G, float(n), w, m, v, G, out, G, s, 2)
    ws, wu, ob, _ = oracle.toy(n, P, 50, 0.01)
    assert np.array_equal(w.view(np.uint32), ws.view(np.uint32))
    assert np.array_equal(out, ob)


def test_host_step_empty_and_errors():
    L = z.zero_pack(4, [0])
    g = np.zeros(4, np.uint16)
    d = np.zeros(4, np.float32)
    z.zero_step_host(L, -1, [g], G, 4.0, d, d.copy(), d.copy(), G, None, G, sc(1))
    L = z.zero_pack(4, [16])
    w = np.zeros(16, np.float32)
    with pytest.raises(z.ZeroError) as e:          # a written buffer aliasing another
        z.zero_step_host(L, -1, [np.zeros(16, np.uint16)] * 4, G, 4.0, w, w, np.zeros(16, np.float32),
                         G, None, G, sc(1))
    assert e.value.status == z.ZERO_EINVAL
    with pytest.raises(z.ZeroError):               # LOCAL with every rank
        z.zero_step_host(L, -1, [np.zeros(4, np.uint16)] * 4, Lc, 4.0, np.zeros(4, np.float32),
                         np.zeros(4, np.float32), np.zeros(4, np.float32), Lc, None, Lc, sc(1))


def _order_cases():
    import f32exact as F
    for c in pins.golden("adamw_order.json")["cases"]:
        hp = [F.value_of(F.from_decimal(c["hyper"][k])) for k in ("lr", "b1", "b2", "eps", "wd")]
        vals = {k: np.uint32(int(c[k], 16)) for k in "wmvg"}
        exp = {k: int(x, 16) for k, x in c["expect"].items()}
        yield c, hp, vals, exp


@pytest.mark.parametrize("copies", [1, 67])
def test_adamw_order_golden_host(copies):
    """The host step on the elements whose bits each alternative association
    of the page's AdamW code would change (exact-arithmetic golden table);
    67 copies run the 8-wide vector loop as well as the scalar tail."""
    for c, hp, vals, exp in _order_cases():
        L = z.zero_pack(1, [copies])
        arr = {k: np.full(copies, vals[k], np.uint32).view(np.float32) for k in "wmvg"}
        s = z.zero_adamw_scalars_for(c["t"], *hp, 1.0)
        z.zero_step_host(L, 0, [arr["g"]], Lc, 1.0, arr["w"], arr["m"], arr["v"], Lc, None, Lc, s, 2)
        for k in "mvw":
            got = arr[k].view(np.uint32)
            assert np.all(got == exp[k]), (c, k, hex(int(got[0])))
