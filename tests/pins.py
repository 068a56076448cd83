"""Pins: checks that tie the oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix: values the pages print, closed forms,
library routines that compute the same definition (torch's AdamW in binary64,
torch's bf16 cast, ``math.fsum``, ``clip_grad_norm_``), brute force on tiny
inputs, and the pages' own invariant (sharded == unsharded, bit for bit).

They are plain functions (not tests) so that the mutation tests can run every
pin against a copy of the oracle with a planted mistake and show that at least
one pin fails.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f32(x) -> float:
    return float(np.float32(x))


def bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ---------------------------------------------------------------------------
# Layout: brute force against an explicit construction of the padded buffer.
# ---------------------------------------------------------------------------

def brute_layout(n, numel):
    """Build the padded flat buffer and the ranks' local shards by listing
    elements, exactly as the words say: pad each unit to a multiple of n, cut
    it into n equal slices, rank r keeps slice r of every unit in unit order."""
    flat = []              # entries: (unit, i) or None for padding
    starts = []
    local = [[] for _ in range(n)]
    for u, p in enumerate(numel):
        unit = [(u, i) for i in range(p)]
        while len(unit) % n:
            unit.append(None)
        starts.append(len(flat))
        base = len(flat)
        flat.extend(unit)
        s = len(unit) // n
        for r in range(n):
            for i in range(s):
                local[r].append(base + r * s + i)    # a position in flat
    return flat, starts, local


def pin_layout_bruteforce(seed=0, cases=400):
    rng = np.random.default_rng(seed)
    combos = [(n, [p]) for n in range(1, 10) for p in range(0, 40)]
    for _ in range(cases):
        n = int(rng.integers(1, 10))
        U = int(rng.integers(1, 5))
        combos.append((n, [int(x) for x in rng.integers(0, 65, size=U)]))
    for n, numel in combos:
        flat, starts, local = brute_layout(n, numel)
        L = oracle.Layout(n, numel)
        assert L.total_padded == len(flat), (n, numel)
        assert L.total_shard == len(local[0]), (n, numel)
        for u, p in enumerate(numel):
            assert L.padded[u] % n == 0 and 0 <= L.padded[u] - p < n, (n, numel)
            assert L.offset[u] == starts[u], (n, numel, u)
            assert L.shard[u] * n == L.padded[u]
        loc_pos = 0
        for u in range(len(numel)):
            assert L.local_offset[u] == loc_pos
            loc_pos += int(L.shard[u])
        for r in range(n):
            for k, j in enumerate(local[r]):
                assert L.global_of_local(r, k) == j, (n, numel, r, k)
                assert L.owner_of_global(j) == (r, k), (n, numel, j)


# ---------------------------------------------------------------------------
# Row-aligned layout: FSDP2 chunks each parameter on dim 0 with torch.chunk
# and pads every rank's piece to the first chunk's row count ("Learn: ZeRO &
# FSDP", section 5, FSDP1 vs FSDP2).  Reshard: a checkpoint saved as per-rank
# shards is re-cut for another N ("ZeRO and FSDP sharding", Implementation
# notes).  Both are pinned to explicit constructions that share nothing with
# the oracle's index maps.
# ---------------------------------------------------------------------------

def fsdp2_local_shards(params, n):
    """Rank r's local shard as FSDP2 lays it out: for each parameter in order,
    torch.chunk(param, n, dim=0)[r] (empty where chunk returns fewer pieces),
    zero-padded to the first chunk's row count, flattened; concatenated."""
    import torch
    shards = []
    for r in range(n):
        parts = []
        for p in params:
            chunks = torch.chunk(p, n, dim=0)
            c = chunks[0].shape[0] if p.shape[0] else 0
            piece = chunks[r] if r < len(chunks) and p.shape[0] else p[:0]
            pad = torch.zeros((c - piece.shape[0],) + tuple(p.shape[1:]), dtype=p.dtype)
            parts.append(torch.cat([piece, pad]).reshape(-1))
        shards.append(torch.cat(parts).numpy() if parts else np.zeros(0))
    return shards


def flat_local_shards(params, n, groups=None):
    """Rank r's local shard of the flat layout, from brute_layout's listing.
    groups: how many consecutive parameters each unit holds (default one)."""
    vals = [np.asarray(p).reshape(-1) for p in params]
    groups = groups or [1] * len(vals)
    units, at = [], 0
    for g in groups:
        units.append(np.concatenate(vals[at:at + g]) if g else np.zeros(0))
        at += g
    flat, _, local = brute_layout(n, [len(v) for v in units])
    dt = vals[0].dtype if vals else np.float64
    return [np.array([0 if flat[j] is None else units[flat[j][0]][flat[j][1]] for j in local[r]],
                     dtype=dt) for r in range(n)]


def random_groups(rng, U):
    """A random split of U parameters into consecutive units (FSDP1-style
    blocks), empty units included now and then."""
    groups, left = [], U
    while left:
        g = int(rng.integers(0, left + 1))
        groups.append(g)
        left -= g
    return groups


def layout_case(rng, params, numel, row_len, n):
    """A random layout of the parameters: per-parameter rows (FSDP2),
    per-parameter flat, or flat blocks of several parameters (FSDP1).
    Returns (shards by explicit construction, unit numels, row lengths)."""
    kind = int(rng.integers(0, 3))
    if kind == 0:
        return fsdp2_local_shards(params, n), numel, row_len
    if kind == 1:
        return flat_local_shards(params, n), numel, None
    groups = random_groups(rng, len(params))
    units, at = [], 0
    for g in groups:
        units.append(sum(numel[at:at + g]))
        at += g
    return flat_local_shards(params, n, groups), units, None


def random_params(rng, U, max_rows=13, max_cols=5):
    """U parameters with unique nonzero values (so zero marks padding only):
    2-D (rows, cols), or 1-D (row length 1); rows may be 0."""
    import torch
    shapes = []
    for _ in range(U):
        rows = int(rng.integers(0, max_rows + 1))
        shapes.append((rows,) if rng.random() < 0.3 else (rows, int(rng.integers(1, max_cols + 1))))
    total = sum(int(np.prod(s)) for s in shapes)
    vals = torch.arange(1, total + 1, dtype=torch.float64)
    params, at = [], 0
    for s in shapes:
        k = int(np.prod(s))
        params.append(vals[at:at + k].reshape(s))
        at += k
    row_len = [int(np.prod(s[1:])) if len(s) > 1 else 1 for s in shapes]
    return params, [int(np.prod(s)) for s in shapes], row_len


def shards_from_layout(L, params, n):
    """Every rank's local shard read through the oracle's own index maps."""
    vals = [np.asarray(p).reshape(-1) for p in params]
    out = []
    for r in range(n):
        v = np.zeros(L.total_shard)
        for k in range(L.total_shard):
            j = L.global_of_local(r, k)
            u = next(u for u in range(L.n_units) if L.offset[u] <= j < L.offset[u] + L.padded[u])
            pos = j - L.offset[u]
            if pos < L.numel[u]:
                v[k] = vals[u][pos]
        out.append(v)
    return out


def pin_rows_vs_torch_chunk(seed=0, cases=150):
    rng = np.random.default_rng(seed)
    for case in range(cases):
        n = int(rng.integers(1, 10))
        params, numel, row_len = random_params(rng, int(rng.integers(1, 5)))
        L = oracle.Layout(n, numel, row_len=row_len)
        want = fsdp2_local_shards(params, n)
        assert L.total_shard == len(want[0]), (case, n, numel, row_len)
        assert L.total_padded == n * L.total_shard
        got = shards_from_layout(L, params, n)
        for r in range(n):
            assert np.array_equal(got[r], want[r]), (case, n, numel, row_len, r)


def pin_reshard(seed=0, cases=80):
    """Reshard between random layouts (rows, flat, flat blocks; any N) equals
    the destination layout's explicit construction, for 4- and 2-byte
    elements; resharding to one flat rank gives the parameters themselves."""
    rng = np.random.default_rng(seed)
    for case in range(cases):
        params, numel, row_len = random_params(rng, int(rng.integers(1, 6)))
        n_a, n_b = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        src, units_a, row_a = layout_case(rng, params, numel, row_len, n_a)
        want, units_b, row_b = layout_case(rng, params, numel, row_len, n_b)
        dt = np.float32 if case % 2 == 0 else np.uint16
        src = [x.astype(dt) for x in src]
        for r in range(n_b):
            got = oracle.reshard(units_a, n_a, src, n_b, r, row_a=row_a, row_b=row_b,
                                 numel_b=units_b)
            assert got.dtype == dt and np.array_equal(got, want[r].astype(dt)), \
                (case, n_a, n_b, units_a, units_b, row_a, row_b, r)
        whole = oracle.reshard(units_a, n_a, src, 1, 0, row_a=row_a, numel_b=[sum(numel)])
        cat = np.concatenate([np.asarray(p).reshape(-1) for p in params]).astype(dt)
        assert np.array_equal(whole, cat), (case, "gather to one rank")


# ---------------------------------------------------------------------------
# bf16 rounding: torch's float32 -> bfloat16 conversion rounds to nearest even.
# ---------------------------------------------------------------------------

def bf16_probe_patterns(seed=0, n_random=1 << 20):
    """Every upper half-word with the low half-words that decide rounding (0,
    1, just below / at / just above the midpoint, all ones), plus random ones."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xC000, 0xFFFE, 0xFFFF], np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rng = np.random.default_rng(seed)
    rnd = rng.integers(0, 1 << 32, size=n_random, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd])


def torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_bf16_vs_torch(seed=0, patterns=None):
    pats = bf16_probe_patterns(seed) if patterns is None else patterns
    x = pats.view(np.float32)
    ours = oracle.bf16(x)
    ref = torch_bf16_bits(x)
    nan = np.isnan(x)
    assert np.all(np.isnan(oracle.bf16_to_f32(ours[nan]))), "NaN must stay NaN"
    bad = np.nonzero(ours[~nan] != ref[~nan])[0]
    assert bad.size == 0, f"bf16 mismatch at {pats[~nan][bad[:5]]!r}"


# ---------------------------------------------------------------------------
# AdamW against torch.optim.AdamW in binary64 (a library implementation of the
# same definition: decoupled weight decay, bias corrections 1 - b1^t and
# sqrt(1 - b2^t)).
# ---------------------------------------------------------------------------

HYPER_SETS = [
    # (lr, b1, b2, eps, wd): the toy's, the GPT runs', and sets that make
    # eps, weight decay and the betas each matter.
    (0.01, 0.9, 0.95, 1e-8, 0.1),
    (3e-4, 0.9, 0.95, 1e-8, 0.1),
    (1e-3, 0.8, 0.99, 5e-4, 0.5),
    (2e-3, 0.5, 0.9, 1e-6, 2.0),
]


def pin_adamw_vs_torch64(seed=0, P=4096, steps=12):
    import torch
    rng = np.random.default_rng(seed)
    for hp in HYPER_SETS:
        lr, b1, b2, eps, wd = (f32(x) for x in hp)
        w0 = rng.normal(0, 0.02, P).astype(np.float32)
        w = w0.copy()
        m = np.zeros(P, np.float32)
        v = np.zeros(P, np.float32)
        p64 = torch.nn.Parameter(torch.from_numpy(w0.astype(np.float64)))
        opt = torch.optim.AdamW([p64], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd,
                                foreach=False, fused=False)
        gmax = 0.0
        for t in range(1, steps + 1):
            scale = 10.0 ** rng.uniform(-4, -1)
            g = (rng.standard_normal(P) * scale).astype(np.float32)
            gmax = max(gmax, float(np.abs(g).max()))
            oracle.adamw_vector(w, m, v, g, t, lr, b1, b2, eps, wd)
            p64.grad = torch.from_numpy(g.astype(np.float64))
            opt.step()
            ref_w = p64.detach().numpy()
            st = opt.state[p64]
            ref_m = st["exp_avg"].numpy()
            ref_v = st["exp_avg_sq"].numpy()
            # Error budget: every binary32 operation adds at most 2^-24 relative
            # error; per step the update is bounded by lr * (1-b1)/sqrt(1-b2) *
            # (1 + small), and errors accumulate at most linearly in t.
            eps32 = 2.0 ** -24
            upd_bound = lr * (1 - b1) / math.sqrt(1 - b2) * 4 + lr
            tol_w = t * 16 * eps32 * (np.abs(ref_w) + upd_bound)
            assert np.all(np.abs(w - ref_w) <= tol_w), (hp, t, float(np.max(np.abs(w - ref_w) - tol_w)))
            tol_m = t * 8 * eps32 * (np.abs(ref_m) + gmax)
            assert np.all(np.abs(m - ref_m) <= tol_m), (hp, t, "m")
            tol_v = t * 8 * eps32 * (np.abs(ref_v) + gmax * gmax)
            assert np.all(np.abs(v - ref_v) <= tol_v), (hp, t, "v")


def pin_adamw_order():
    """The association of the AdamW update that the page's code fixes ("ZeRO and
    FSDP sharding", Code: `(1.0 - b2) * g[i] * g[i]`, `lr / bc1 * m / (v.sqrt()
    / bc2 + eps)`), on elements whose bits change under each alternative
    association.  Expected bits come from tests/golden/adamw_order.json, written
    by exact rational arithmetic with one binary32 rounding per operation
    (tests/golden/make_adamw_order.py), not by the oracle."""
    import f32exact as F
    gold = golden("adamw_order.json")
    seen = set()
    for c in gold["cases"]:
        hp = [F.value_of(F.from_decimal(c["hyper"][k])) for k in ("lr", "b1", "b2", "eps", "wd")]
        w, m, v, g = (np.array([int(c[k], 16)], np.uint32).view(np.float32) for k in "wmvg")
        oracle.adamw_vector(w, m, v, g, c["t"], *hp)
        got = {"m": int(bits(m)[0]), "v": int(bits(v)[0]), "w": int(bits(w)[0])}
        exp = {k: int(x, 16) for k, x in c["expect"].items()}
        assert got == exp, (c, {k: hex(x) for k, x in got.items()})
        seen.update(c["alternatives_that_differ"])
    assert seen >= {"v_assoc", "u_assoc", "den_recip", "den_sqrt"}, seen


def pin_scalars(t_max=3000):
    """b^t as a running binary32 product (numpy's sequential float32 cumprod),
    and the closed forms of the bias corrections in binary64."""
    for (lr, b1, b2, _eps, wd) in HYPER_SETS:
        lr, b1, b2, wd = f32(lr), f32(b1), f32(b2), f32(wd)
        p1 = np.cumprod(np.full(t_max, b1, np.float32), dtype=np.float32)
        p2 = np.cumprod(np.full(t_max, b2, np.float32), dtype=np.float32)
        for t in (1, 2, 3, 4, 7, 10, 100, 1000, t_max):
            s = oracle.adamw_scalars(t, lr, b1, b2, wd)
            assert s["pow1"] == p1[t - 1] and s["pow2"] == p2[t - 1], (t, b1, b2)
            e = 2.0 ** -24
            bc1 = 1 - b1 ** t
            bc2 = math.sqrt(1 - b2 ** t)
            assert abs(s["bc1"] - bc1) <= (t + 2) * 2 * e * max(bc1, b1 ** t) + 1e-45, (t, "bc1")
            assert abs(s["bc2"] - bc2) <= (t + 2) * 2 * e * max(1.0, b2 ** t / bc2 ** 2) * bc2 + 1e-45, (t, "bc2")
            assert abs(s["lr_over_bc1"] - lr / bc1) <= (t + 4) * 2 * e * lr / bc1 * max(1.0, b1 ** t / bc1), (t, "a")
            assert abs(s["decay"] - (1 - lr * wd)) <= 4 * e, "decay"
            assert s["one_minus_b1"] == f32(np.float32(1) - np.float32(b1))


# ---------------------------------------------------------------------------
# The pages' invariant: sharded == unsharded, bit for bit (also at P % N != 0,
# with several units, bf16 and fp32 gradients and rank counts 1, 2, 4, 8).
# ---------------------------------------------------------------------------

def make_grads(rng, n, P, bf16=True, scale=1e-3):
    gs = []
    for _ in range(n):
        g = (rng.standard_normal(P) * scale).astype(np.float32)
        gs.append(oracle.bf16(g) if bf16 else g)
    return gs


def pack_global(L, vectors_per_unit, dtype):
    """Place per-unit vectors into a padded flat buffer (zeros in padding)."""
    flat = np.zeros(L.total_padded, dtype)
    for u, vec in enumerate(vectors_per_unit):
        flat[L.offset[u]:L.offset[u] + len(vec)] = vec
    return flat


def pin_sharded_equals_unsharded(seed=0, steps=4):
    rng = np.random.default_rng(seed)
    hp = dict(lr=f32(1e-3), b1=f32(0.9), b2=f32(0.95), eps=f32(1e-8), wd=f32(0.1))
    cases = [(n, numel, bf) for n in (1, 2, 4, 8) for numel in ([1000], [1001, 37, 64, 5]) for bf in (True, False)]
    cases += [(3, [10, 11, 12], True), (7, [1, 0, 50], True)]
    for n, numel, bf in cases:
        L = oracle.Layout(n, numel)
        P = sum(numel)
        w_flat = rng.normal(0, 0.02, P).astype(np.float32)
        # sharded: every rank's slice of a padded flat buffer
        units_w = np.split(w_flat, np.cumsum(numel)[:-1])
        master = pack_global(L, units_w, np.float32)
        m = np.zeros_like(master)
        v = np.zeros_like(master)
        out = np.zeros(L.total_padded, np.uint16)
        wu = w_flat.copy()
        mu = np.zeros(P, np.float32)
        vu = np.zeros(P, np.float32)
        for t in range(1, steps + 1):
            gs = make_grads(rng, n, P, bf16=bf)
            gdt = np.uint16 if bf else np.float32
            gflat = [pack_global(L, np.split(g, np.cumsum(numel)[:-1]), gdt) for g in gs]
            oracle.zero_step_all(n, numel, gflat, divisor=float(n), clip=1.0, master=master, m=m, v=v,
                                 out=out, t=t, **hp)
            oracle.adamw_unsharded(gs, divisor=float(n), clip=1.0, w=wu, m=mu, v=vu, t=t, **hp)
        for u in range(len(numel)):
            a = master[L.offset[u]:L.offset[u] + numel[u]]
            b = np.split(wu, np.cumsum(numel)[:-1])[u]
            assert np.array_equal(bits(a), bits(b)), (n, numel, bf, u)
            pad = master[L.offset[u] + numel[u]:L.offset[u] + L.padded[u]]
            assert np.all(bits(pad) == 0), "padding must stay +0"
            assert np.array_equal(out[L.offset[u]:L.offset[u] + numel[u]], oracle.bf16(b))


def pin_rank_local_equals_global(seed=1):
    """A rank's step with LOCAL (reduce-scatter chunk) gradients and LOCAL
    state equals the same rank's slice of the all-ranks GLOBAL step."""
    rng = np.random.default_rng(seed)
    hp = dict(lr=f32(1e-3), b1=f32(0.9), b2=f32(0.95), eps=f32(1e-8), wd=f32(0.1))
    for n, numel in [(4, [9, 16, 3]), (8, [64, 100]), (3, [5])]:
        L = oracle.Layout(n, numel)
        gflat = [oracle.bf16(rng.standard_normal(L.total_padded).astype(np.float32) * 1e-3) for _ in range(n)]
        for g in gflat:   # zero the padding, as the packer does
            for u in range(len(numel)):
                g[L.offset[u] + numel[u]:L.offset[u] + L.padded[u]] = 0
        master0 = rng.normal(0, 0.02, L.total_padded).astype(np.float32)
        M, Mm, Mv = master0.copy(), np.zeros_like(master0), np.zeros_like(master0)
        out_all = np.zeros(L.total_padded, np.uint16)
        oracle.zero_step_all(n, numel, gflat, divisor=float(n), clip=1.0, master=M, m=Mm, v=Mv,
                             out=out_all, t=1, **hp)
        for r in range(n):
            idx = np.array([L.global_of_local(r, k) for k in range(L.total_shard)], np.int64)
            glocal = [np.ascontiguousarray(g[idx]) for g in gflat]
            ms = np.ascontiguousarray(master0[idx])
            mm = np.zeros_like(ms)
            vv = np.zeros_like(ms)
            o = np.zeros(L.total_shard, np.uint16)
            oracle.zero_step_rank(n, numel, r, glocal, grad_local=True, divisor=float(n), clip=1.0,
                                  master=ms, m=mm, v=vv, state_global=False, out=o, out_gather=False,
                                  t=1, **hp)
            assert np.array_equal(bits(ms), bits(M[idx])), (n, numel, r)
            assert np.array_equal(bits(vv), bits(Mv[idx]))
            assert np.array_equal(o, out_all[idx])


def pin_reduced_grad(seed=5):
    """The averaged gradient of a rank's shard (the reduction half of the
    reduce-scatter, then the division by N: "ZeRO and FSDP sharding", Code).

    - Exact case: dyadic gradients whose rank sums are exact in binary32; the
      mean is then fl(sum / N), one rounding of an exactly known rational,
      read at the brute-force listing's positions (tests/f32exact.py).
    - Both index spaces: a rank's reduce-scatter chunks (LOCAL, cut from the
      full gradients by the brute-force listing) give the same g as the full
      gradients (GLOBAL).
    - Tied to the pinned step: the step on the N gradients equals, bit for bit,
      the step on the one reduced gradient with divisor 1."""
    import f32exact as F
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    hp = dict(lr=f32(1e-3), b1=f32(0.9), b2=f32(0.95), eps=f32(1e-8), wd=f32(0.1))
    for n in (1, 3, 8):
        for trial in range(4):
            U = int(rng.integers(1, 4))
            numel = [int(x) for x in rng.integers(0, 40, U)]
            numel[0] = max(numel[0], 1)
            L = oracle.Layout(n, numel)
            flat, _, local = brute_layout(n, numel)
            real = np.array([e is not None for e in flat], bool)
            for bf in (True, False):
                # dyadic integers a * 2^-12 with |a| <= 200: bf16-exact, and
                # any sum of up to 8 of them is exact in binary32
                ints = [np.where(real, rng.integers(-200, 201, len(flat)), 0) for _ in range(n)]
                dyad = [(a * 2.0 ** -12).astype(np.float32) for a in ints]
                gglob = [oracle.bf16(x) if bf else x for x in dyad]
                for r in range(n):
                    pos = np.array(local[r], np.int64)
                    gloc = [np.ascontiguousarray(g[pos]) for g in gglob]
                    got_g = oracle.reduced_grad(n, numel, r, gglob, grad_local=False, divisor=float(n))
                    got_l = oracle.reduced_grad(n, numel, r, gloc, grad_local=True, divisor=float(n))
                    assert np.array_equal(bits(got_g), bits(got_l)), (n, numel, r, "GLOBAL vs LOCAL")
                    tot = sum(a[pos] for a in ints)
                    exp = np.array([F.encode(Fraction(int(x), 4096 * n)) for x in tot], np.uint32)
                    assert np.array_equal(bits(got_g), exp), (n, numel, r, bf, "exact mean")
                    # the step on N gradients == the step on the reduced one
                    base = rng.normal(0, 0.02, L.total_shard).astype(np.float32)
                    st = [base.copy(), np.zeros_like(base), np.zeros_like(base)]
                    s1 = [base.copy(), np.zeros_like(base), np.zeros_like(base)]
                    o, o1 = np.zeros(L.total_shard, np.uint16), np.zeros(L.total_shard, np.uint16)
                    for t in (1, 2):
                        oracle.zero_step_rank(n, numel, r, gloc, grad_local=True, divisor=float(n), clip=1.0,
                                              master=st[0], m=st[1], v=st[2], state_global=False, out=o,
                                              out_gather=False, t=t, **hp)
                        oracle.zero_step_rank(n, numel, r, [got_l], grad_local=True, divisor=1.0, clip=1.0,
                                              master=s1[0], m=s1[1], v=s1[2], state_global=False, out=o1,
                                              out_gather=False, t=t, **hp)
                    for a, b in zip(st, s1):
                        assert np.array_equal(bits(a), bits(b)), (n, numel, r, "step on reduced g")
                    assert np.array_equal(o, o1)
    # random (not dyadic) gradients, GLOBAL vs LOCAL and vs the step
    for n, numel in [(3, [10, 11, 12]), (8, [64, 100, 3])]:
        L = oracle.Layout(n, numel)
        flat, _, local = brute_layout(n, numel)
        real = np.array([e is not None for e in flat], bool)
        gglob = [oracle.bf16(np.where(real, rng.standard_normal(len(flat)) * 1e-3, 0).astype(np.float32))
                 for _ in range(n)]
        for r in range(n):
            pos = np.array(local[r], np.int64)
            gloc = [np.ascontiguousarray(g[pos]) for g in gglob]
            got_g = oracle.reduced_grad(n, numel, r, gglob, grad_local=False, divisor=float(n))
            got_l = oracle.reduced_grad(n, numel, r, gloc, grad_local=True, divisor=float(n))
            assert np.array_equal(bits(got_g), bits(got_l)), (n, numel, r)
            base = rng.normal(0, 0.02, L.total_shard).astype(np.float32)
            st = [base.copy(), np.zeros_like(base), np.zeros_like(base)]
            s1 = [base.copy(), np.zeros_like(base), np.zeros_like(base)]
            oracle.zero_step_rank(n, numel, r, gloc, grad_local=True, divisor=float(n), clip=1.0,
                                  master=st[0], m=st[1], v=st[2], state_global=False, out=None,
                                  out_gather=False, t=1, **hp)
            oracle.zero_step_rank(n, numel, r, [got_g], grad_local=True, divisor=1.0, clip=1.0,
                                  master=s1[0], m=s1[1], v=s1[2], state_global=False, out=None,
                                  out_gather=False, t=1, **hp)
            for a, b in zip(st, s1):
                assert np.array_equal(bits(a), bits(b)), (n, numel, r)


# ---------------------------------------------------------------------------
# The pages' toy.
# ---------------------------------------------------------------------------

def pin_toy():
    gold = golden("toy_printed.json")
    n, P, steps, lr = gold["n"], gold["P"], gold["steps"], gold["lr"]
    ws, wu, ob, trace = oracle.toy(n, P, steps, lr)
    assert np.array_equal(bits(ws), bits(wu)), "sharded != unsharded"
    assert np.array_equal(ob, oracle.bf16(ws))
    # ledger line the toy prints
    assert 3 * P // n == gold["optimizer_floats_per_rank"] and 3 * P == gold["optimizer_floats_unsharded"]
    tbar = np.array([np.mean([(i * 7 + r * 13) % 11 for r in range(n)]) for i in range(P)])
    # convergence toward the rank-mean target: the distance falls every step,
    # and with Adam's step of about lr per element from w = 0 every element
    # stays strictly between 0 and its target after 50 steps.
    assert np.all(np.diff(trace) < 0), "mean |w - tbar| must fall every step"
    assert np.all(ws > 0) and np.all(ws < tbar), "0 < w_i < tbar_i"
    assert abs(trace[0] - (np.mean(tbar) - lr)) < 1e-4
    # step-1 closed form: from w0 = 0 the first update is
    # lr * ghat / (|ghat| + eps) = lr * tbar / (tbar + eps), i.e. lr to 1e-8 rel.
    w1, _, _, _ = oracle.toy(n, P, 1, lr)
    exact1 = lr * tbar / (tbar + 1e-8)
    assert np.all(np.abs(w1 - exact1) <= 8 * 2.0 ** -24 * lr), "step-1 closed form"
    # long run: converges to the rank-mean target (weight decay 0.1 shifts the
    # fixed point only by O(lr * wd * w / (update size)), here far below 1e-2).
    wl, _, _, _ = oracle.toy(n, P, 3000, lr)
    assert np.max(np.abs(wl - tbar)) < 1e-2


# ---------------------------------------------------------------------------
# Gradient norm and clip coefficient.
# ---------------------------------------------------------------------------

def pin_norm(seed=0):
    import torch
    rng = np.random.default_rng(seed)
    # closed form: a constant gradient c over n elements has sum of squares n c^2
    for c, n in [(0.5, 1 << 20), (3.0, 12345), (2.0 ** -20, 77)]:
        g = np.full(n, c, np.float32)
        assert oracle.sumsq(g) == n * c * c
    # random heavy-tailed data: within 1e-13 of the exactly rounded sum
    for n in (1, 1000, 1 << 18):
        g = (rng.standard_t(3, n) * 1e-3).astype(np.float32)
        exact = math.fsum(float(x) * float(x) for x in g.astype(np.float64))
        got = oracle.sumsq(g)
        assert abs(got - exact) <= 1e-13 * exact + 1e-300, (n, got, exact)
        # clip coefficient vs torch's clip_grad_norm_ in binary64
        for max_norm in (1.0, 1e-3, 1e3):
            p = torch.nn.Parameter(torch.zeros(n, dtype=torch.float64))
            p.grad = torch.from_numpy(g.astype(np.float64))
            total = torch.nn.utils.clip_grad_norm_([p], max_norm)
            ref_coef = min(1.0, max_norm / (float(total) + 1e-6))
            assert oracle.clip_coef(got, max_norm) == f32(ref_coef), (n, max_norm)
    assert oracle.clip_coef(0.0, 1.0) == 1.0


# ---------------------------------------------------------------------------
# Ledger: the values the pages print.
# ---------------------------------------------------------------------------

def pin_ledger():
    gold = golden("ledger_worked_values.json")
    GB, GiB = 1e9, float(1 << 30)
    for case in gold["memory"]:
        unit = GB if case["unit"] == "GB" else GiB
        for stage, val in case["stage_values"].items():
            got = oracle.ledger_bytes(case["psi"], case["n"], int(stage), case["grads_transient"]) / unit
            assert abs(got - val) <= case["tol"], (case["cite"], stage, got, val)
    for case in gold["ratios_in_psi"]:
        got = oracle.ledger_bytes(1.0, case["n"], case["stage"], case["grads_transient"])
        assert abs(got - case["bytes_per_param"]) < 1e-12, case["cite"]
    d = gold["stage0_to_1_drop"]
    drop = (oracle.ledger_bytes(d["psi"], d["n"], 0, True) - oracle.ledger_bytes(d["psi"], d["n"], 1, True)) / GiB
    assert abs(drop - d["GiB"]) <= d["tol"], drop
    z = gold["zero3_min_ranks"]
    nmin = next(n for n in range(1, 10000) if oracle.ledger_bytes(z["psi"], n, 3) <= z["budget_GB"] * GB)
    assert nmin == z["n_min"], nmin
    z2 = gold["zero2_no_fit"]
    assert oracle.ledger_bytes(z2["psi"], 1 << 20, 2) > z2["budget_GB"] * GB
    for c in gold["comm_elements_per_step"]:
        assert oracle.comm_elements(1.0, 8, c["stage"]) == c["in_psi"], c
    r = gold["ring_exact"]
    assert abs(oracle.comm_elements(1.0, r["n"], r["stage"], True) - r["in_psi"]) < 1e-12


def pin_sim_footprint(seed=9):
    """The simulation's resident bytes ("Learn: ZeRO & FSDP", section 3: 2
    bytes of bf16 gradient, 12 of fp32 master + m + v, 2 of bf16 parameters
    per element) equal the bytes of the buffers a simulation actually
    allocates, sized from the brute-force listing: n gradient buffers, three
    state arrays, the output and, for the clipped step, the reduced gradient."""
    rng = np.random.default_rng(seed)
    for _ in range(60):
        n = int(rng.integers(1, 10))
        numel = [int(x) for x in rng.integers(0, 50, int(rng.integers(1, 4)))]
        flat, _, local = brute_layout(n, numel)
        for every_rank in (True, False):
            elems = len(flat) if every_rank else len(local[0])
            for bf in (True, False):
                for with_out, with_g in ((True, False), (False, False), (True, True)):
                    bufs = [np.zeros(elems, np.uint16 if bf else np.float32) for _ in range(n)]
                    bufs += [np.zeros(elems, np.float32) for _ in range(3)]
                    if with_out:
                        bufs.append(np.zeros(elems, np.uint16))
                    if with_g:
                        bufs.append(np.zeros(elems, np.float32))
                    got = oracle.sim_footprint(n, numel, every_rank=every_rank, n_grads=n,
                                               grad_bytes=2 if bf else 4, with_out=with_out, with_g=with_g)
                    assert got == sum(b.nbytes for b in bufs), (n, numel, every_rank, bf, with_out, with_g)


ALL_PINS = [pin_layout_bruteforce, pin_bf16_vs_torch, pin_adamw_vs_torch64, pin_adamw_order,
            pin_scalars, pin_sharded_equals_unsharded, pin_rank_local_equals_global, pin_reduced_grad,
            pin_toy, pin_norm, pin_ledger, pin_sim_footprint, pin_rows_vs_torch_chunk, pin_reshard]
