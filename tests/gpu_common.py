"""Helpers for the GPU parity tests: buffers sized from the layout, device <->
numpy views, and the sampled oracle check used at full workload sizes.

Every device buffer a test hands to the library is allocated here with the
exact extent of its index space (P^ for GLOBAL, S for LOCAL), optionally
shifted by a few elements inside a larger allocation so that the library's
unaligned head / tail pieces get exercised."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import fsdp_sharded_optimizer_flat_amd as z
from fsdp_sharded_optimizer_flat_amd import synth

DEV = torch.device("cuda:0")


def extent(L, index):
    return L.padded if index == z.ZERO_GLOBAL else L.shard


def dev_buffer(n, dtype, shift=0, fill=0.0):
    """A contiguous device tensor of n elements starting `shift` elements into
    its allocation (shift > 0 gives a pointer that is not 16-byte aligned)."""
    base = torch.full((n + shift,), fill, dtype=dtype, device=DEV)
    return base[shift:shift + n]


def dev_buffer_guarded(n, dtype, shift=0, fill=0.0, guard=64, sentinel=-99):
    """dev_buffer with `sentinel` in the `shift` elements before the view and
    in `guard` elements after it.  Returns (view, check) where check(what)
    asserts that both guards still hold the sentinel."""
    base = torch.full((shift + n + guard,), fill, dtype=dtype, device=DEV)
    base[:shift] = sentinel
    base[shift + n:] = sentinel
    view = base[shift:shift + n]

    def check(what):
        head, tail = base[:shift], base[shift + n:]
        assert bool((head == sentinel).all()) and bool((tail == sentinel).all()), \
            f"{what}: written outside its {n} elements"
    return view, check


def to_np(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.int16:
        return t.cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits32(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


def assert_same_f32(got, want, what=""):
    """Bitwise equality, with NaN compared as NaN-ness only."""
    g, w = np.asarray(got, np.float32), np.asarray(want, np.float32)
    assert g.shape == w.shape, what
    gn, wn = np.isnan(g), np.isnan(w)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    bad = np.nonzero(bits32(g)[~gn] != bits32(w)[~wn])[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}: " \
                          f"{g[~gn][bad[:3]]} vs {w[~wn][bad[:3]]}"


def assert_same_bf16(got, want, what=""):
    g, w = np.asarray(got, np.uint16), np.asarray(want, np.uint16)
    gnan = ((g & 0x7FFF) > 0x7F80)
    wnan = ((w & 0x7FFF) > 0x7F80)
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ"
    bad = np.nonzero(g[~gnan] != w[~wnan])[0]
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at {bad[:5]}"


def hyper_args(h):
    return dict(lr=h["lr"], b1=h["b1"], b2=h["b2"], eps=h["eps"], wd=h["wd"])


def scalars(t, h, clip=1.0):
    return z.zero_adamw_scalars_for(t, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], clip)


def sampled_indices(n_total, unit_table, index_kind, rng, k=4096):
    """Random indices plus the first and last element of every unit's range
    in the given index space (offset/padded for GLOBAL, local_offset/shard
    for LOCAL), sorted and unique."""
    picks = set(int(x) for x in rng.integers(0, n_total, size=k))
    for numel, padded, shard, offset, loff in unit_table:
        a, ln = (offset, padded) if index_kind == z.ZERO_GLOBAL else (loff, shard)
        if ln > 0:
            picks.update([int(a), int(a + ln - 1), int(a + ln // 2)])
    picks.update([0, n_total - 1])
    return np.array(sorted(p for p in picks if 0 <= p < n_total), dtype=np.int64)


def oracle_on_samples(n, grads_per_step, master0, steps, h, clips=None, divisor=None):
    """Run the oracle on sampled elements: grads_per_step[s][q] holds rank q's
    gradient at the sampled elements for step s.  The elements are treated as
    one rank's shard of a one-unit layout (LOCAL gradients and state), which
    is exactly the per-element arithmetic of the full problem."""
    K = master0.size
    w = master0.astype(np.float32).copy()
    m = np.zeros(K, np.float32)
    v = np.zeros(K, np.float32)
    out = np.zeros(K, np.uint16)
    for s in range(steps):
        gs = [np.ascontiguousarray(g) for g in grads_per_step[s]]
        oracle.zero_step_rank(n, [K * n], 0, gs, grad_local=True,
                              divisor=float(n if divisor is None else divisor),
                              clip=1.0 if clips is None else clips[s], master=w, m=m, v=v,
                              state_global=False, out=out, out_gather=False, t=s + 1,
                              **hyper_args(h))
    return w, m, v, out


def gather_np(t, idx_t):
    return to_np(t.index_select(0, idx_t))
