"""The binding refuses buffers shorter than the layout extent the call reads
or writes (the C library sees only pointers).  Host entry points, CPU only:
nothing is written when the call is refused."""
import numpy as np
import pytest

z = pytest.importorskip("fsdp_sharded_optimizer_flat_amd")
G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL


def _sc():
    return z.zero_adamw_scalars_for(1, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0)


def _step_buffers(L, gidx, sidx, oidx, n):
    ext = lambda i: L.padded if i == G else L.shard
    gs = [np.ones(ext(gidx), np.float32) for _ in range(n)]
    st = [np.full(ext(sidx), 0.5, np.float32) for _ in range(3)]
    out = np.zeros(ext(oidx), np.uint16)
    return gs, st, out


@pytest.mark.parametrize("which", ["grad", "master", "exp_avg", "exp_avg_sq", "out"])
@pytest.mark.parametrize("rank,idx", [(-1, (G, G, G)), (1, (Lc, Lc, Lc)), (2, (G, Lc, G))])
def test_step_host_short_buffer(which, rank, idx):
    n = 4
    L = z.zero_pack(n, [37, 64, 5])
    gs, st, out = _step_buffers(L, *idx, n)
    short = lambda a: a[:-1].copy()
    if which == "grad":
        gs[2] = short(gs[2])
    elif which == "out":
        out = short(out)
    else:
        k = ["master", "exp_avg", "exp_avg_sq"].index(which)
        st[k] = short(st[k])
    before = [a.copy() for a in st] + [out.copy()]
    with pytest.raises(ValueError, match=which):
        z.zero_step_host(L, rank, gs, idx[0], float(n), *st, idx[1], out, idx[2], _sc(), 1)
    for a, b in zip(st + [out], before):
        assert np.array_equal(a, b), "a refused call must not write"


def test_step_host_exact_extent_accepted():
    L = z.zero_pack(4, [37, 64, 5])
    gs, st, out = _step_buffers(L, Lc, Lc, Lc, 4)
    z.zero_step_host(L, 1, gs, Lc, 4.0, *st, Lc, out, Lc, _sc(), 1)


@pytest.mark.parametrize("which", ["src", "dst"])
def test_reshard_host_short_buffer(which):
    A = z.zero_pack(4, [37, 64, 5])
    B = z.zero_pack_rows(3, [37, 64, 5], [1, 8, 5])
    src = [np.arange(A.shard, dtype=np.float32) + 1000 * q for q in range(4)]
    dst = np.full(B.shard, -1, np.float32)
    if which == "src":
        src[3] = src[3][:-2].copy()
    else:
        dst = dst[:-1].copy()
    before = dst.copy()
    with pytest.raises(ValueError, match=which):
        z.zero_reshard_host(A, src, B, 1, dst)
    assert np.array_equal(dst, before)
