"""Row-aligned (FSDP2, dim-0) layouts and checkpoint resharding on the host:
the library's zero_pack_rows against the oracle's row layout and torch.chunk,
its index maps on row layouts, and zero_reshard_host against the oracle's
reshard.  No GPU needed: nothing here launches a kernel."""
import ctypes as C

import numpy as np
import pytest

import oracle
import pins

z = pytest.importorskip("fsdp_sharded_optimizer_flat_amd")


def lib_layout(n, units, row_len):
    return z.zero_pack(n, units) if row_len is None else z.zero_pack_rows(n, units, row_len)


def test_pack_rows_matches_oracle_and_torch_chunk():
    rng = np.random.default_rng(3)
    for case in range(120):
        n = int(rng.integers(1, 12))
        params, numel, row_len = pins.random_params(rng, int(rng.integers(1, 6)))
        L = z.zero_pack_rows(n, numel, row_len)
        O = oracle.Layout(n, numel, row_len=row_len)
        t = L.unit_table()
        assert np.array_equal(t[:, 0], numel)
        assert np.array_equal(t[:, 1], O.padded) and np.array_equal(t[:, 2], O.shard)
        assert np.array_equal(t[:, 3], O.offset) and np.array_equal(t[:, 4], O.local_offset)
        assert np.array_equal(L.unit_granules(), row_len)
        assert (L.padded, L.shard, L.numel) == (O.total_padded, O.total_shard, sum(numel))
        # every rank's local shard through the library's maps == FSDP2's chunks
        want = pins.fsdp2_local_shards(params, n)
        vals = [np.asarray(p).reshape(-1) for p in params]
        for r in range(n):
            got = np.zeros(L.shard)
            for k in range(L.shard):
                j = z.zero_global_index(L, r, k)
                u = int(np.searchsorted(t[:, 3], j, side="right")) - 1
                while t[u, 1] == 0 or j >= t[u, 3] + t[u, 1]:
                    u += 1
                pos = j - t[u, 3]
                got[k] = vals[u][pos] if pos < numel[u] else 0
                assert z.zero_owner(L, j) == (r, k)
            assert np.array_equal(got, want[r]), (case, n, numel, row_len, r)


def test_pack_rows_granule_one_is_the_flat_layout():
    numel = [0, 1, 7, 100, 4099]
    for n in (1, 3, 8, 64):
        a = z.zero_pack(n, numel).unit_table()
        b = z.zero_pack_rows(n, numel, [1] * len(numel)).unit_table()
        assert np.array_equal(a, b)


def test_pack_rows_errors():
    for numel, gran, status in (([10], [3], z.ZERO_EINVAL),     # 3 does not divide 10
                                ([10], [0], z.ZERO_EINVAL),
                                ([-2], [1], z.ZERO_EINVAL),
                                ([2 ** 62], [2 ** 61], z.ZERO_ERANGE)):  # N g overflows
        with pytest.raises(z.ZeroError) as e:
            z.zero_pack_rows(8, numel, gran)
        assert e.value.status == status, (numel, gran)
    lib = z.raw_library()
    numel = np.array([10], np.int64)
    need = C.c_size_t()
    assert lib.zero_pack_rows(4, 1, numel.ctypes.data, None, None, 0, C.byref(need)) == z.ZERO_EINVAL


def test_row_layout_corrupted_is_refused():
    """The layout check bounds the padding by N g: a row layout whose padding
    is a whole rank's rows too long is refused by every entry point."""
    L = z.zero_pack_rows(4, [12], [3])
    L.units[0].padded += 12
    L.units[0].shard += 3
    L.header.padded += 12
    L.header.shard += 3
    with pytest.raises(z.ZeroError):
        z.zero_global_index(L, 0, 0)
    L = z.zero_pack_rows(4, [12], [3])
    L.units[0].granule = 5           # shard 3 is not a multiple of 5
    with pytest.raises(z.ZeroError):
        z.zero_global_index(L, 0, 0)


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_reshard_host_matches_oracle(dtype):
    rng = np.random.default_rng(11 if dtype is np.float32 else 12)
    for case in range(60):
        params, numel, row_len = pins.random_params(rng, int(rng.integers(1, 7)))
        n_a, n_b = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        src, units_a, row_a = pins.layout_case(rng, params, numel, row_len, n_a)
        _, units_b, row_b = pins.layout_case(rng, params, numel, row_len, n_b)
        src = [s.astype(dtype) for s in src]
        A, B = lib_layout(n_a, units_a, row_a), lib_layout(n_b, units_b, row_b)
        for r in range(n_b):
            want = oracle.reshard(units_a, n_a, src, n_b, r, row_a=row_a, row_b=row_b,
                                  numel_b=units_b)
            got = np.full(B.shard, 0x5a5a, dtype)      # the padding must be written
            z.zero_reshard_host(A, src, B, r, got)
            assert np.array_equal(got, want), (case, units_a, units_b, n_a, n_b, r)


def test_reshard_traffic_counts():
    A = z.zero_pack(8, [1000, 24])
    B = z.zero_pack_rows(4, [1000, 24], [10, 8])
    for r in range(4):
        b, e = z.zero_reshard_traffic(A, B, r, z.ZERO_F32)
        live = 0
        for u, (p, g) in enumerate(((1000, 10), (24, 8))):
            shard = B.unit_table()[u, 2]
            live += max(0, min(p, (r + 1) * shard) - r * shard)
        assert e == B.shard and b == 4 * (live + B.shard)
    b, e = z.zero_reshard_traffic(A, B, 0, z.ZERO_BF16)
    assert b == 2 * (250 + 8 + B.shard)


def test_reshard_argument_errors():
    A = z.zero_pack(4, [100])
    B = z.zero_pack_rows(2, [100], [10])
    src = [np.zeros(A.shard, np.float32) for _ in range(4)]
    dst = np.zeros(B.shard, np.float32)
    for bad_rank in (-1, 2):
        with pytest.raises(z.ZeroError) as e:
            z.zero_reshard_host(A, src, B, bad_rank, dst)
        assert e.value.status == z.ZERO_EINVAL
    with pytest.raises(z.ZeroError) as e:              # element counts differ
        z.zero_reshard_host(A, src, z.zero_pack(2, [101]), 0, np.zeros(51, np.float32))
    assert e.value.status == z.ZERO_EINVAL
    big = np.zeros(A.shard + B.shard, np.float32)       # dst overlaps a source
    with pytest.raises(z.ZeroError) as e:
        z.zero_reshard_host(A, [src[0], big[:A.shard], src[2], src[3]], B, 0, big[10:10 + B.shard])
    assert e.value.status == z.ZERO_EINVAL
    lib = z.raw_library()
    arr = (C.c_void_p * 4)(*[s.ctypes.data for s in src])
    assert lib.zero_reshard_host(A.ptr, C.addressof(arr), B.ptr, 0, dst.ctypes.data + 2,
                                 z.ZERO_F32) == z.ZERO_EALIGN
    assert lib.zero_reshard_host(A.ptr, C.addressof(arr), B.ptr, 0, dst.ctypes.data,
                                 7) == z.ZERO_EINVAL
    arr[2] = None
    assert lib.zero_reshard_host(A.ptr, C.addressof(arr), B.ptr, 0, dst.ctypes.data,
                                 z.ZERO_F32) == z.ZERO_EINVAL


def test_reshard_plan_is_batched():
    """Forty GPT-2 Large parameters in four flat blocks at N = 8, resharded
    to one dim-0 unit per parameter at N = 4: every element of rank 3's shard
    holds its own stream position (a property that fixes the whole shard)."""
    from fsdp_sharded_optimizer_flat_amd import workloads
    shapes = workloads.param_shapes(workloads.gpt2_large_units())[2:42]   # blocks 0-3 + 4
    numel = [workloads.numel_of(s) for s in shapes]
    row_len = workloads.row_lengths(shapes)
    groups = [len(shapes) // 4] * 3 + [len(shapes) - 3 * (len(shapes) // 4)]
    units = [sum(numel[sum(groups[:i]):sum(groups[:i + 1])]) for i in range(4)]
    A, B = z.zero_pack(8, units), z.zero_pack_rows(4, numel, row_len)
    # source values: the stream position itself, as uint32 bits in float32
    # slots (the reshard copies bits; NaN patterns included)
    src = []
    t = A.unit_table()
    for q in range(8):
        s = np.zeros(A.shard, np.uint32)
        start = 0
        for u in range(len(units)):
            lo, hi = q * t[u, 2], min((q + 1) * t[u, 2], units[u])
            if hi > lo:
                s[t[u, 4]:t[u, 4] + hi - lo] = np.arange(start + lo, start + hi, dtype=np.uint32)
            start += units[u]
        src.append(s.view(np.float32))
    assert sum(numel) < 2 ** 32
    r = 3
    got = np.zeros(B.shard, np.float32)
    z.zero_reshard_host(A, src, B, r, got)
    got = got.view(np.uint32)
    tb = B.unit_table()
    stream_start = np.concatenate([[0], np.cumsum(numel)])
    for u in range(len(numel)):
        lo = r * tb[u, 2]
        seg = got[tb[u, 4]:tb[u, 4] + tb[u, 2]]
        pos = np.arange(lo, lo + tb[u, 2])
        want = np.where(pos < numel[u], stream_start[u] + pos, 0).astype(np.uint32)
        assert np.array_equal(seg, want), u


def test_reshard_empty_shards_take_null_pointers():
    """All-empty layouts: nothing to read or write, NULL buffers accepted."""
    lib = z.raw_library()
    A, B = z.zero_pack(4, [0, 0]), z.zero_pack_rows(3, [0], [5])
    arr = (C.c_void_p * 4)()
    assert lib.zero_reshard_host(A.ptr, C.addressof(arr), B.ptr, 2, None, z.ZERO_F32) == z.ZERO_OK
    assert lib.zero_reshard_host(A.ptr, C.addressof(arr), z.zero_pack(1, [0]).ptr, 0, None,
                                 z.ZERO_BF16) == z.ZERO_OK
