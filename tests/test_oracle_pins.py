"""The oracle against what the pages and the mathematics fix (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import pins


def test_layout_bruteforce():
    pins.pin_layout_bruteforce()


def test_bf16_rounding_vs_torch():
    pins.pin_bf16_vs_torch()


@pytest.mark.slow
def test_bf16_rounding_exhaustive():
    """All 2^32 binary32 patterns, in chunks (about a minute)."""
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        pats = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        pins.pin_bf16_vs_torch(patterns=pats)


def test_adamw_vs_torch_binary64():
    pins.pin_adamw_vs_torch64()


def test_adamw_operation_order():
    """The association the page's code fixes, on elements where each
    alternative association changes the bits (exact-arithmetic golden)."""
    pins.pin_adamw_order()


def test_adamw_order_golden_is_reproducible(tmp_path):
    """The committed golden table is what its generator writes."""
    import json
    import subprocess
    import sys
    here = os.path.dirname(os.path.abspath(__file__))
    gen = os.path.join(here, "golden", "make_adamw_order.py")
    src = open(gen).read().replace('os.path.join(HERE, "adamw_order.json")',
                                   repr(str(tmp_path / "adamw_order.json")))
    (tmp_path / "gen.py").write_text(src.replace("HERE = os.path.dirname(os.path.abspath(__file__))",
                                                 f"HERE = {os.path.join(here, 'golden')!r}"))
    subprocess.run([sys.executable, str(tmp_path / "gen.py")], check=True, capture_output=True)
    assert json.load(open(tmp_path / "adamw_order.json")) == pins.golden("adamw_order.json")


def test_reduced_grad():
    pins.pin_reduced_grad()


def test_step_scalars():
    pins.pin_scalars()


def test_sharded_equals_unsharded():
    pins.pin_sharded_equals_unsharded()


def test_rank_local_equals_global():
    pins.pin_rank_local_equals_global()


def test_toy():
    pins.pin_toy()


def test_norm_and_clip():
    pins.pin_norm()


def test_ledger_values_printed_on_pages():
    pins.pin_ledger()


def test_sim_footprint():
    pins.pin_sim_footprint()


def test_bf16_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 3.4028235e38, 1e-45, -1e-45], np.float32)
    got = oracle.bf16(x)
    want = np.array([0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F80, 0xBF80, 0x7F80, 0x0000, 0x8000], np.uint16)
    assert np.array_equal(got, want), [hex(v) for v in got]


def test_padding_stays_positive_zero():
    """Padding with zero gradient and zero state stays +0 through any number
    of steps: g = 0 gives m = v = 0, update 0 / eps = 0, w = 0 * decay - 0."""
    n, numel = 4, [5]
    L = oracle.Layout(n, numel)
    gs = [np.zeros(L.total_padded, np.uint16) for _ in range(n)]
    for g in gs:
        g[:5] = oracle.bf16(np.ones(5, np.float32) * 1e-3)
    master = np.zeros(L.total_padded, np.float32)
    master[:5] = 0.5
    m = np.zeros_like(master)
    v = np.zeros_like(master)
    out = np.zeros(L.total_padded, np.uint16)
    for t in range(1, 30):
        oracle.zero_step_all(n, numel, gs, divisor=4.0, clip=1.0, master=master, m=m, v=v, out=out,
                             t=t, lr=0.01, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    assert np.all(master[5:].view(np.uint32) == 0) and np.all(out[5:] == 0)
    assert np.all(m[5:].view(np.uint32) == 0) and np.all(v[5:].view(np.uint32) == 0)


def test_row_layout_vs_torch_chunk():
    pins.pin_rows_vs_torch_chunk()


def test_reshard_vs_explicit_layouts():
    pins.pin_reshard()


def test_reshard_round_trip_and_edges():
    """A -> B -> A gives A back; empty units and single-rank layouts pass
    through; mismatched arguments are refused."""
    rng = np.random.default_rng(7)
    for case in range(20):
        params, numel, row_len = pins.random_params(rng, int(rng.integers(1, 6)))
        n_a, n_b = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        groups = pins.random_groups(rng, len(numel))
        units = [sum(numel[sum(groups[:i]):sum(groups[:i + 1])]) for i in range(len(groups))]
        src = pins.flat_local_shards(params, n_a, groups)
        src = [s.astype(np.float32) for s in src]
        mid = [oracle.reshard(units, n_a, src, n_b, r, row_b=row_len, numel_b=numel)
               for r in range(n_b)]
        back = [oracle.reshard(numel, n_b, mid, n_a, r, row_a=row_len, numel_b=units)
                for r in range(n_a)]
        for r in range(n_a):
            assert np.array_equal(back[r], src[r]), (case, r)
    with pytest.raises(ValueError):
        oracle.reshard([4], 2, [np.zeros(2, np.float32)] * 2, 2, 2)   # no rank 2
    with pytest.raises(ValueError):                                    # 4 vs 5 elements
        oracle.reshard([4], 2, [np.zeros(2, np.float32)] * 2, 2, 0, numel_b=[5])
    with pytest.raises(ValueError):
        oracle.Layout(2, [5], row_len=[2])                              # 2 does not divide 5


def test_reshard_span_is_a_slice_of_reshard():
    rng = np.random.default_rng(8)
    params, numel, row_len = pins.random_params(rng, 5)
    src = [s.astype(np.float32) for s in pins.flat_local_shards(params, 3)]
    whole = oracle.reshard(numel, 3, src, 2, 1, row_b=row_len)
    for a, b in ((0, len(whole)), (1, 5), (len(whole) // 2, len(whole)), (3, 3)):
        part = oracle.reshard_span(numel, 3, src, 2, 1, a, b, row_b=row_len)
        assert np.array_equal(part, whole[a:b]), (a, b)
    with pytest.raises(ValueError):
        oracle.reshard_span(numel, 3, src, 2, 1, 0, len(whole) + 1, row_b=row_len)
