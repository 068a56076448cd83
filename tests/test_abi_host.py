"""The C ABI on the host: the library loads, exports every declared symbol,
and its host-side parts (layout, index maps, step scalars, clip coefficient,
ledger, traffic counts, argument validation) agree with the oracle and the
pages.  No GPU needed: nothing here launches a kernel."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero.h")

z = pytest.importorskip("fsdp_sharded_optimizer_flat_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(zero_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 19, names
    lib = z.raw_library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in zero.h but not exported"
    assert set(names) == set(z.EXPORTED)
    assert z.zero_abi_version() == z.ZERO_ABI_VERSION == 2


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name in ["ZERO_OK", "ZERO_EINVAL", "ZERO_ERANGE", "ZERO_EALIGN", "ZERO_ENOSPC", "ZERO_EHIP",
                 "ZERO_F32", "ZERO_BF16", "ZERO_GLOBAL", "ZERO_LOCAL", "ZERO_MAX_RANKS"]:
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(z, name), name
    assert C.sizeof(z.ZeroLayoutHeader) == 40 and C.sizeof(z.ZeroUnit) == 48
    assert z.zero_layout_bytes(36) == 40 + 36 * 48


# -- layout ---------------------------------------------------------------------

def test_layout_matches_oracle_and_bruteforce():
    rng = np.random.default_rng(3)
    cases = [(n, [p]) for n in range(1, 10) for p in range(0, 30)]
    cases += [(int(rng.integers(1, 10)), [int(x) for x in rng.integers(0, 65, rng.integers(1, 5))])
              for _ in range(300)]
    for n, numel in cases:
        L = z.zero_pack(n, numel)
        O = oracle.Layout(n, numel)
        t = L.unit_table()
        assert L.padded == O.total_padded and L.shard == O.total_shard and L.numel == sum(numel)
        assert np.array_equal(t[:, 1], O.padded) and np.array_equal(t[:, 2], O.shard)
        assert np.array_equal(t[:, 3], O.offset) and np.array_equal(t[:, 4], O.local_offset)
        flat, _starts, local = pins.brute_layout(n, numel)
        for r in range(n):
            for k, j in enumerate(local[r]):
                assert z.zero_global_index(L, r, k) == j
                assert z.zero_owner(L, j) == (r, k)


def test_layout_of_the_workloads():
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS
    want = {"toy": (1000, 250), "gpt2l_block": (19_677_440, 2_459_680),
            "gpt2l": (774_090_240, 96_761_280), "llama8b_z3": (8_030_261_248, 125_472_832)}
    for name, (ph, s) in want.items():
        w = WORKLOADS[name]
        L = z.zero_pack(w.n_ranks, w.unit_numel)
        assert (L.padded, L.shard) == (ph, s), name


def test_pack_errors():
    with pytest.raises(z.ZeroError) as e:
        z.zero_pack(0, [10])
    assert e.value.status == z.ZERO_EINVAL
    with pytest.raises(z.ZeroError) as e:
        z.zero_pack(4, [-1])
    assert e.value.status == z.ZERO_EINVAL
    with pytest.raises(z.ZeroError) as e:
        z.zero_pack(4, [2 ** 63 - 2])
    assert e.value.status == z.ZERO_ERANGE
    lib = z.raw_library()
    numel = np.array([10], np.int64)
    buf = (C.c_char * 8)()
    need = C.c_size_t()
    assert lib.zero_pack(4, 1, numel.ctypes.data, C.addressof(buf), 8, C.byref(need)) == z.ZERO_ENOSPC
    assert need.value == 88
    L = z.zero_pack(4, [10])
    with pytest.raises(z.ZeroError):
        z.zero_global_index(L, 4, 0)
    with pytest.raises(z.ZeroError):
        z.zero_owner(L, 12)


def test_empty_layout():
    L = z.zero_pack(8, [])
    assert (L.padded, L.shard, L.n_units) == (0, 0, 0)
    L = z.zero_pack(8, [0, 0])
    assert (L.padded, L.shard) == (0, 0)


# -- scalars --------------------------------------------------------------------------

def test_scalars_match_oracle_bitwise():
    for (lr, b1, b2, eps, wd) in pins.HYPER_SETS:
        prev = None
        for t in range(1, 3001):
            s = z.zero_adamw_scalars_for(t, lr, b1, b2, eps, wd) if t <= 40 or t % 97 == 0 else None
            nxt = z.zero_adamw_scalars_next(prev) if prev is not None else z.zero_adamw_scalars_for(1, lr, b1, b2, eps, wd)
            if s is not None:
                o = oracle.adamw_scalars(t, lr, b1, b2, wd)
                got = np.array([s.one_minus_b1, s.one_minus_b2, s.pow1, s.pow2, s.bc1, s.bc2,
                                s.step_size, s.decay], np.float32)
                assert np.array_equal(got.view(np.uint32), o["_raw"].view(np.uint32)), (t, lr)
                assert s.as_dict() == nxt.as_dict(), t
            prev = nxt


def test_scalars_hex_pins():
    """bc1, bc2, lr/bc1 and 1 - lr*wd for t = 1..3 as binary32 bit patterns
    (independent of how b^t is formed, since b^t is exact-rounded for t <= 3)."""
    want = {
        0.01: dict(bc1=[0x3dccccd0, 0x3e428f60, 0x3e8ac086], bc2=[0x3e64f930, 0x3e9fdf39, 0x3ec15c4c],
                   step=[0x3dccccc9, 0x3d579431, 0x3d1724d4], decay=0x3f7fbe77),
        3e-4: dict(bc1=[0x3dccccd0, 0x3e428f60, 0x3e8ac086], bc2=[0x3e64f930, 0x3e9fdf39, 0x3ec15c4c],
                   step=[0x3b449ba3, 0x3acef4ab, 0x3a91191e], decay=0x3f7ffe09),
    }
    u = lambda x: int(np.float32(x).view(np.uint32))
    for lr, w in want.items():
        for t in (1, 2, 3):
            s = z.zero_adamw_scalars_for(t, lr, 0.9, 0.95, 1e-8, 0.1)
            assert (u(s.bc1), u(s.bc2), u(s.step_size), u(s.decay)) == \
                (w["bc1"][t - 1], w["bc2"][t - 1], w["step"][t - 1], w["decay"])


def test_scalar_errors():
    with pytest.raises(z.ZeroError):
        z.zero_adamw_scalars_for(0, 1e-3, 0.9, 0.95, 1e-8, 0.1)
    with pytest.raises(z.ZeroError):
        z.zero_adamw_scalars_for(1, float("nan"), 0.9, 0.95, 1e-8, 0.1)


def test_clip_coef_matches_oracle():
    rng = np.random.default_rng(5)
    for s in list(10.0 ** rng.uniform(-12, 8, 2000)) + [0.0, 1.0, 1e-12]:
        for mx in (1.0, 0.5, 3.0):
            assert z.zero_clip_coef(float(s), mx) == oracle.clip_coef(float(s), mx)
    with pytest.raises(z.ZeroError):
        z.zero_clip_coef(-1.0, 1.0)
    with pytest.raises(z.ZeroError):
        z.zero_clip_coef(1.0, 0.0)


def test_nonfinite_norm_has_no_coefficient():
    """A gradient with an infinite or NaN element has an infinite or NaN sum
    of squares: the host refuses it (the device chain writes a NaN coefficient
    and skips the step instead, tested on the GPU), also when finite rank sums
    overflow in their rank-ordered total."""
    for bad in (float("inf"), float("nan"), -0.5):
        with pytest.raises(z.ZeroError) as e:
            z.zero_clip_coef(bad, 1.0)
        assert e.value.status == z.ZERO_EINVAL
        with pytest.raises(z.ZeroError):
            z.zero_clip_coef_ranks([1.0, bad, 2.0], 1.0)
    with pytest.raises(z.ZeroError):
        z.zero_clip_coef_ranks([1.7e308, 1.7e308], 1.0)      # the total overflows
    assert z.zero_clip_coef(1.7e308, 1.0) == oracle.clip_coef(1.7e308, 1.0)   # finite: as before
    assert z.zero_clip_coef_ranks([1.0, 3.0], 1.0)[0] == oracle.clip_coef(4.0, 1.0)


def test_gradnorm_noalloc_validation_without_device():
    """zero_gradnorm_async_noalloc checks every argument, and the size of the
    selection's partials against its fixed array, before its first HIP call:
    on this host (no GPU) the errors come back as status codes."""
    lib = z.raw_library()
    f = lib.zero_gradnorm_async_noalloc
    f.restype = C.c_int32
    f.argtypes = [C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_int32,
                  C.c_int32, C.c_float, C.c_void_p, C.c_int32, C.c_void_p,
                  C.c_void_p]
    fake = 1 << 40                       # never dereferenced: no launch happens
    grads = (C.c_void_p * 2)(fake, fake + (1 << 34))
    big = z.zero_pack(1, [1 << 31])     # 4M partials: 32 MiB > the 16 MiB array
    need = z.zero_gradnorm_workspace_bytes(big, 0)
    assert need > z.ZERO_NOALLOC_SCRATCH_BYTES
    G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
    args = lambda L, rank=0, n=1, gi=Lc, div=1.0, gidx=Lc, sq=fake + (1 << 36): (
        L.ptr, rank, C.addressof(grads), n, z.ZERO_BF16, gi, div, None, gidx, sq, None)
    assert f(*args(big)) == z.ZERO_ENOSPC
    ok = z.zero_pack(2, [1 << 20])      # 2048 partials: fits
    assert z.zero_gradnorm_workspace_bytes(ok, 0) <= z.ZERO_NOALLOC_SCRATCH_BYTES
    assert f(*args(ok, sq=None)) == z.ZERO_EINVAL
    assert f(*args(ok, sq=fake + 4)) == z.ZERO_EALIGN
    assert f(*args(ok, rank=2)) == z.ZERO_EINVAL
    assert f(*args(ok, n=0)) == z.ZERO_ERANGE
    assert f(*args(ok, div=0.0)) == z.ZERO_EINVAL
    assert f(*args(ok, rank=-1, gi=Lc)) == z.ZERO_EINVAL
    assert f(*args(ok, gidx=5)) == z.ZERO_EINVAL


# -- ledger -------------------------------------------------------------------------------

def test_sim_footprint_matches_oracle_and_workloads():
    """The simulation's resident bytes: library against the oracle on random
    layouts (every rank GLOBAL, one rank LOCAL, mixed spaces), and the
    workloads' figures: the GPT-2 Large model with all N = 8 shards, (2N + 14)
    P^ = 30 x 774,090,240 = 23,222,707,200 bytes; one N = 64 rank of the 8B
    Llama shape, (2N + 14) S = 142 x 125,472,832 = 17,817,142,144 bytes, plus 4
    S for the clipped step's reduced gradient."""
    from fsdp_sharded_optimizer_flat_amd import workloads as W
    rng = np.random.default_rng(3)
    G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
    for _ in range(40):
        n = int(rng.integers(1, 9))
        numel = [int(x) for x in rng.integers(0, 5000, int(rng.integers(1, 5)))]
        L = z.zero_pack(n, numel)
        for bf in (True, False):
            for with_out, with_g in ((True, False), (False, False), (True, True)):
                gb, dt = (2, z.ZERO_BF16) if bf else (4, z.ZERO_F32)
                for every, idx in ((True, G), (False, Lc)):
                    got = z.zero_sim_footprint(L, n, dt, idx, idx, idx, with_out, with_g)
                    want = oracle.sim_footprint(n, numel, every_rank=every, n_grads=n, grad_bytes=gb,
                                                with_out=with_out, with_g=with_g)
                    assert got["total_bytes"] == want
                # mixed spaces: GLOBAL gradients, LOCAL state and out
                mix = z.zero_sim_footprint(L, n, dt, G, Lc, Lc, with_out, with_g)
                assert mix["grads_bytes"] == n * gb * L.padded
                assert mix["total_bytes"] == n * gb * L.padded + (12 + 2 * with_out + 4 * with_g) * L.shard
    g = W.WORKLOADS["gpt2l"]
    L = z.zero_pack(g.n_ranks, list(g.unit_numel))
    assert z.zero_sim_footprint(L, 8, z.ZERO_BF16, G, G, G)["total_bytes"] == 23_222_707_200
    ll = W.WORKLOADS["llama8b_z3"]
    L = z.zero_pack(ll.n_ranks, list(ll.unit_numel))
    assert z.zero_sim_footprint(L, 64, z.ZERO_BF16, Lc, Lc, Lc)["total_bytes"] == 17_817_142_144
    assert z.zero_sim_footprint(L, 64, z.ZERO_BF16, Lc, Lc, Lc, True, True)["total_bytes"] == \
        17_817_142_144 + 4 * 125_472_832
    for bad in ((0, z.ZERO_BF16, G, G, G), (8, 7, G, G, G), (8, z.ZERO_BF16, 2, G, G)):
        with pytest.raises(z.ZeroError):
            z.zero_sim_footprint(L, *bad)


def test_ledger_matches_oracle_and_pages():
    for psi in (1.0, 0.774e9, 7.5e9, 70e9):
        for n in (1, 2, 8, 64):
            for stage in range(4):
                for tr in (False, True):
                    led = z.zero_ledger(psi, n, stage, tr)
                    assert led["model_state_bytes"] == pytest.approx(oracle.ledger_bytes(psi, n, stage, tr), rel=1e-15)
                    assert led["comm_elements"] == oracle.comm_elements(psi, n, stage)
                    assert led["comm_elements_ring"] == pytest.approx(oracle.comm_elements(psi, n, stage, True), rel=1e-15)
    gold = pins.golden("ledger_worked_values.json")
    for case in gold["memory"]:
        unit = 1e9 if case["unit"] == "GB" else float(1 << 30)
        for stage, val in case["stage_values"].items():
            got = z.zero_ledger(case["psi"], case["n"], int(stage), case["grads_transient"])
            assert abs(got["model_state_bytes"] / unit - val) <= case["tol"], (case["cite"], stage)
    toy = pins.golden("toy_printed.json")
    assert z.zero_ledger(toy["P"], toy["n"], 1)["optimizer_floats_per_rank"] == toy["optimizer_floats_per_rank"]
    assert z.zero_ledger(toy["P"], toy["n"], 0)["optimizer_floats_per_rank"] == toy["optimizer_floats_unsharded"]
    gb = gold["zero3_gather_buffer"]
    per_unit = gb["psi"] / gb["units"]
    L = z.zero_pack(64, [int(per_unit)] * 4)
    assert abs(z.zero_gather_buffer_bytes(L, 1) / 1e9 - gb["GB_per_unit"]) <= gb["tol"]


def test_traffic_counts():
    L = z.zero_pack(8, [774_090_240])
    b, e = z.zero_step_traffic(L, -1, 8, z.ZERO_BF16, True)
    assert e == 774_090_240 and b == (2 * 8 + 26) * e
    L = z.zero_pack(64, [8_030_261_248])
    b, e = z.zero_step_traffic(L, 0, 64, z.ZERO_BF16, True)
    assert e == 125_472_832 and b == (2 * 64 + 26) * e
    b, e = z.zero_gradnorm_traffic(L, 0, 64, z.ZERO_BF16, True)
    assert b == (2 * 64 + 4) * e
    b, e = z.zero_step_traffic(z.zero_pack(4, [1000]), -1, 4, z.ZERO_F32, True)
    assert b == (4 * 4 + 26) * 1000


# -- argument validation (rejected before any device work) -------------------------------
# These calls pass made-up device addresses that validation must reject; they
# are skipped where a GPU is visible so that a validation bug can never turn
# into a launch on fake pointers.

def _no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation test with made-up addresses; runs only without a GPU")


def _raw_step(L, rank=-1, grads=(0x1000,), n_grads=None, gdt=1, gidx=0, div=1.0,
              w=0x10000000, m=0x20000000, v=0x30000000, sidx=0, out=0x40000000, oidx=0, sc=True):
    lib = z.raw_library()
    arr = (C.c_void_p * max(len(grads), 1))(*grads) if grads is not None else None
    s = z.zero_adamw_scalars_for(1, 1e-3, 0.9, 0.95, 1e-8, 0.1) if sc else None
    if n_grads is None:
        n_grads = len(grads) if grads is not None else 1
    return lib.zero_step(L.ptr, rank, C.addressof(arr) if arr is not None else None,
                         n_grads, gdt, gidx, div, w, m, v, sidx,
                         out, oidx, C.byref(s) if s is not None else None, None)


def test_step_argument_errors():
    _no_gpu()
    L = z.zero_pack(4, [1000])
    assert _raw_step(L, rank=4) == z.ZERO_EINVAL                       # rank >= N
    assert _raw_step(L, rank=-1, sidx=1) == z.ZERO_EINVAL              # all-ranks needs GLOBAL
    assert _raw_step(L, grads=None) == z.ZERO_EINVAL
    assert _raw_step(L, n_grads=0) == z.ZERO_ERANGE
    assert _raw_step(L, grads=(0x1000,) * 257) == z.ZERO_ERANGE
    assert _raw_step(L, grads=(0,)) == z.ZERO_EINVAL                    # NULL gradient
    assert _raw_step(L, div=0.0) == z.ZERO_EINVAL
    assert _raw_step(L, div=float("inf")) == z.ZERO_EINVAL
    assert _raw_step(L, gdt=7) == z.ZERO_EINVAL
    assert _raw_step(L, gidx=5) == z.ZERO_EINVAL
    assert _raw_step(L, w=0) == z.ZERO_EINVAL
    assert _raw_step(L, sc=False) == z.ZERO_EINVAL
    assert _raw_step(L, grads=(0x1001,)) == z.ZERO_EALIGN              # bf16 needs 2-byte alignment
    assert _raw_step(L, gdt=0, grads=(0x1002,)) == z.ZERO_EALIGN       # f32 needs 4
    assert _raw_step(L, w=0x10000002) == z.ZERO_EALIGN
    assert _raw_step(L, out=0x40000001) == z.ZERO_EALIGN
    # aliasing: a written buffer inside a gradient, or two written buffers overlapping
    assert _raw_step(L, grads=(0x10000000 - 100,)) == z.ZERO_EINVAL
    assert _raw_step(L, m=0x10000000 + 3996) == z.ZERO_EINVAL
    assert _raw_step(L, out=0x30000000 + 8) == z.ZERO_EINVAL
    bad = z.zero_pack(4, [1000])
    bad.header.magic = 0
    assert _raw_step(bad) == z.ZERO_EINVAL
    bad = z.zero_pack(4, [1000])
    bad.units[0].shard = 7                                               # inconsistent layout
    assert _raw_step(bad) == z.ZERO_EINVAL


def test_gradnorm_argument_errors():
    _no_gpu()
    L = z.zero_pack(4, [1000])
    lib = z.raw_library()
    need = z.zero_gradnorm_workspace_bytes(L, -1)
    np_ = 1000 // 512 + 2                 # partials: one per 512-element tile, the first of a
                                          # segment starting up to 56 elements before it
    tree = 1                              # one 1024-way level reduces them to the result
    assert need == 8 * (np_ + 1 + tree)
    arr = (C.c_void_p * 1)(0x1000)
    res = C.c_double()
    # short workspace
    assert lib.zero_gradnorm(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000000,
                             need - 8, C.byref(res), None) == z.ZERO_ENOSPC
    # NULL result
    assert lib.zero_gradnorm(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000000,
                             need, None, None) == z.ZERO_EINVAL
    # workspace misaligned / overlapping the gradient
    assert lib.zero_gradnorm(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000004,
                             need, C.byref(res), None) == z.ZERO_EALIGN
    assert lib.zero_gradnorm(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x1000 + 8,
                             need, C.byref(res), None) == z.ZERO_EINVAL
    # async: NULL / misaligned result, result inside a gradient
    assert lib.zero_gradnorm_async(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000000,
                                   need, None, None) == z.ZERO_EINVAL
    assert lib.zero_gradnorm_async(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000000,
                                   need, 0x30000004, None) == z.ZERO_EALIGN
    assert lib.zero_gradnorm_async(L.ptr, -1, C.addressof(arr), 1, 1, 0, 1.0, None, 0, 0x20000000,
                                   need, 0x1000 + 16, None) == z.ZERO_EINVAL


def test_strerror():
    for s in (0, -1, -2, -3, -4, -5):
        assert z.zero_strerror(s) and z.zero_strerror(s) != "unknown status"
    assert z.zero_last_hip_error() == ""


# -- build flags --------------------------------------------------------------------------------

def test_device_code_has_no_contraction_or_flush():
    """The device IR carries no fast-math flags that could fuse or reassociate
    (contract / reassoc / afn / fast) and no denormal flushing; the gfx950
    assembly has no packed-fp32 arithmetic and no scratch spills."""
    from fsdp_sharded_optimizer_flat_amd import _build
    for src in ("step_kernels.hip", "norm_kernels.hip"):
        ir = _build.device_ir(src)
        for flag in (" contract ", " reassoc ", " afn ", " fast ", " nnan ", " ninf "):
            assert flag not in ir, (src, flag)
        assert '"denormal-fp-math-f32"="preserve-sign' not in ir
        asm = _build.device_asm(src)
        assert not re.search(r"v_pk_(fma|mul|add)_f32", asm), src
        assert ".amdhsa_float_denorm_mode_32 3" in asm
        for m in re.finditer(r"\.private_segment_fixed_size:\s+(\d+)", asm):
            assert int(m.group(1)) == 0, (src, "scratch use")


def test_overlap_condition_worked_numbers():
    """The overlap condition against the numbers the pages work out."""
    o = pins.golden("ledger_worked_values.json")["overlap"]
    for key in ("intra_node", "cross_node"):
        c = o[key]
        r = z.zero_overlap(o["psi_unit"], c["n"], c["busbw"], o["tokens"], o["implied_flops_per_s"])
        assert abs(r["gather_s"] * 1e3 - c["gather_ms"]) <= c["tol_rel"] * c["gather_ms"], (key, r)
        assert abs(r["compute_flops"] / 1e12 - o["compute_tflop"]) <= o["compute_tol_rel"] * o["compute_tflop"]
        assert abs(r["compute_s"] * 1e3 - o["compute_ms"]) <= 0.05 * o["compute_ms"]
        assert r["hidden"] == 1 and r["ratio"] < 1
    # a tiny batch cannot hide the gather (the page's caveat)
    r = z.zero_overlap(o["psi_unit"], 64, 50e9, 64, o["implied_flops_per_s"])
    assert r["hidden"] == 0
    with pytest.raises(z.ZeroError):
        z.zero_overlap(1e9, 8, 0.0, 1.0, 1.0)


def test_clip_coef_across_ranks():
    """The ranks' binary64 sums added in rank order, then the coefficient:
    equal to the oracle's coefficient of the same rank-ordered total."""
    rng = np.random.default_rng(17)
    for n in (1, 2, 8, 64, 1000):
        sums = np.abs(rng.standard_normal(n)) * 10.0 ** rng.integers(-12, 3, n)
        total = 0.0
        for s in sums:               # Python floats: binary64, one rounding per add
            total = total + float(s)
        coef, t = z.zero_clip_coef_ranks(sums, 0.5)
        assert t == total
        assert coef == oracle.clip_coef(total, 0.5)
    assert z.zero_clip_coef_ranks([1e-30, 1e-30], 1.0)[0] == 1.0
    for bad in ([], [1.0, -1.0], [float("nan")]):
        with pytest.raises(z.ZeroError):
            z.zero_clip_coef_ranks(bad, 1.0)
    with pytest.raises(z.ZeroError):
        z.zero_clip_coef_ranks([1.0], 0.0)


def test_arena_plan():
    """zero_arena_plan: buffers in order, non-overlapping, buffer i at phase
    (i * 256 KiB) mod 2 MiB, no more than one 2 MiB page of slack per buffer
    (sizes drawn at random: no run of more than 32 equal sizes, where one
    more page is taken -- tests/test_bench_cli.py checks that case against
    its own statement of the rule); argument errors."""
    rng = np.random.default_rng(3)
    page, stag = 2 << 20, 256 << 10
    cases = [[], [0], [1], [page], [page + 1] * 9, [0, 0, 0]]
    cases += [list(rng.integers(0, 5 * page, int(rng.integers(1, 70)))) for _ in range(200)]
    for sizes in cases:
        offs, total = z.zero_arena_plan(sizes)
        end = 0
        for i, (o, s) in enumerate(zip(offs, sizes)):
            assert o >= end and o % page == (i * stag) % page
            assert o - end < page           # the first such offset at or after the previous end
            end = o + int(s)
        assert total == end
    lib = z.raw_library()
    b = (C.c_int64 * 2)(10, -1)
    o = (C.c_int64 * 2)()
    t = C.c_int64()
    assert lib.zero_arena_plan(2, C.addressof(b), C.addressof(o), C.byref(t)) == z.ZERO_EINVAL
    assert lib.zero_arena_plan(-1, None, None, C.byref(t)) == z.ZERO_EINVAL
    assert lib.zero_arena_plan(1, None, None, C.byref(t)) == z.ZERO_EINVAL
    assert lib.zero_arena_plan(0, None, None, None) == z.ZERO_EINVAL
    assert lib.zero_arena_plan(0, None, None, C.byref(t)) == z.ZERO_OK and t.value == 0
    big = (C.c_int64 * 2)(2**62, 2**62)
    assert lib.zero_arena_plan(2, C.addressof(big), C.addressof(o), C.byref(t)) == z.ZERO_ERANGE


def test_staged_step_workspace_and_errors():
    """zero_step_staged_workspace_bytes: 0 up to 24 gradients (the fused
    step runs below 25 fp32 / 33 bf16 gradients), else one chunk's fp32
    elements (the selection rounded up to whole 512-element tiles, at most
    32M); the staged step's workspace errors, raised before any device
    work."""
    _no_gpu()
    L = z.zero_pack(64, [64 * 1000 + 5, 64 * 3])
    assert z.zero_step_staged_workspace_bytes(L, 0, 8) == 0
    assert z.zero_step_staged_workspace_bytes(L, 0, 24) == 0
    assert z.zero_step_staged_workspace_bytes(L, 0, 25) > 0
    assert z.zero_step_staged_workspace_bytes(L, 0, 32) == z.zero_step_staged_workspace_bytes(L, 0, 33) > 0
    # one chunk of whole 512-element tiles, plus 4 elements to place it at the
    # state's 16-byte phase
    assert z.zero_step_staged_workspace_bytes(L, 0, 64) == 4 * ((L.shard + 511) // 512 * 512 + 4)
    assert z.zero_step_staged_workspace_bytes(L, -1, 64) == 4 * ((L.padded + 511) // 512 * 512 + 4)
    big = z.zero_pack(64, [64 * (1 << 26)])
    assert z.zero_step_staged_workspace_bytes(big, -1, 64) == 4 * ((1 << 25) + 4)
    lib = z.raw_library()
    sc = z.zero_adamw_scalars_for(1, 3e-4, 0.9, 0.95, 1e-8, 0.1)
    n = 64
    base = 0x100000000
    arr = (C.c_void_p * n)(*[base + q * 0x100000 for q in range(n)])
    w, m, v, o = (base + 0x10000000 + k * 0x1000000 for k in range(4))
    ws = base + 0x40000000

    def call(wsp, wsb):
        return lib.zero_step_staged(L.ptr, 0, C.addressof(arr), n, z.ZERO_BF16, z.ZERO_LOCAL, 64.0, w, m, v,
                                    z.ZERO_LOCAL, o, z.ZERO_LOCAL, C.byref(sc), wsp, wsb, None)
    assert call(None, 1 << 20) == z.ZERO_EINVAL
    assert call(ws + 8, 1 << 20) == z.ZERO_EALIGN
    assert call(ws, 2047) == z.ZERO_ENOSPC
    assert call(w, 1 << 20) == z.ZERO_EINVAL          # workspace overlapping master
    assert call(base, 1 << 20) == z.ZERO_EINVAL       # workspace overlapping a gradient
    # a claimed size past what any call writes (one chunk of at most 32M fp32):
    # overlaps inside the chunk are still refused, SIZE_MAX included
    assert call(w, (1 << 64) - 1) == z.ZERO_EINVAL
    assert call(w - 4096, 1 << 40) == z.ZERO_EINVAL
    assert lib.zero_step_staged_workspace_bytes(L.ptr, 0, 0, C.byref(C.c_size_t())) == z.ZERO_ERANGE


def test_occupancy_caps_table_and_setter():
    """The measured defaults per kernel family (from the streams a wave keeps
    in flight), the run-time setter, and its argument checks."""
    S, S1, NRM = z.ZERO_CAP_STEP, z.ZERO_CAP_STEP1, z.ZERO_CAP_NORM
    want = {1: 10, 2: 10, 3: 10, 4: 8, 5: 8, 6: 7, 7: 7, 8: 7, 12: 6, 16: 6, 20: 6, 21: 5,
            24: 5, 31: 5, 32: 5, 33: 7, 48: 7, 64: 5, 100: 7, 256: 7}
    if any(os.environ.get(v) for v in ("ZERO_STEP_WAVES_PER_CU", "ZERO_STEP1_WAVES_PER_CU",
                                      "ZERO_NORM_WAVES_PER_CU")):
        pytest.skip("occupancy environment overrides set")
    assert {n: z.zero_get_waves_per_cu(S, n) for n in want} == want
    assert z.zero_get_waves_per_cu(S1, 1) == 10
    assert [z.zero_get_waves_per_cu(NRM, n) for n in (8, 12, 17, 24, 25, 32, 48, 64, 128, 192,
                                                       193, 256)] == \
        [7, 7, 6, 6, 5, 5, 6, 5, 6, 6, 7, 7]
    try:
        z.zero_set_waves_per_cu(S, 3)
        assert z.zero_get_waves_per_cu(S, 64) == 3 and z.zero_get_waves_per_cu(S, 8) == 3
        assert z.zero_get_waves_per_cu(NRM, 64) == 5          # other families untouched
        z.zero_set_waves_per_cu(S1, 0)
        assert z.zero_get_waves_per_cu(S1, 1) == 0
    finally:
        z.zero_set_waves_per_cu(S, -1)
        z.zero_set_waves_per_cu(S1, -1)
    assert z.zero_get_waves_per_cu(S, 64) == 5
    for kind, waves in ((3, 5), (-1, 5), (S, 65), (S, -2)):
        with pytest.raises(z.ZeroError):
            z.zero_set_waves_per_cu(kind, waves)
    with pytest.raises(z.ZeroError):
        z.zero_get_waves_per_cu(S, 0)


def test_occupancy_caps_by_gradient_type_and_staged():
    """zero_get_waves_per_cu_for: equal to zero_get_waves_per_cu for bf16
    gradients outside the staged step; fp32 gradients on their own kernels
    (compiled for 2, 4, 8, 16, 32 ranks: caps from the bytes a lane keeps in
    flight; the run-time kernel at other N) and on the run-time reduction;
    the staged step's second half and its reduction (compiled for 32 and 64
    bf16 ranks only)."""
    S, S1, NRM = z.ZERO_CAP_STEP, z.ZERO_CAP_STEP1, z.ZERO_CAP_NORM
    BF, F32 = z.ZERO_BF16, z.ZERO_F32
    if any(os.environ.get(v) for v in ("ZERO_STEP_WAVES_PER_CU", "ZERO_STEP1_WAVES_PER_CU",
                                      "ZERO_NORM_WAVES_PER_CU")):
        pytest.skip("occupancy environment overrides set")
    for kind in (S, S1, NRM):
        for n in range(1, 257):
            assert z.zero_get_waves_per_cu_for(kind, n, BF) == z.zero_get_waves_per_cu(kind, n), (kind, n)
    assert {n: z.zero_get_waves_per_cu_for(S, n, F32) for n in (2, 4, 8, 16, 32, 3, 12, 24, 48)} == \
        {2: 8, 4: 7, 8: 6, 16: 5, 32: 5, 3: 12, 12: 7, 24: 5, 48: 5}
    assert z.zero_get_waves_per_cu_for(S, 64, BF, True) == z.zero_get_waves_per_cu(S, 64)
    assert z.zero_get_waves_per_cu_for(S1, 64, BF, True) == 12
    assert z.zero_get_waves_per_cu_for(S1, 64, F32, False) == 10
    assert [z.zero_get_waves_per_cu_for(NRM, n, F32) for n in (8, 48, 128, 129, 256)] == [4, 4, 4, 5, 5]
    assert [z.zero_get_waves_per_cu_for(NRM, n, F32, True) for n in (25, 64, 128, 192)] == [4, 4, 4, 5]
    assert [z.zero_get_waves_per_cu_for(NRM, n, BF, True) for n in (32, 33, 48, 64, 100, 192, 193, 256)] == \
        [5, 6, 6, 5, 6, 6, 7, 7]
    for args in ((3, 8, BF, 0), (S, 0, BF, 0), (S, 257, BF, 0), (S, 8, 2, 0), (S, 8, -1, 0)):
        with pytest.raises(z.ZeroError):
            z.zero_get_waves_per_cu_for(*args)
