"""GPU parity for row-aligned (FSDP2, dim-0) layouts and checkpoint
resharding, called through the C ABI.

- zero_reshard against the oracle's reshard, element by element, over random
  flat / block / row layouts, both element sizes, shifted base pointers
  (unaligned heads and tails, mismatched phases) and plans that need several
  launches;
- the fused step and the norm on a row layout against the oracle;
- training that stops, reshards its master / m / v from N = 8 flat blocks to
  N = 4 row-aligned parameters and resumes, against unsharded AdamW run
  straight through: bit for bit;
- the full-size reshards (GPT-2 Large and 8B Llama fp32 state) checked whole
  against the stream-position property."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import pins  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd import workloads  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import GPT_HYPER  # noqa: E402
from gpu_common import (DEV, assert_same_bf16, assert_same_f32, dev_buffer, hyper_args,  # noqa: E402
                        scalars, to_np)

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL


def log(msg):
    print(msg, flush=True)


def lib_layout(n, units, row_len):
    return z.zero_pack(n, units) if row_len is None else z.zero_pack_rows(n, units, row_len)


def to_dev(a, shift):
    """numpy float32 / uint16 -> device tensor at a shifted address."""
    if a.dtype == np.float32:
        t = dev_buffer(a.size, torch.float32, shift=shift)
        t.copy_(torch.from_numpy(a))
    else:
        t = dev_buffer(a.size, torch.int16, shift=shift)
        t.copy_(torch.from_numpy(a.view(np.int16)))
    return t


@pytest.mark.parametrize("dtype", [np.float32, np.uint16], ids=["f32", "bf16"])
def test_reshard_vs_oracle(dtype):
    rng = np.random.default_rng(21 if dtype is np.float32 else 22)
    for case in range(40):
        params, numel, row_len = pins.random_params(rng, int(rng.integers(1, 8)), max_rows=60,
                                                    max_cols=9)
        n_a, n_b = int(rng.integers(1, 10)), int(rng.integers(1, 10))
        src_np, units_a, row_a = pins.layout_case(rng, params, numel, row_len, n_a)
        _, units_b, row_b = pins.layout_case(rng, params, numel, row_len, n_b)
        src_np = [s.astype(dtype) for s in src_np]
        A, B = lib_layout(n_a, units_a, row_a), lib_layout(n_b, units_b, row_b)
        log(f"reshard case {case}: {units_a} N={n_a} rows={row_a is not None} -> "
            f"{units_b} N={n_b} rows={row_b is not None}")
        src = [to_dev(s, shift=int(rng.integers(0, 8))) for s in src_np]
        for r in range(n_b):
            want = oracle.reshard(units_a, n_a, src_np, n_b, r, row_a=row_a, row_b=row_b,
                                  numel_b=units_b)
            tdt = torch.float32 if dtype is np.float32 else torch.int16
            dst = dev_buffer(B.shard, tdt, shift=int(rng.integers(0, 8)), fill=7)
            z.zero_reshard(A, src, B, r, dst)
            torch.cuda.synchronize()
            got = to_np(dst)
            if dtype is np.float32:
                assert_same_f32(got, want, f"case {case} rank {r}")
            else:
                assert_same_bf16(got, want, f"case {case} rank {r}")


def test_reshard_many_runs_several_launches():
    """Hundreds of small parameters: the copy plan has far more pieces than
    one launch carries."""
    rng = np.random.default_rng(23)
    shapes = [(int(rng.integers(1, 40)), int(rng.integers(1, 7))) for _ in range(300)]
    numel = [a * b for a, b in shapes]
    row_len = [b for _, b in shapes]
    vals = np.arange(1, sum(numel) + 1, dtype=np.float32)
    groups = [37, 100, 63, 100]
    units_a = [sum(numel[sum(groups[:i]):sum(groups[:i + 1])]) for i in range(len(groups))]
    n_a, n_b = 7, 3
    A, B = z.zero_pack(n_a, units_a), z.zero_pack_rows(n_b, numel, row_len)
    whole = [vals]
    src_np = [oracle.reshard([sum(numel)], 1, whole, n_a, q, numel_b=units_a) for q in range(n_a)]
    src = [to_dev(s, shift=q % 4) for q, s in enumerate(src_np)]
    for r in range(n_b):
        want = oracle.reshard(units_a, n_a, src_np, n_b, r, row_b=row_len, numel_b=numel)
        dst = dev_buffer(B.shard, torch.float32, shift=r, fill=-1)
        z.zero_reshard(A, src, B, r, dst)
        torch.cuda.synchronize()
        assert_same_f32(to_np(dst), want, f"rank {r}")


def test_reshard_argument_errors_on_device():
    A = z.zero_pack(2, [64])
    B = z.zero_pack_rows(2, [64], [8])
    src = [torch.zeros(A.shard, device=DEV) for _ in range(2)]
    dst = torch.zeros(B.shard, device=DEV)
    with pytest.raises(z.ZeroError):
        z.zero_reshard(A, src, B, 2, dst)                   # no rank 2
    with pytest.raises(z.ZeroError):
        z.zero_reshard(A, src, B, 0, src[1])                # overwrites a source
    with pytest.raises(ValueError):
        z.zero_reshard(A, src[:1], B, 0, dst)               # one shard short
    with pytest.raises(TypeError):
        z.zero_reshard(A, src, B, 0, dst.to(torch.float64))


# ---------------------------------------------------------------------------
# The step and the norm on a row-aligned layout
# ---------------------------------------------------------------------------

def row_model(rng, n_params=14):
    shapes = []
    for i in range(n_params):
        if i % 3 == 0:
            shapes.append((int(rng.integers(1, 700)),))
        else:
            shapes.append((int(rng.integers(1, 90)), int(rng.integers(1, 70))))
    return shapes


@pytest.mark.parametrize("n,rank", [(4, 0), (4, 3), (8, 5)])
def test_step_on_row_layout_vs_oracle(n, rank):
    rng = np.random.default_rng(31 + rank)
    shapes = row_model(rng)
    numel = [workloads.numel_of(s) for s in shapes]
    row_len = workloads.row_lengths(shapes)
    L = z.zero_pack_rows(n, numel, row_len)
    O = oracle.Layout(n, numel, row_len=row_len)
    log(f"row-layout step n={n} rank={rank} units={len(numel)} shard={L.shard}")
    # each rank's whole padded gradient (GLOBAL), padding zero, bf16
    g = (rng.standard_normal((n, L.padded)) * 1e-3).astype(np.float32)
    for u in range(len(numel)):
        g[:, O.offset[u] + numel[u]:O.offset[u] + O.padded[u]] = 0
    gdev = torch.from_numpy(g).to(torch.bfloat16).to(DEV)
    gnp = [np.ascontiguousarray(to_np(gdev[q])) for q in range(n)]
    js = np.array([O.global_of_local(rank, k) for k in range(L.shard)], np.int64)
    g_local = [np.ascontiguousarray(x[js]) for x in gnp]
    w0 = rng.normal(0, 0.02, L.shard).astype(np.float32)
    W = torch.from_numpy(w0).to(DEV)
    M, V = torch.zeros_like(W), torch.zeros_like(W)
    out = torch.zeros(L.padded, dtype=torch.int16, device=DEV)
    ow, om, ov = w0.copy(), np.zeros_like(w0), np.zeros_like(w0)
    oo = np.zeros(L.shard, np.uint16)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64,
                     device=DEV)
    for t in range(1, 4):
        ss = z.zero_gradnorm(L, rank, list(gdev), G, float(n), None, Lc, ws)
        og = oracle.reduced_grad(n, [L.shard * n], 0, g_local, grad_local=True, divisor=float(n))
        osum = oracle.sumsq(og)
        assert abs(ss - osum) <= 1e-12 * max(osum, 1e-300), (t, ss, osum)
        clip = oracle.clip_coef(osum, 0.01)
        assert z.zero_clip_coef(ss, 0.01) == clip and clip < 1.0
        z.zero_step(L, rank, list(gdev), G, float(n), W, M, V, Lc, out, G,
                    scalars(t, GPT_HYPER, z.zero_clip_coef(ss, 0.01)))
        # the oracle on the same elements as one rank's LOCAL shard
        oracle.zero_step_rank(n, [L.shard * n], 0, g_local, grad_local=True, divisor=float(n),
                              clip=clip, master=ow, m=om, v=ov, state_global=False, out=oo,
                              out_gather=False, t=t, **hyper_args(GPT_HYPER))
    torch.cuda.synchronize()
    assert_same_f32(to_np(W), ow, "master")
    assert_same_f32(to_np(M), om, "m")
    assert_same_f32(to_np(V), ov, "v")
    got_out = to_np(out)
    assert_same_bf16(got_out[js], oo, "bf16 out in its gather slots")
    rest = np.ones(L.padded, bool)
    rest[js] = False
    assert not got_out[rest].any(), "the step wrote outside rank's slots"


# ---------------------------------------------------------------------------
# Stop, reshard, resume
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("via_files", [False, True])
def test_resume_after_reshard_flat8_to_rows4(via_files, tmp_path):
    """Three steps on N = 8 flat blocks, reshard master / m / v to N = 4
    row-aligned parameters -- on the device, or through a sharded checkpoint
    (every rank saves its shard to a file, each new rank loads its shard of
    the new layout from the files) -- three more steps; gathering the shards
    gives exactly six steps of unsharded AdamW on the same gradients."""
    rng = np.random.default_rng(41)
    block = [(96,), (288, 96), (288,), (96, 96), (96,), (384, 96), (384,), (96, 384), (96,)]
    shapes = [(1000, 96)] + block + block + [(96,)]
    numel = [workloads.numel_of(s) for s in shapes]
    row_len = workloads.row_lengths(shapes)
    P = sum(numel)
    groups = [1 + len(block), len(block) + 1]
    units_a = [sum(numel[:groups[0]]), sum(numel[groups[0]:])]
    n_a, n_b = 8, 4
    A = z.zero_pack(n_a, units_a)
    B = z.zero_pack_rows(n_b, numel, row_len)
    full = z.zero_pack(1, [P])
    h = GPT_HYPER
    w0 = rng.normal(0, 0.02, P).astype(np.float32)
    gsteps = [(rng.standard_normal(P) * 1e-3).astype(np.float32) for _ in range(6)]

    def split(vec, n, units, row=None, numel_b=None):
        return [oracle.reshard([P], 1, [vec], n, q, row_b=row, numel_b=numel_b)
                for q in range(n)]

    # phase 1: flat blocks, N = 8, pre-reduced gradient (one buffer, divisor 1)
    state = {k: [torch.from_numpy(x).to(DEV) for x in split(v, n_a, units_a, numel_b=units_a)]
             for k, v in (("w", w0), ("m", np.zeros(P, np.float32)), ("v", np.zeros(P, np.float32)))}
    for t in range(1, 4):
        gl = [torch.from_numpy(x).to(DEV) for x in split(gsteps[t - 1], n_a, units_a, numel_b=units_a)]
        for q in range(n_a):
            z.zero_step(A, q, [gl[q]], Lc, 1.0, state["w"][q], state["m"][q], state["v"][q], Lc,
                        None, Lc, scalars(t, h))
    new = {}
    if via_files:
        # every rank saves its shard; each new rank loads its shard of B
        paths = [str(tmp_path / f"rank{q}.zck") for q in range(n_a)]
        for q in range(n_a):
            z.zero_ckpt_save(paths[q], A, q, 3, state["w"][q], state["m"][q], state["v"][q])
        del state
        loaded = [z.zero_ckpt_load(paths, B, r) for r in range(n_b)]
        assert all(x[0] == 3 for x in loaded)
        for i, k in enumerate(("w", "m", "v")):
            new[k] = [torch.from_numpy(loaded[r][1 + i]).to(DEV) for r in range(n_b)]
    else:
        # reshard every state array to the row layout, on the device
        for k in ("w", "m", "v"):
            new[k] = [torch.full((B.shard,), float("nan"), device=DEV) for _ in range(n_b)]
            for r in range(n_b):
                z.zero_reshard(A, state[k], B, r, new[k][r])
    # phase 2: row layout, N = 4
    outs = [torch.zeros(B.shard, dtype=torch.int16, device=DEV) for _ in range(n_b)]
    for t in range(4, 7):
        gl = [torch.from_numpy(x).to(DEV)
              for x in split(gsteps[t - 1], n_b, numel, row=row_len, numel_b=numel)]
        for r in range(n_b):
            z.zero_step(B, r, [gl[r]], Lc, 1.0, new["w"][r], new["m"][r], new["v"][r], Lc,
                        outs[r], Lc, scalars(t, h))
    # gather to one rank, on the device
    got = {}
    for k in ("w", "m", "v"):
        dst = torch.zeros(P, device=DEV)
        z.zero_reshard(B, new[k], full, 0, dst)
        got[k] = to_np(dst)
    out_full = torch.zeros(P, dtype=torch.int16, device=DEV)
    z.zero_reshard(B, outs, full, 0, out_full)
    torch.cuda.synchronize()
    # unsharded AdamW straight through
    w, m, v = w0.copy(), np.zeros(P, np.float32), np.zeros(P, np.float32)
    for t in range(1, 7):
        oracle.adamw_unsharded([gsteps[t - 1]], divisor=1.0, clip=1.0, w=w, m=m, v=v, t=t,
                               **hyper_args(h))
    assert_same_f32(got["w"], w, "master")
    assert_same_f32(got["m"], m, "m")
    assert_same_f32(got["v"], v, "v")
    assert_same_bf16(to_np(out_full), oracle.bf16(w), "bf16 parameters")


# ---------------------------------------------------------------------------
# Full-size reshards: the whole destination shard against the stream-position
# property (element of stream position s holds s mod 2^32, padding holds 0)
# ---------------------------------------------------------------------------

def fill_stream_positions(L, q, buf):
    """Rank q's LOCAL shard of layout L filled with each element's stream
    position mod 2^32 (as uint32 bits), padding 0."""
    t = L.unit_table()
    start = 0
    buf.zero_()
    for numel, padded, shard, offset, loff in t:
        lo, hi = q * shard, min((q + 1) * shard, numel)
        if hi > lo:
            vals = torch.arange(start + lo, start + hi, dtype=torch.int64, device=DEV)
            buf[loff:loff + hi - lo] = (vals & 0xFFFFFFFF).to(torch.int64).to(torch.int32)
        start += numel


@pytest.mark.parametrize("name", ["gpt2l_reshard", "llama8b_reshard"])
def test_full_size_reshard(name):
    R = workloads.RESHARDS[name]
    units = [list(u) for u in R.units]
    A = z.zero_pack(R.from_ranks, workloads.unit_numels(units))
    shapes = workloads.param_shapes(units)
    B = z.zero_pack_rows(R.to_ranks, [workloads.numel_of(s) for s in shapes],
                         workloads.row_lengths(shapes))
    log(f"{name}: {R.from_ranks} x {A.shard} -> rank {R.dst_rank} of {R.to_ranks}: {B.shard}")
    src = []
    for q in range(R.from_ranks):
        b = torch.empty(A.shard, dtype=torch.int32, device=DEV)
        fill_stream_positions(A, q, b)
        src.append(b.view(torch.float32))
    dst = torch.full((B.shard,), -1, dtype=torch.int32, device=DEV)
    z.zero_reshard(A, src, B, R.dst_rank, dst.view(torch.float32))
    want = torch.empty(B.shard, dtype=torch.int32, device=DEV)
    fill_stream_positions(B, R.dst_rank, want)
    torch.cuda.synchronize()
    bad = int((dst != want).sum().item())
    assert bad == 0, f"{bad} elements differ"


@pytest.mark.parametrize("dst_shift", [0, 1])
def test_reshard_large_launch_group_table(dst_shift):
    """One launch of more than 2^18 blocks (its group table at 2^11 blocks
    per group) in which long runs and runs of a few elements share groups;
    the destination at the sources' 16-byte phase, or one element off it."""
    units = [70_000_003, 5, 3, 70_000_001, 7, 2]
    A, B = z.zero_pack(2, units), z.zero_pack(1, units)
    log(f"large launch: 2 x {A.shard} -> {B.shard}, destination shifted by {dst_shift}")
    src = []
    for q in range(2):
        b = torch.empty(A.shard, dtype=torch.int32, device=DEV)
        fill_stream_positions(A, q, b)
        src.append(b.view(torch.float32))
    dst = dev_buffer(B.shard, torch.int32, shift=dst_shift, fill=-1)
    z.zero_reshard(A, src, B, 0, dst.view(torch.float32))
    want = torch.empty(B.shard, dtype=torch.int32, device=DEV)
    fill_stream_positions(B, 0, want)
    torch.cuda.synchronize()
    bad = int((dst != want).sum().item())
    assert bad == 0, f"{bad} elements differ"



@pytest.mark.parametrize("dst_shift", [0, 1])
def test_reshard_run_past_2_31_bytes(dst_shift):
    """One unit of 2^31 + 24,692 fp32 elements from N = 1 to rank 1 of N = 2:
    a single run of 2^30 + 12,346 elements (4.3 GB, longer than one copy
    piece addresses, so it is cut into pieces of one launch) read from source
    byte offsets past 2^32; the destination at the source's 16-byte phase, or
    one element off it."""
    P = (1 << 31) + 2 * 12_345 + 2
    A, B = z.zero_pack(1, [P]), z.zero_pack(2, [P])
    log(f"run past 2^31 bytes: 1 x {A.shard} -> rank 1 of 2: {B.shard}, destination shifted by {dst_shift}")
    src = torch.empty(A.shard, dtype=torch.int32, device=DEV)
    fill_stream_positions(A, 0, src)
    dst = dev_buffer(B.shard, torch.int32, shift=dst_shift, fill=-1)
    z.zero_reshard(A, [src.view(torch.float32)], B, 1, dst.view(torch.float32))
    want = torch.empty(B.shard, dtype=torch.int32, device=DEV)
    fill_stream_positions(B, 1, want)
    torch.cuda.synchronize()
    bad = int((dst != want).sum().item())
    assert bad == 0, f"{bad} elements differ"

def fill_stream_positions16(L, q, buf):
    """As fill_stream_positions for 2-byte elements: stream position mod 2^16."""
    t = L.unit_table()
    start = 0
    buf.zero_()
    for numel, padded, shard, offset, loff in t:
        lo, hi = q * shard, min((q + 1) * shard, numel)
        if hi > lo:
            vals = torch.arange(start + lo, start + hi, dtype=torch.int64, device=DEV)
            buf[loff:loff + hi - lo] = ((vals & 0xFFFF) - ((vals & 0x8000) << 1)).to(torch.int16)
        start += numel


@pytest.mark.parametrize("seed,kind", [(902, 0), (903, 1), (910, 2)])
def test_reshard_large_random_plans(seed, kind):
    """Random layouts of a few hundred million elements (launches whose group
    table runs at 2^11 and 2^12 blocks per group), long units mixed with units
    of a few elements, flat blocks or dim-0 rows on both sides, 4- and
    2-byte elements, destinations at any 16-byte phase: every element of the
    destination shard holds its stream position."""
    rng = np.random.default_rng(seed)
    big = [int(rng.integers(40_000_000, 150_000_000)) for _ in range(int(rng.integers(2, 6)))]
    units = []
    for b in big:
        units += [b] + [int(rng.integers(1, 40)) for _ in range(int(rng.integers(0, 4)))]
    rows = [1 if u < 40 or u % 7 else 7 for u in units]
    n_a, n_b = int(rng.integers(1, 7)), int(rng.integers(1, 3))
    A = z.zero_pack(n_a, units) if kind != 1 else z.zero_pack_rows(n_a, units, rows)
    B = z.zero_pack_rows(n_b, units, rows) if kind != 2 else z.zero_pack(n_b, units)
    r = int(rng.integers(0, n_b))
    two = kind == 2
    tdt = torch.int16 if two else torch.int32
    fill = fill_stream_positions16 if two else fill_stream_positions
    log(f"large random plan {seed}/{kind}: {len(units)} units, {sum(units)} elements, N {n_a} -> {n_b} "
        f"rank {r}, {'bf16' if two else 'f32'}")
    src = []
    for q in range(n_a):
        b = torch.empty(A.shard, dtype=tdt, device=DEV)
        fill(A, q, b)
        src.append(b.view(torch.bfloat16) if two else b.view(torch.float32))
    dst = dev_buffer(B.shard, tdt, shift=int(rng.integers(0, 8)), fill=-1)
    z.zero_reshard(A, src, B, r, dst.view(torch.bfloat16) if two else dst.view(torch.float32))
    want = torch.empty(B.shard, dtype=tdt, device=DEV)
    fill(B, r, want)
    torch.cuda.synchronize()
    bad = int((dst != want).sum().item())
    assert bad == 0, f"{bad} elements differ"
    del src, dst, want
    torch.cuda.empty_cache()


def test_reshard_with_prepared_source_pointers():
    """src_ptrs (sources marshalled once) gives the same bytes as passing
    the tensors, and a mismatched destination type is still refused."""
    A = z.zero_pack(4, [1000, 37])
    B = z.zero_pack_rows(3, [1000, 37], [10, 1])
    g = torch.Generator(device="cpu").manual_seed(7)
    src = [torch.randn(A.shard, generator=g).to(DEV) for _ in range(4)]
    sp = z.reshard_pointer_array(src)
    for r in range(3):
        d1 = torch.full((B.shard,), -1.0, device=DEV)
        d2 = torch.full((B.shard,), -2.0, device=DEV)
        z.zero_reshard(A, src, B, r, d1)
        z.zero_reshard(A, None, B, r, d2, src_ptrs=sp)
        torch.cuda.synchronize()
        assert torch.equal(d1.view(torch.int32), d2.view(torch.int32))
    with pytest.raises(TypeError):
        z.zero_reshard(A, None, B, 0, torch.zeros(B.shard, dtype=torch.int16, device=DEV), src_ptrs=sp)
