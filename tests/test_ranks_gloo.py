"""The multi-rank protocol of the sharded step, on host cores with real
processes (torch.distributed over gloo, CPU tensors only): every rank holds
its own gradient and only its own shard of master / m / v; the ranks'
gradients are pulled to every rank (an all-gather standing in for the
fixed-order pull reduce-scatter), each rank steps its shard with the
library's host step (rank-ordered sum inside), the ranks' binary64 sums of
squares are exchanged and combined in rank order by zero_clip_coef_ranks so
every rank scales by the same coefficient, and the bf16 shards are gathered.
The gathered parameters and state must equal the single-process all-ranks
step bit for bit ("ZeRO and FSDP sharding", Code: reduce-scatter, the local
AdamW, all-gather; Implementation notes: the global norm from the shards'
sums of squares).

A second test runs the checkpoint across world sizes: every rank of one world
writes its own shard file, the ranks of another world size each load their
shard from all the files (resharded from flat blocks to dim-0 rows) and train
on; the result equals unsharded AdamW on the same gradients, bit for bit."""
import os
import socket

import numpy as np
import pytest
import torch
import torch.distributed as dist
import torch.multiprocessing as mp

import fsdp_sharded_optimizer_flat_amd as z

NUMEL = [1000, 37, 2053]
H = dict(lr=1e-3, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
MAX_NORM = 1.0
STEPS = 2


def _grad(q, t, ge):
    # rank q's gradient at step t: heavy-tailed, large enough to clip
    return (np.random.default_rng(1000 * t + q).standard_t(3, ge) * 0.2).astype(np.float32)


def _master(pe):
    return np.random.default_rng(7).normal(0, 0.02, pe).astype(np.float32)


def _shard_index(L, r):
    """Global flat index of each element of rank r's LOCAL shard."""
    idx = []
    for numel, padded, shard, offset, loff in L.unit_table():
        idx.append(np.arange(offset + r * shard, offset + (r + 1) * shard, dtype=np.int64))
    return np.concatenate(idx) if idx else np.zeros(0, np.int64)


def _worker(rank, world, port, out_dir):
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    dist.init_process_group("gloo", rank=rank, world_size=world)
    try:
        L = z.zero_pack(world, NUMEL)
        js = _shard_index(L, rank)
        w = _master(L.padded)[js].copy()                # this rank's shard of the state only
        m, v = np.zeros_like(w), np.zeros_like(w)
        out = np.zeros(L.shard, np.uint16)
        coefs = []
        sc = None
        for t in range(1, STEPS + 1):
            own = torch.from_numpy(_grad(rank, t, L.padded))
            allg = [torch.empty_like(own) for _ in range(world)]
            dist.all_gather(allg, own)                  # the pull: every rank's gradient
            grads = [a.numpy() for a in allg]
            # this rank's sum of squares of its averaged gradient (binary32
            # rank-ordered sum, divided by N, squared and summed in binary64)
            s = grads[0][js].copy()
            for q in range(1, world):
                s = s + grads[q][js]
            g = s / np.float32(world)
            mine = torch.tensor([float(np.sum(g.astype(np.float64) ** 2))], dtype=torch.float64)
            sums = [torch.empty(1, dtype=torch.float64) for _ in range(world)]
            dist.all_gather(sums, mine)
            coef, _ = z.zero_clip_coef_ranks([float(x) for x in sums], MAX_NORM)
            coefs.append(coef)
            sc = (z.zero_adamw_scalars_for(t, H["lr"], H["b1"], H["b2"], H["eps"], H["wd"], coef) if t == 1
                  else z.zero_adamw_scalars_next(sc))
            sc.clip_coef = coef
            z.zero_step_host(L, rank, grads, z.ZERO_GLOBAL, float(world), w, m, v, z.ZERO_LOCAL,
                             out, z.ZERO_LOCAL, sc)
        # gather the shards (the all-gather of the bf16 parameters) and the state
        parts = {}
        # (the bf16 bit patterns travel widened to int32: gloo has no 16-bit ints)
        for name, a in (("w", w), ("m", m), ("v", v), ("out", out.astype(np.int32))):
            ta = torch.from_numpy(a.copy())
            lst = [torch.empty_like(ta) for _ in range(world)]
            dist.all_gather(lst, ta)
            parts[name] = [x.numpy() for x in lst]
        cl = [torch.empty(STEPS, dtype=torch.float64) for _ in range(world)]
        dist.all_gather(cl, torch.tensor(coefs, dtype=torch.float64))
        if rank == 0:
            np.savez(os.path.join(out_dir, "ranks.npz"),
                     **{f"{k}{q}": parts[k][q] for k in parts for q in range(world)},
                     coefs=np.stack([c.numpy() for c in cl]))
    finally:
        dist.destroy_process_group()


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


@pytest.mark.parametrize("world", [2, 3])
def test_ranks_over_gloo_equal_the_all_ranks_step(world, tmp_path):
    mp.spawn(_worker, args=(world, _free_port(), str(tmp_path)), nprocs=world, join=True)
    res = np.load(tmp_path / "ranks.npz")
    coefs = res["coefs"]
    assert np.all(coefs == coefs[0]), "every rank must scale by the same coefficient"
    assert np.all(coefs < 1.0), "the data should make clipping active"
    # the single-process all-ranks step with the same gradients and coefficients
    L = z.zero_pack(world, NUMEL)
    w = _master(L.padded)
    m, v = np.zeros_like(w), np.zeros_like(w)
    out = np.zeros(L.padded, np.uint16)
    sc = None
    for t in range(1, STEPS + 1):
        grads = [_grad(q, t, L.padded) for q in range(world)]
        c = float(coefs[0][t - 1])
        sc = (z.zero_adamw_scalars_for(t, H["lr"], H["b1"], H["b2"], H["eps"], H["wd"], c) if t == 1
              else z.zero_adamw_scalars_next(sc))
        sc.clip_coef = c
        z.zero_step_host(L, -1, grads, z.ZERO_GLOBAL, float(world), w, m, v, z.ZERO_GLOBAL, out,
                         z.ZERO_GLOBAL, sc)
    for q in range(world):
        js = _shard_index(L, q)
        for name, ref in (("w", w), ("m", m), ("v", v)):
            assert np.array_equal(res[f"{name}{q}"].view(np.uint32), ref[js].view(np.uint32)), (name, q)
        assert np.array_equal(res[f"out{q}"].astype(np.uint16), out[js]), ("out", q)


# ---------------------------------------------------------------------------
# Every rank writes its own checkpoint shard; another world size loads it
# ---------------------------------------------------------------------------

SHAPES = [(100, 10), (37,), (2053,), (64, 48)]


def _ck_grad(q, t, p):
    return (np.random.default_rng(5000 * t + q).standard_normal(p) * 1e-3).astype(np.float32)


def _ck_model():
    from fsdp_sharded_optimizer_flat_amd import workloads
    numel = [workloads.numel_of(s) for s in SHAPES]
    return numel, workloads.row_lengths(SHAPES), sum(numel)


def _global_buffer(L, vec):
    """vec (the parameters' elements in order) placed in L's padded GLOBAL
    index space, padding zero."""
    buf = np.zeros(L.padded, np.float32)
    start = 0
    for numel, padded, shard, offset, loff in L.unit_table():
        buf[offset:offset + numel] = vec[start:start + numel]
        start += numel
    return buf


def _ck_worker(rank, world, port, ck_dir, phase, steps, out_dir):
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    dist.init_process_group("gloo", rank=rank, world_size=world)
    try:
        numel, row_len, P = _ck_model()
        h = H
        if phase == 0:    # flat blocks, state from the initial parameters
            L = z.zero_pack(world, [numel[0] + numel[1], numel[2] + numel[3]])
            w = _global_buffer(L, np.random.default_rng(9).normal(0, 0.02, P).astype(np.float32))
            w = w[_shard_index(L, rank)].copy()
            m, v = np.zeros_like(w), np.zeros_like(w)
            t0 = 0
        else:             # dim-0 rows per parameter, state loaded from the files
            L = z.zero_pack_rows(world, numel, row_len)
            paths = sorted(os.path.join(ck_dir, f) for f in os.listdir(ck_dir) if f.endswith(".zck"))
            t0, w, m, v = z.zero_ckpt_load(paths, L, rank)
        sc = None
        for t in range(t0 + 1, t0 + steps + 1):
            own = torch.from_numpy(_global_buffer(L, _ck_grad(rank, t, P)))
            allg = [torch.empty_like(own) for _ in range(world)]
            dist.all_gather(allg, own)
            sc = (z.zero_adamw_scalars_for(t, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0)
                  if sc is None else z.zero_adamw_scalars_next(sc))
            z.zero_step_host(L, rank, [a.numpy() for a in allg], z.ZERO_GLOBAL, float(world), w, m, v,
                             z.ZERO_LOCAL, None, z.ZERO_LOCAL, sc)
        if phase == 0:
            z.zero_ckpt_save(os.path.join(ck_dir, f"rank{rank:03d}.zck"), L, rank, t0 + steps, w, m, v)
        else:
            parts = {}
            for name, a in (("w", w), ("m", m), ("v", v)):
                ta = torch.from_numpy(a.copy())
                lst = [torch.empty_like(ta) for _ in range(world)]
                dist.all_gather(lst, ta)
                parts[name] = [x.numpy() for x in lst]
            if rank == 0:
                np.savez(os.path.join(out_dir, "resumed.npz"),
                         **{f"{k}{q}": parts[k][q] for k in parts for q in range(world)})
        dist.barrier()
    finally:
        dist.destroy_process_group()


@pytest.mark.parametrize("worlds", [(3, 2), (2, 4)])
def test_checkpoint_written_per_rank_resumed_at_another_world_size(worlds, tmp_path):
    """World size a trains 2 steps on flat blocks and each rank writes its own
    shard file; world size b loads its shards from those files (resharded to
    dim-0 rows per parameter) and trains 2 more steps.  The state gathered
    from the b ranks equals 4 steps of unsharded AdamW whose gradient at each
    step is the rank-ordered mean of that step's world's gradients (the
    oracle), bit for bit ("ZeRO and FSDP sharding", Implementation notes)."""
    import oracle
    wa, wb = worlds
    ck = tmp_path / "ck"
    ck.mkdir()
    mp.spawn(_ck_worker, args=(wa, _free_port(), str(ck), 0, 2, str(tmp_path)), nprocs=wa, join=True)
    assert len(list(ck.glob("*.zck"))) == wa
    mp.spawn(_ck_worker, args=(wb, _free_port(), str(ck), 1, 2, str(tmp_path)), nprocs=wb, join=True)
    res = np.load(tmp_path / "resumed.npz")
    numel, row_len, P = _ck_model()
    B = z.zero_pack_rows(wb, numel, row_len)
    full = z.zero_pack(1, [P])
    h = H
    w = np.random.default_rng(9).normal(0, 0.02, P).astype(np.float32)
    m, v = np.zeros(P, np.float32), np.zeros(P, np.float32)
    for t in range(1, 5):
        n = wa if t <= 2 else wb
        oracle.adamw_unsharded([_ck_grad(q, t, P) for q in range(n)], divisor=float(n), clip=1.0,
                               w=w, m=m, v=v, t=t, lr=h["lr"], b1=h["b1"], b2=h["b2"], eps=h["eps"],
                               wd=h["wd"])
    for name, want in (("w", w), ("m", m), ("v", v)):
        got = np.zeros(P, np.float32)
        z.zero_reshard_host(B, [res[f"{name}{q}"] for q in range(wb)], full, 0, got)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), name
