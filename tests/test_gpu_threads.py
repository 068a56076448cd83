"""The library from several host threads at once, each enqueueing on its own
stream: the fused step over every shard (N = 8), one rank's staged step
(N = 48, many workspace chunks), one rank's clipped step with no host
synchronization (norm pass -> coefficient -> step, N = 8) and a checkpoint
reshard (flat N = 4 -> row-aligned N = 2), three calls each, all started
together.  Each thread's results must be bit for bit those of the same calls
made afterwards one after another on one stream, and the fused step's those
of the oracle: the entry points share no mutable host state (launch tables
travel by value, the device-property caches are locked)."""
import threading

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd import synth  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import GPT_HYPER  # noqa: E402
from gpu_common import DEV, assert_same_bf16, assert_same_f32, hyper_args, scalars, to_np  # noqa: E402

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
H = GPT_HYPER
CALLS = 3


def log(msg):
    print(msg, flush=True)


def _state(n_elems, seed):
    m = torch.empty(n_elems, device=DEV)
    synth.fill_normal_(m, 0.02, seed)
    return [m, torch.zeros(n_elems, device=DEV), torch.zeros(n_elems, device=DEV),
            torch.zeros(n_elems, dtype=torch.int16, device=DEV)]


def _grads(n, n_elems, seed, dtype=torch.bfloat16, std=1e-3):
    gs = [torch.empty(n_elems, dtype=dtype, device=DEV) for _ in range(n)]
    for q, g in enumerate(gs):
        synth.fill_normal_(g, std, seed + q)
    return gs


class Fused:
    """Every shard of a two-unit layout, N = 8, GLOBAL everything."""
    name = "fused step"

    def __init__(self):
        self.n, self.numel = 8, [8 * 100_003, 8 * 7_777 + 3]
        self.L = z.zero_pack(self.n, self.numel)
        self.grads = _grads(self.n, self.L.padded, 1000)
        for g in self.grads:   # the padding of a flat buffer holds +0.0
            for nu, pad, sh, off, loff in self.L.unit_table():
                g[off + nu:off + pad] = 0
        self.st = _state(self.L.padded, 1100)
        self.w0 = to_np(self.st[0]).copy()

    def run(self, stream):
        for t in range(1, CALLS + 1):
            z.zero_step(self.L, -1, self.grads, G, float(self.n), *self.st[:3], G, self.st[3], G,
                        scalars(t, H), stream)

    def outputs(self):
        return self.st


class Staged:
    """Rank 5's shard at N = 48 from LOCAL chunks, 64K-element workspace."""
    name = "staged step"

    def __init__(self):
        self.n, self.numel = 48, [48 * 50_000 + 1, 48 * 777]
        self.L = z.zero_pack(self.n, self.numel)
        self.grads = _grads(self.n, self.L.shard, 2000)
        self.st = _state(self.L.shard, 2100)
        self.ws = torch.empty(64 * 1024 + 4, device=DEV)

    def run(self, stream):
        for t in range(1, CALLS + 1):
            z.zero_step_staged(self.L, 5, self.grads, Lc, float(self.n), *self.st[:3], Lc, self.st[3], Lc,
                               scalars(t, H), self.ws, stream)

    def outputs(self):
        return self.st


class Clipped:
    """Rank 3's slice from GLOBAL gradients, N = 8: norm pass writing g and
    the sum to device memory, the coefficient on the device, the step on g."""
    name = "clipped chain"

    def __init__(self):
        self.n, self.numel = 8, [8 * 96_032, 8 * 64_032 + 5]
        self.L = z.zero_pack(self.n, self.numel)
        self.grads = _grads(self.n, self.L.padded, 3000, std=3e-2)
        self.st = _state(self.L.shard, 3100)
        self.ws = torch.zeros(z.zero_gradnorm_workspace_bytes(self.L, 3) // 8, dtype=torch.float64, device=DEV)
        self.g = torch.zeros(self.L.shard, device=DEV)
        self.ss = torch.zeros(1, dtype=torch.float64, device=DEV)
        self.coef = torch.zeros(1, device=DEV)

    def run(self, stream):
        for t in range(1, CALLS + 1):
            z.zero_gradnorm_async(self.L, 3, self.grads, G, float(self.n), self.g, Lc, self.ws, self.ss, stream)
            z.zero_clip_coef_async(self.ss, 0.05, self.coef, stream)
            z.zero_step_device_clip(self.L, 3, [self.g], Lc, 1.0, *self.st[:3], Lc, self.st[3], Lc,
                                    scalars(t, H), self.coef, stream)

    def outputs(self):
        return self.st + [self.g, self.ss, self.coef]


class Reshard:
    """Three parameters, flat N = 4 -> row-aligned N = 2, rank 1, fp32."""
    name = "reshard"

    def __init__(self):
        shapes = [(3001, 128), (77,), (640, 96)]
        numel = [int(np.prod(s)) for s in shapes]
        self.A = z.zero_pack(4, [sum(numel)])
        self.B = z.zero_pack_rows(2, numel, [s[1] if len(s) > 1 else 1 for s in shapes])
        self.src = [torch.empty(self.A.shard, device=DEV) for _ in range(4)]
        for q, s in enumerate(self.src):
            synth.fill_normal_(s, 1.0, 4000 + q)
        self.dst = torch.full((self.B.shard,), -1.0, device=DEV)

    def run(self, stream):
        for _ in range(CALLS):
            z.zero_reshard(self.A, self.src, self.B, 1, self.dst, stream)

    def outputs(self):
        return [self.dst]


JOBS = (Fused, Staged, Clipped, Reshard)


def _same(a, b, what):
    if a.dtype == torch.float32:
        assert_same_f32(to_np(a), to_np(b), what)
    elif a.dtype == torch.int16:
        assert_same_bf16(to_np(a), to_np(b), what)
    else:
        assert torch.equal(a.view(torch.int64), b.view(torch.int64)), what


def test_entry_points_from_concurrent_threads():
    threaded = [J() for J in JOBS]
    serial = [J() for J in JOBS]
    torch.cuda.synchronize()
    # the library's one-time set-up (device properties, code objects) outside the race
    warm = [J() for J in JOBS]
    for j in warm:
        j.run(None)
    torch.cuda.synchronize()
    del warm

    streams = [torch.cuda.Stream() for _ in JOBS]
    start = threading.Barrier(len(JOBS))
    errors = []

    def worker(job, stream):
        try:
            start.wait()
            job.run(stream)
            stream.synchronize()
        except BaseException as e:  # reported by the main thread
            errors.append((job.name, repr(e)))

    threads = [threading.Thread(target=worker, args=(j, s)) for j, s in zip(threaded, streams)]
    log(f"{len(threads)} threads, one stream each: " + ", ".join(j.name for j in threaded))
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()

    for j in serial:
        j.run(None)
    torch.cuda.synchronize()
    for a, b in zip(threaded, serial):
        for k, (x, y) in enumerate(zip(a.outputs(), b.outputs())):
            _same(x, y, f"{a.name}, output {k}: threaded vs serial")
        log(f"{a.name}: threaded == serial")

    f = threaded[0]   # the fused step against the oracle
    gnp = [np.ascontiguousarray(to_np(g)) for g in f.grads]
    w, m, v = f.w0.copy(), np.zeros_like(f.w0), np.zeros_like(f.w0)
    out = np.zeros(f.L.padded, np.uint16)
    for t in range(1, CALLS + 1):
        oracle.zero_step_all(f.n, f.numel, gnp, divisor=float(f.n), clip=1.0, master=w, m=m, v=v, out=out,
                             t=t, **hyper_args(H))
    for name, dev_t, ref in (("master", f.st[0], w), ("m", f.st[1], m), ("v", f.st[2], v)):
        assert_same_f32(to_np(dev_t), ref, f"fused step {name} vs oracle")
    assert_same_bf16(to_np(f.st[3]), out, "fused step out vs oracle")
    log("fused step: threaded == oracle")
