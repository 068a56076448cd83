#!/usr/bin/env python3
"""Benchmark of the fused ZeRO sharded optimizer step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload gpt2l|gpt2l_block|llama8b_z3|llama8b_z3_clip]

A step is one call of the whole hot path over one batch of synthetic input:
for the default workload (a GPT-2-Large-sized model, 36 units, 774,090,240
parameters, N = 8 simulated ranks) every rank's shard is reduced over the 8
bf16 gradient buffers, averaged, stepped with AdamW on the fp32 master / m / v
and cast to bf16 into the all-gather slots.  The clipped workload adds the
two-stage norm pass and steps from the reduced gradient it writes.

Prints ONE JSON line: throughput in shard elements per second (value), the
achieved HBM bandwidth of the dominant kernel against MI355X's 8 TB/s
(roofline; with this box's plain-copy bandwidth, measured in the same process
after the timed region, as context), and the serial CPU oracle on a bounded
sample (cpu_baseline).
Inputs are resident in HBM before the timed region; gradients are generated
once and reused by every timed step (their values do not change the work).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = ["fsdp_sharded_optimizer_flat_amd/csrc/step_kernels.hip",
                  "fsdp_sharded_optimizer_flat_amd/csrc/norm_kernels.hip",
                  "fsdp_sharded_optimizer_flat_amd/csrc/stage_kernels.hip",
                  "fsdp_sharded_optimizer_flat_amd/csrc/reshard_kernels.hip",
                  "fsdp_sharded_optimizer_flat_amd/csrc/device_common.h",
                  "fsdp_sharded_optimizer_flat_amd/csrc/zero_internal.h",
                  "fsdp_sharded_optimizer_flat_amd/csrc/capi.cpp"]   # launch shapes and caps


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and blank lines are left
    out, so the committed counters stay valid across comment edits."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed PMC summary, or None when the kernels changed since."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    with open(PMC_SUMMARY) as f:
        pmc = json.load(f)
    ent = pmc.get("workloads", {}).get(workload)
    if ent and pmc.get("kernel_source_hash") == kernel_source_hash():
        return ent["traffic_bytes_per_launch"]
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2l")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-box-copy", action="store_true",
                    help="skip the plain-copy ceiling (for profiler runs: it launches the "
                         "reshard's copy kernel too)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain device copy of known size (PMC calibration)")
    ap.add_argument("--host-step", action="store_true",
                    help="time the offload step on host cores (zero_step_host) instead of the GPU")
    ap.add_argument("--threads", type=int, default=0, help="host-step worker threads (0: all)")
    ap.add_argument("--offload", action="store_true",
                    help="time the ZeRO-Offload step: norm pass on the GPU, reduced gradient "
                         "down over PCIe, host step, bf16 parameters up (one rank's shard)")
    ap.add_argument("--chunk", type=int, default=1 << 22, help="offload pipeline chunk (elements)")
    ap.add_argument("--ranks", type=int, default=None,
                    help="simulated ranks N (default: the workload's); the same model at another N "
                         "(one rank's shard for the ZeRO-3 workloads)")
    ap.add_argument("--clip", type=float, default=None, metavar="MAX_NORM",
                    help="clip the workload's gradients to this global norm (the norm pass, the "
                         "coefficient and the step on g, as llama8b_z3_clip does)")
    ap.add_argument("--rank", type=int, default=None,
                    help="step this rank's shard only (its slice of every unit) instead of the "
                         "workload's selection (gpt2l: every rank's shards)")
    ap.add_argument("--grad-dtype", default="bf16", choices=["bf16", "f32"],
                    help="gradient element type of the workload (f32: a reduce dtype of fp32)")
    ap.add_argument("--fused", action="store_true",
                    help="above 32 ranks, time the fused step instead of the staged one")
    ap.add_argument("--sweep-waves", default=None, metavar="FAMILY:CAPS",
                    help="instead of the JSON contract line, time the step at several occupancy caps "
                         "in interleaved rounds, e.g. step:4,5,6,7 (families: step, step1, norm)")
    ap.add_argument("--rounds", type=int, default=3, help="rounds of --sweep-waves")
    ap.add_argument("--norm-only", action="store_true",
                    help="clipped workload: time the norm pass alone (it writes g unless --no-g)")
    ap.add_argument("--no-g", action="store_true",
                    help="with --norm-only: the norm pass without writing the reduced gradient")
    ap.add_argument("--stage-chunk", type=int, default=None,
                    help="elements per chunk of the staged step (default: the largest, 32M)")
    ap.add_argument("--toggle", action="store_true",
                    help="with --stagger-kib: one 2 MiB page more wherever consecutive buffers would "
                         "start a multiple of 4 MiB (plus the step) apart")
    ap.add_argument("--gap-mib", type=int, default=0,
                    help="with --stagger-kib: leave this many more MiB (a multiple of 2) between "
                         "consecutive buffers, to move their bases modulo larger powers of two")
    ap.add_argument("--stagger-kib", type=int, default=None,
                    help="place buffer i at phase (i * KiB) mod 2 MiB instead of zero_arena_plan's "
                         "256 KiB step (0: all at phase 0)")
    ap.add_argument("--streamed", action="store_true",
                    help="time the per-unit step streamed beside a backward stand-in: each unit's "
                         "gradient buckets written in backward order, the unit stepped serially "
                         "after it or overlapped on a side stream (two recycled bucket slots)")
    ap.add_argument("--producer", default="gemm", choices=["gemm", "copy"],
                    help="backward stand-in for --streamed: the weight-gradient GEMMs "
                         "dW = dY^T X (MFMA) or a copy of resident gradients (HBM)")
    ap.add_argument("--tokens", type=int, default=1024,
                    help="tokens per simulated rank of the --streamed GEMM producer")
    ap.add_argument("--reshard", default=None, metavar="NAME",
                    help="time a checkpoint reshard (gpt2l_reshard, llama8b_reshard) instead of "
                         "the step: one destination rank's fp32 shard from flat block units to "
                         "row-aligned per-parameter units at another N")
    return ap.parse_args()


def copy_calibration():
    """A plain copy of 4 GiB (2 GiB read + 2 GiB written): the reference the
    FETCH_SIZE / WRITE_SIZE counters are scaled by."""
    import torch
    n = 1 << 29  # fp32 elements = 2 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "dispatches": 3}))


def box_copy_ceiling(z, torch, stream, reps: int = 10):
    """Context for `frac`: this box's own streaming ceiling, a plain 1 GiB
    device-to-device copy (2 GiB of traffic) through the library's reshard
    copy kernel -- one rank to one rank under the same flat layout, i.e. a
    single run, 1 KiB of destination per wave, whole-span stores -- timed
    with HIP events on the launch stream in this process.  HBM bandwidth
    differs by a few percent from box to box; the ratio to this copy does
    not."""
    import numpy as np
    n = 1 << 28
    L1 = z.zero_pack(1, [n])
    a = torch.zeros(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        z.zero_reshard(L1, [a], L1, 0, b, stream)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(stream)
        z.zero_reshard(L1, [a], L1, 0, b, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))
    del a, b
    return 8.0 * n / (ms / 1e3) / 1e9


def _oracle_sample(wl, seconds: float, threads: int, start_at=None):
    """Run the oracle as it stands on `threads` independent copies of a
    bounded sample of the workload at once (one Python thread each; the
    oracle's C calls release the GIL), until `seconds` have passed.  Returns
    (oracle steps over all copies, elements per step, seconds)."""
    import threading

    import numpy as np
    import torch

    import oracle
    from fsdp_sharded_optimizer_flat_amd import synth

    n = wl.n_ranks
    P = 1 << 22 if n <= 8 else 1 << 19
    numel = [P * n] if wl.rank >= 0 else [P]
    K = P                                    # elements one oracle step processes
    h = wl.hyper

    def inputs():
        grads = []
        for r in range(n):
            g = torch.empty(K, dtype=torch.bfloat16)
            synth.fill_grad_(g, wl.grad_dist, wl.grad_scale,
                             synth.seed_of(wl.seed, synth.TAG_GRAD, 1, r))
            grads.append(np.ascontiguousarray(g.view(torch.int16).numpy().view(np.uint16)))
        w = torch.empty(K, dtype=torch.float32)
        synth.fill_normal_(w, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
        return (grads, w.numpy().copy(), np.zeros(K, np.float32), np.zeros(K, np.float32),
                np.zeros(K, np.uint16))

    def one_step(st, t):
        grads, w, m, v, out = st
        if wl.rank >= 0:
            clip = 1.0
            if wl.clip_max_norm is not None:     # the norm pass, then the clipped step
                g = oracle.reduced_grad(n, numel, 0, grads, grad_local=True, divisor=float(n))
                clip = oracle.clip_coef(oracle.sumsq(g), wl.clip_max_norm)
            oracle.zero_step_rank(n, numel, 0, grads, grad_local=True, divisor=float(n), clip=clip,
                                  master=w, m=m, v=v, state_global=False, out=out,
                                  out_gather=False, t=t, **h)
        else:
            oracle.zero_step_all(n, numel, grads, divisor=float(n), clip=1.0, master=w, m=m, v=v,
                                 out=out, t=t, **h)

    first = inputs()                              # input generation outside the timing
    states = [first] + [([g.copy() for g in first[0]],) + tuple(a.copy() for a in first[1:])
                        for _ in range(threads - 1)]
    oracle.load()
    counts = [0] * threads
    go = threading.Barrier(threads + 1)
    stop = threading.Event()

    def worker(i):
        go.wait()
        while not stop.is_set():
            counts[i] += 1
            one_step(states[i], counts[i])

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
    for t in ts:
        t.start()
    go.wait()
    t0 = time.perf_counter()
    time.sleep(seconds)
    stop.set()
    for t in ts:
        t.join()
    el = time.perf_counter() - t0               # includes the steps running when stopped
    return sum(counts), K, el


def cpu_baseline(wl, seconds: float):
    """The oracle as it stands (serial C) on a bounded sample of the
    workload -- a one-unit layout of 2^22 elements (2^19 at more than 8 ranks)
    with the workload's rank count, gradient type and distributions; for the
    clipped workload the oracle's reduced gradient, sum of squares and
    coefficient precede each step -- first on one thread, then on as many
    threads as the host share allows (up to 16), each on its own copy.
    Returns elements per second."""
    steps, K, el = _oracle_sample(wl, seconds, 1)
    what = ("norm passes, each followed by the clipped step," if wl.clip_max_norm is not None
            else "steps")
    res = {"value": steps * K / el, "unit": "elements/s", "cores": 1, "kind": "oracle",
           "sample": f"{steps} oracle {what} over a {K}-element one-unit sample of the workload "
                     f"(N={wl.n_ranks}, {wl.grad_dist} bf16 gradients), serial C, {el:.1f} s"}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = min(16, avail)
    if threads > 1:
        steps_t, K, el_t = _oracle_sample(wl, seconds, threads)
        res["all_cores"] = {
            "value": steps_t * K / el_t, "unit": "elements/s", "cores": threads,
            "sample": f"{threads} threads, each running the serial oracle on its own copy of the "
                      f"same sample: {steps_t} {what} in {el_t:.1f} s"}
    return res


def host_step_bench(args):
    """The ZeRO-Offload step on host cores: the workload's rank count and
    distributions on host memory, every element of one rank's shard (or of
    all shards) per step.  Prints one JSON line."""
    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import synth
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    n, h = wl.n_ranks, wl.hyper
    L = z.zero_pack(n, wl.unit_numel)
    G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
    gidx = G if wl.grad_index == "global" else Lc
    sidx = G if wl.rank < 0 else Lc
    oidx = G if wl.out_index == "global" else Lc
    ge = L.padded if gidx == G else L.shard
    se = L.padded if sidx == G else L.shard
    oe = L.padded if oidx == G else L.shard
    master = torch.empty(se, dtype=torch.float32)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(oe, dtype=torch.int16)
    grads = torch.empty(n, ge, dtype=torch.bfloat16)
    for r in range(n):
        synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, 1, r))
    gl = list(grads)
    sc = z.zero_adamw_scalars_for(1, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0)
    for _ in range(args.warmup):
        z.zero_step_host(L, wl.rank, gl, gidx, float(n), master, m, v, sidx, out, oidx, sc, args.threads)
        sc = z.zero_adamw_scalars_next(sc)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        z.zero_step_host(L, wl.rank, gl, gidx, float(n), master, m, v, sidx, out, oidx, sc, args.threads)
        sc = z.zero_adamw_scalars_next(sc)
    wall = time.perf_counter() - t0
    elements = se if wl.rank < 0 else L.shard
    step_bytes, _ = z.zero_step_traffic(L, wl.rank, n, z.ZERO_BF16, True)
    threads = args.threads if args.threads > 0 else os.cpu_count()
    res = {"metric": "offload (host-core) optimizer-step shard elements/sec", "value": elements * args.steps / wall,
           "unit": "elements/s", "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True, "dtype": "f32",
           "data": "synthetic",
           "config": {"workload": wl.name, "simulated_ranks": n, "elements_per_step": int(elements),
                      "threads": threads, "host_GBps": step_bytes * args.steps / wall / 1e9},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(res))


def offload_bench(args):
    """One rank's ZeRO-Offload step: the GPU reduces the N ranks' gradients
    (norm pass, fp32 reduced gradient in HBM), the pipelined offload step
    brings it down, steps the host-resident state and sends the bf16
    parameters back.  Prints one JSON line."""
    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import synth
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS

    wl = WORKLOADS[args.workload]
    if wl.rank < 0:
        raise SystemExit("--offload needs a one-rank workload (llama8b_z3, llama8b_z3_clip)")
    n, h = wl.n_ranks, wl.hyper
    dev = torch.device("cuda:0")
    L = z.zero_pack(n, wl.unit_numel)
    G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
    S = L.shard
    grads = torch.empty(n, S, dtype=torch.bfloat16, device=dev)
    for r in range(n):
        synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, 1, r))
    g_red = torch.empty(S, dtype=torch.float32, device=dev)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, wl.rank) // 8, dtype=torch.float64, device=dev)
    master = torch.empty(S, dtype=torch.float32)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    chunk = args.chunk
    gst = torch.zeros(2 * chunk, dtype=torch.float32, pin_memory=True)
    ost = torch.zeros(2 * chunk, dtype=torch.int16, pin_memory=True)
    d_out = torch.zeros(S, dtype=torch.int16, device=dev)
    s_down, s_up = torch.cuda.Stream(), torch.cuda.Stream()
    gl = list(grads)
    sc = z.zero_adamw_scalars_for(1, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0)

    def step():
        nonlocal sc
        ss = z.zero_gradnorm(L, wl.rank, gl, Lc, float(n), g_red, Lc, ws)
        sc.clip_coef = z.zero_clip_coef(ss, wl.clip_max_norm) if wl.clip_max_norm else 1.0
        t0 = time.perf_counter()
        z.zero_offload_step(L, wl.rank, g_red, gst, master, m, v, ost, d_out, chunk, sc,
                            args.threads, s_down, s_up)
        dt = time.perf_counter() - t0
        sc = z.zero_adamw_scalars_next(sc)
        return dt

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    off = [step() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    off_s = float(np.mean(off))
    res = {"metric": "offload optimizer-step shard elements/sec (GPU reduce + PCIe + host step)",
           "value": S * args.steps / wall, "unit": "elements/s", "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
           "dtype": "f32", "data": "synthetic",
           "config": {"workload": wl.name, "simulated_ranks": n, "elements_per_step": int(S),
                      "chunk": chunk, "threads": args.threads if args.threads > 0 else os.cpu_count(),
                      "offload_ms": off_s * 1e3,
                      "pcie_GBps": 6.0 * S / off_s / 1e9,
                      "host_GBps": 30.0 * S / off_s / 1e9}}
    print(json.dumps(res))


def reshard_layouts(R, z, workloads):
    units = [list(u) for u in R.units]
    A = z.zero_pack(R.from_ranks, workloads.unit_numels(units))
    shapes = workloads.param_shapes(units)
    numel = [workloads.numel_of(sh) for sh in shapes]
    row_len = workloads.row_lengths(shapes)
    B = z.zero_pack_rows(R.to_ranks, numel, row_len)
    return A, B, workloads.unit_numels(units), numel, row_len


def reshard_cpu_baseline(R, seconds: float):
    """The oracle's reshard (serial C) on contiguous spans of the same
    destination shard, from the same source layout, until the budget is
    spent: on one thread, then on as many threads as the host share allows
    (up to 16), each with its own destination spans.  Returns destination
    elements per second."""
    import threading

    import numpy as np

    import oracle
    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import workloads

    A, B, units_a, numel, row_len = reshard_layouts(R, z, workloads)
    # the oracle reads only the source elements the spans need; the rest of
    # each source shard may hold anything, so the sources are views of one
    # shared array (the oracle's inputs are host memory)
    shared = np.random.default_rng(R.seed).standard_normal(A.shard).astype(np.float32)
    src = [shared] * R.from_ranks
    span = 1 << 14
    oracle.load()

    def run(threads):
        counts = [0] * threads
        go = threading.Barrier(threads + 1)
        stop = threading.Event()

        def worker(i):
            k0 = (i * 104729 * span) % max(B.shard - span, 1)
            go.wait()
            while not stop.is_set():
                k1 = min(k0 + span, B.shard)
                oracle.reshard_span(units_a, R.from_ranks, src, R.to_ranks, R.dst_rank, k0, k1,
                                    row_b=row_len, numel_b=numel)
                counts[i] += k1 - k0
                k0 = (k0 + 7919 * span) % max(B.shard - span, 1)

        ts = [threading.Thread(target=worker, args=(i,)) for i in range(threads)]
        for t in ts:
            t.start()
        go.wait()
        t0 = time.perf_counter()
        time.sleep(seconds)
        stop.set()
        for t in ts:
            t.join()
        return sum(counts), time.perf_counter() - t0

    done, el = run(1)
    res = {"value": done / el, "unit": "elements/s", "cores": 1, "kind": "oracle",
           "sample": f"{done} destination elements in {span}-element spans spread over the "
                     f"{B.shard}-element shard, serial C, {el:.1f} s"}
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = min(16, avail)
    if threads > 1:
        done_t, el_t = run(threads)
        res["all_cores"] = {"value": done_t / el_t, "unit": "elements/s", "cores": threads,
                            "sample": f"{threads} threads, each running the serial oracle on its "
                                      f"own spans: {done_t} elements in {el_t:.1f} s"}
    return res


def reshard_bench(args):
    """One destination rank's fp32 state shard resharded on the device from
    the flat block layout to the row-aligned per-parameter layout; the
    sources are every source rank's shard, resident in HBM."""
    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import synth, workloads

    R = workloads.RESHARDS[args.reshard]
    dev = torch.device("cuda:0")
    A, B, units_a, numel, row_len = reshard_layouts(R, z, workloads)
    src = []
    for q in range(R.from_ranks):
        t = torch.empty(A.shard, dtype=torch.float32, device=dev)
        synth.fill_normal_(t, 0.02, synth.seed_of(R.seed, synth.TAG_MASTER, 0, q))
        src.append(t)
    dst = torch.empty(B.shard, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sp = z.reshard_pointer_array(src)   # marshalled once, outside the timed loop
    for _ in range(args.warmup):
        z.zero_reshard(A, src, B, R.dst_rank, dst, stream, src_ptrs=sp)
    torch.cuda.synchronize()
    # two events bracket the timed region on the launch stream; the average
    # call is the span / K (an event pair around every call would add its
    # own markers to each call's time)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        z.zero_reshard(A, src, B, R.dst_rank, dst, stream, src_ptrs=sp)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_s = e0.elapsed_time(e1) / 1e3 / args.steps
    per_call = []
    for _ in range(10):   # per-call spread, after the timed region
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        z.zero_reshard(A, src, B, R.dst_rank, dst, stream, src_ptrs=sp)
        b.record(stream)
        per_call.append((a, b))
    torch.cuda.synchronize()
    per_ms = sorted(a.elapsed_time(b) for a, b in per_call)
    nbytes, elements = z.zero_reshard_traffic(A, B, R.dst_rank, z.ZERO_F32)
    achieved = nbytes / call_s / 1e9
    box_copy = None if args.no_box_copy else box_copy_ceiling(z, torch, stream)
    result = {
        "metric": "checkpoint reshard destination elements/sec and achieved HBM GB/s",
        "value": elements * args.steps / wall, "unit": "elements/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": R.name, "description": R.description,
                   "from": f"{len(units_a)} flat units, N={R.from_ranks}",
                   "to": f"{len(numel)} row-aligned units, N={R.to_ranks}",
                   "dst_rank": R.dst_rank, "elements_per_step": int(elements),
                   "algorithmic_bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "kernel": "copy_batch_kernel (all launches of one reshard)",
                     "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBPS, "traffic": measured_traffic(R.name),
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": call_s * 1e3,
                     "timing": "HIP events on the launch stream at the two ends of the timed "
                               "region; average = span / steps",
                     "per_call_ms": {"median": float(np.median(per_ms)), "min": per_ms[0],
                                     "calls": len(per_ms),
                                     "timing": "an event pair around each call, 10 calls after "
                                               "the timed region"},
                     "launches_per_call": "one reshard = several copy_batch_kernel launches "
                                          "back to back; achieved and traffic are per call",
                     "box_copy_GBps": box_copy,
                     "frac_of_box_copy": achieved / box_copy if box_copy else None},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del src, dst
        torch.cuda.empty_cache()
        result["cpu_baseline"] = reshard_cpu_baseline(R, args.cpu_seconds)
    print(json.dumps(result))


def workload_from_args(args):
    """The named workload, at --ranks N if given."""
    import dataclasses

    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS
    wl = WORKLOADS[args.workload]
    if args.ranks and args.ranks != wl.n_ranks:
        wl = dataclasses.replace(wl, n_ranks=args.ranks, name=f"{wl.name}_n{args.ranks}",
                                 description=wl.description + f" (at N = {args.ranks})")
    clip = getattr(args, "clip", None)
    if clip is not None and clip != wl.clip_max_norm:
        wl = dataclasses.replace(wl, clip_max_norm=clip, name=f"{wl.name}_clip{clip:g}",
                                 description=wl.description + f" (clipped at {clip:g})")
    rank = getattr(args, "rank", None)
    if rank is not None and rank != wl.rank:
        if not 0 <= rank < wl.n_ranks:
            raise SystemExit(f"--rank must be in 0..{wl.n_ranks - 1}")
        wl = dataclasses.replace(wl, rank=rank, name=f"{wl.name}_r{rank}",
                                 description=wl.description + f" (rank {rank}'s shard only)")
    return wl


def stagger_plan(sizes, step_bytes, gap_bytes=0, toggle=False, alias_fix=False):
    """Buffer offsets in one allocation with buffer i at phase (i * step) mod
    2 MiB (step 0: every buffer at phase 0), and gap_bytes (whole 2 MiB pages)
    more between consecutive buffers; toggle: one 2 MiB page more wherever a
    buffer would start a multiple of 4 MiB (plus the phase step) after the
    one before; alias_fix: the library's exception (one page more where a
    buffer of a run of more than 32 equal sizes would start a multiple of
    2 MiB plus 32 MiB, modulo 64 MiB, after the one before).  The library's
    zero_arena_plan is this rule with a 256 KiB step, no gap, no toggle and
    the exception.  For sweeping the placement."""
    page = 2 << 20
    offs, at = [], 0
    run_begin = run_end = 0
    for i, b in enumerate(sizes):
        if i >= run_end:
            run_begin, run_end = i, i + 1
            while run_end < len(sizes) and sizes[run_end] == b:
                run_end += 1
        if i:
            at += gap_bytes
        want = (i * step_bytes) % page
        at += (want - at % page) % page
        if toggle and i and (at - offs[-1]) % (2 * page) < page:
            at += page
        if alias_fix and i > run_begin and run_end - run_begin > 32 and \
                ((at - offs[-1]) // page) % 32 == 16:
            at += page
        offs.append(at)
        at += b
    return offs, at


def setup_step(wl, fused=False, stage_chunk=None, stagger_kib=None, norm_only=None, grad_dtype="bf16",
               gap_mib=0, toggle=False):
    """The benchmark's resident inputs and its step, as bench.py times them:
    every streamed buffer in one allocation placed by zero_arena_plan, the
    workload's seeded gradients (the same every step) and master weights,
    zeroed m / v / out, gradient pointers marshalled once, and `one_step(t,
    ev)` -- the staged step above 32 ranks, the device-side clip chain for the
    clipped workload, else the fused step.  Returns a namespace of them."""
    import types

    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import synth

    n, h = wl.n_ranks, wl.hyper
    dev = torch.device("cuda:0")
    L = z.zero_pack(n, wl.unit_numel)
    G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
    gidx = G if wl.grad_index == "global" else Lc
    sidx = G if wl.rank < 0 else Lc
    oidx = G if wl.out_index == "global" else Lc
    ge = L.padded if gidx == G else L.shard
    se = L.padded if sidx == G else L.shard
    oe = L.padded if oidx == G else L.shard
    clip = wl.clip_max_norm is not None

    # -- inputs, resident before the timed region --------------------------------------
    # Every streamed buffer in one allocation, placed by zero_arena_plan
    # (gradients, master, m, v, out, and the reduced gradient when clipping).
    # Unclipped above 32 bf16 / 24 fp32 ranks: the staged step, through a
    # workspace chunk the memory-side cache holds (zero_step_staged).
    stages = n > 32 or (grad_dtype == "f32" and n > 24)
    ws_elems = 0 if clip or fused or not stages else \
        z.zero_step_staged_workspace_bytes(L, wl.rank, n) // 4
    if ws_elems and stage_chunk:   # a chosen chunk (whole 512-element tiles) plus the spare
        ws_elems = stage_chunk + 4
    staged = ws_elems > 0
    gdt = torch.float32 if grad_dtype == "f32" else torch.bfloat16
    specs = [(ge, gdt)] * n + [(se, torch.float32)] * 3 + [(oe, torch.int16)]
    if clip:
        specs.append((se, torch.float32))
    if staged:
        specs.append((ws_elems, torch.float32))
    sizes = [cnt * torch.empty(0, dtype=dt).element_size() for cnt, dt in specs]
    if stagger_kib is None:
        offs, total = z.zero_arena_plan(sizes)
    else:
        offs, total = stagger_plan(sizes, stagger_kib << 10, gap_mib << 20, toggle)
    arena = torch.empty(total, dtype=torch.uint8, device=dev)
    views = [arena[o:o + b].view(dt) for o, b, (_, dt) in zip(offs, sizes, specs)]
    grads, (master, m, v, out) = views[:n], views[n:n + 4]
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m.zero_()
    v.zero_()
    out.zero_()
    for r in range(n):
        synth.fill_grad_(grads[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, 1, r))
    gp = z.grad_pointer_array(grads)
    if staged:
        stage_ws = views[n + 4]
    if clip:
        g_red = views[n + 4]
        ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, wl.rank) // 8, dtype=torch.float64, device=dev)
        ss_dev = torch.zeros(1, dtype=torch.float64, device=dev)
        coef_dev = torch.zeros(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sc = z.zero_adamw_scalars_for(1, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0)

    def one_step(t, ev=None):
        # ev: (start, end) events around the dominant kernel on the launch
        # stream -- the norm pass for the clipped workload, else the step.
        nonlocal sc
        sc = z.zero_adamw_scalars_for(t, h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0) \
            if t == 1 else z.zero_adamw_scalars_next(sc)
        if clip:
            # norm pass -> coefficient on the device -> step reading it: no
            # host round trip inside the step
            if ev:
                ev[0].record(stream)
            z.zero_gradnorm_async(L, wl.rank, grads, gidx, float(n), None if norm_only == "no_g" else g_red,
                                  sidx, ws, ss_dev, stream)
            if ev:
                ev[1].record(stream)
            if norm_only:   # the norm pass alone (--norm-only), with or without writing g
                return
            z.zero_clip_coef_async(ss_dev, wl.clip_max_norm, coef_dev, stream)
            z.zero_step_device_clip(L, wl.rank, [g_red], sidx, 1.0, master, m, v, sidx, out, oidx, sc,
                                    coef_dev, stream)
        else:
            if ev:
                ev[0].record(stream)
            if staged:
                z.zero_step_staged(L, wl.rank, None, gidx, float(n), master, m, v, sidx, out, oidx, sc,
                                   stage_ws, stream, grad_ptrs=gp)
            else:
                z.zero_step(L, wl.rank, None, gidx, float(n), master, m, v, sidx, out, oidx, sc, stream,
                            grad_ptrs=gp)
            if ev:
                ev[1].record(stream)

    ns = types.SimpleNamespace(
        wl=wl, n=n, h=h, L=L, gidx=gidx, sidx=sidx, oidx=oidx, se=se, clip=clip, staged=staged,
        ws_elems=ws_elems, arena=arena, grads=grads, master=master, m=m, v=v, out=out,
        stream=stream, one_step=one_step, grad_dtype=z.ZERO_F32 if grad_dtype == "f32" else z.ZERO_BF16)
    if clip:
        ns.g_red, ns.ss_dev, ns.coef_dev = g_red, ss_dev, coef_dev
    if staged:
        ns.stage_ws = stage_ws
    return ns


def streamed_bench(args):
    """The per-unit step streamed beside a backward stand-in (one GPU).

    "ZeRO and FSDP sharding", How it works: each unit's gradients are
    reduce-scattered as soon as backward has produced them, and the unit's
    shards stepped; "ZeRO: Three Ledgers", section 4: bucketed reduce-scatter
    makes gradients transient.  For the all-ranks workload (every simulated
    rank's shards, GLOBAL buckets) a producer writes each unit's N gradient
    buckets into one of two bucket slots, last unit first (backward order):

      gemm -- every 2-D parameter's weight gradient dW = dY^T X with `tokens`
              rows per simulated rank (bf16 MFMA through torch.matmul, written
              straight into the bucket): the shape of backward's weight-
              gradient work (the vector parameters, 0.05 % of a GPT-2 block,
              keep their values: thousands of tiny launches per pass would
              make the stand-in launch-bound);
      copy -- the unit's buckets copied from resident gradients (HBM-bound).

    Three passes over the whole model, each timed between synchronizations
    (median of `steps` repetitions after `warmup`): the producer alone;
    serial -- produce unit k, then step it (zero_step_units), one stream;
    overlapped -- produce on the main stream, step unit k on a side stream
    while unit k-1 is produced (events order the slot reuse).  Also the
    whole-model step in one zero_step call.  hidden_fraction = (serial -
    overlapped) / step-only time: how much of the optimizer step the overlap
    hides behind the producer."""
    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd import synth, workloads
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS

    wl = workload_from_args(args)
    if wl.rank >= 0 or wl.grad_index != "global":
        raise SystemExit("--streamed runs the all-ranks workloads (gpt2l, gpt2l_block)")
    n, h = wl.n_ranks, wl.hyper
    dev = torch.device("cuda:0")
    L = z.zero_pack(n, wl.unit_numel)
    T = L.unit_table()
    U, P = L.n_units, L.padded
    G = z.ZERO_GLOBAL
    shapes = {"gpt2l": workloads.gpt2_large_units(),
              "gpt2l_block": [workloads.gpt2_block()]}[args.workload]
    shapes = [[s for _, s in u] for u in shapes]
    cap = int(T[:, 1].max())
    master = torch.empty(P, dtype=torch.float32, device=dev)
    synth.fill_normal_(master, wl.master_std, synth.seed_of(wl.seed, synth.TAG_MASTER))
    m, v = torch.zeros_like(master), torch.zeros_like(master)
    out = torch.zeros(P, dtype=torch.int16, device=dev)
    slots = torch.empty(2, n, cap, dtype=torch.bfloat16, device=dev)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    tok = args.tokens
    if args.producer == "gemm":
        # one contiguous activation matrix per input width, one dY^T per
        # output height (row slices of the tallest are contiguous)
        X = {k: (torch.randn(tok, k, device=dev) * 0.5).to(torch.bfloat16)
             for k in sorted({s[1] for u in shapes for s in u if len(s) == 2})}
        max_out = max(s[0] for u in shapes for s in u if len(s) == 2)
        dYT = (torch.randn(max_out, tok, device=dev) * 1e-3).to(torch.bfloat16)
        flops = 2.0 * tok * n * sum(s[0] * s[1] for u in shapes for s in u if len(s) == 2)
    else:
        src = torch.empty(n, P, dtype=torch.bfloat16, device=dev)
        for r in range(n):
            synth.fill_grad_(src[r], wl.grad_dist, wl.grad_scale, synth.seed_of(wl.seed, synth.TAG_GRAD, 1, r))
        flops = 0.0

    def produce(u, slot):
        pad = int(T[u, 1])
        if args.producer == "copy":
            off = int(T[u, 3])
            slots[slot, :, :pad].copy_(src[:, off:off + pad])
            return
        for r in range(n):
            at = 0
            for s in shapes[u]:
                k = workloads.numel_of(s)
                if len(s) == 2:   # dW [out, in] = dY^T [out, T] @ X [T, in]
                    torch.matmul(dYT[:s[0]], X[s[1]], out=slots[slot, r, at:at + k].view(s[0], s[1]))
                at += k

    sc_t = [0]

    def sc():
        sc_t[0] += 1
        return z.zero_adamw_scalars_for(sc_t[0], h["lr"], h["b1"], h["b2"], h["eps"], h["wd"], 1.0)

    def step_unit(u, slot, stream, s):
        pad = int(T[u, 1])
        z.zero_step_units(L, -1, u, u + 1, [slots[slot, r, :pad] for r in range(n)], G, float(n),
                          master, m, v, G, out, G, s, stream=stream)

    order = list(range(U - 1, -1, -1))

    def producer_only():
        for i, u in enumerate(order):
            produce(u, i % 2)

    def serial():
        s = sc()
        for i, u in enumerate(order):
            produce(u, i % 2)
            step_unit(u, i % 2, main, s)

    def overlapped():
        s = sc()
        stepped = [None] * U
        for i, u in enumerate(order):
            if i >= 2:
                main.wait_event(stepped[i - 2])
            produce(u, i % 2)
            ready = torch.cuda.Event()
            ready.record(main)
            side.wait_event(ready)
            step_unit(u, i % 2, side, s)
            stepped[i] = torch.cuda.Event()
            stepped[i].record(side)
        main.wait_event(stepped[-1])

    def overlapped_uncapped():
        # the step's occupancy cap reserves LDS per workgroup, which can keep
        # a GEMM's workgroups from becoming resident beside it: uncapped here
        z.zero_set_waves_per_cu(z.ZERO_CAP_STEP, 0)
        try:
            overlapped()
        finally:
            z.zero_set_waves_per_cu(z.ZERO_CAP_STEP, -1)

    def steps_only():
        s = sc()
        for i, u in enumerate(order):
            step_unit(u, i % 2, main, s)

    grads_full = None

    def whole_step():
        nonlocal grads_full
        if grads_full is None:   # one resident set of N full gradients (12.4 GB for gpt2l)
            grads_full = [torch.zeros(P, dtype=torch.bfloat16, device=dev) for _ in range(n)]
        z.zero_step(L, -1, grads_full, G, float(n), master, m, v, G, out, G, sc())

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(args.steps):
            t0 = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts)) * 1e3, float(np.min(ts)) * 1e3

    res = {}
    for name, fn in (("producer_only", producer_only), ("steps_only", steps_only),
                     ("serial", serial), ("overlapped", overlapped), ("serial_again", serial),
                     ("overlapped_again", overlapped), ("overlapped_uncapped", overlapped_uncapped)):
        res[name] = timed(fn)
    del slots
    if args.producer == "copy":
        del src
    torch.cuda.empty_cache()
    res["whole_model_step"] = timed(whole_step)
    ser = min(res["serial"][0], res["serial_again"][0])
    ovl = min(res["overlapped"][0], res["overlapped_again"][0])
    step_ms = res["steps_only"][0]
    step_bytes, elements = z.zero_step_traffic(L, -1, n, z.ZERO_BF16, True)
    result = {
        "metric": "streamed per-unit optimizer step beside a backward stand-in: fraction of the "
                  "step's time hidden by overlap",
        "value": (ser - ovl) / step_ms,
        "unit": "fraction of step time",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "simulated_ranks": n, "units": U, "elements": int(elements),
                   "producer": args.producer, "tokens_per_rank": tok if args.producer == "gemm" else None,
                   "producer_tflop_per_pass": flops / 1e12 if flops else None,
                   "bucket_slots_bytes": 2 * n * cap * 2,
                   "full_gradients_bytes": n * P * 2},
        "ms": {k: {"median": a, "min": b} for k, (a, b) in res.items()},
        "serial_ms": ser,
        "overlapped_ms": ovl,
        "steps_only_hbm_GBps": step_bytes / (step_ms / 1e3) / 1e9,
        "whole_model_step_hbm_GBps": step_bytes / (res["whole_model_step"][0] / 1e3) / 1e9,
        "producer_tflops": flops / (res["producer_only"][0] / 1e3) / 1e12 if flops else None,
        "timing": "wall clock between synchronizations, median of `steps` passes after `warmup`",
    }
    print(json.dumps(result))


def sweep_waves(args, wl, S):
    """Time the workload's step at several occupancy caps of one kernel
    family, in interleaved rounds in one process (the buffers stay where they
    are, so placement does not differ between caps).  Prints one JSON line
    with each cap's % of 8 TB/s per round and the best cap."""
    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z

    fam, caps = args.sweep_waves.split(":")
    kind = {"step": z.ZERO_CAP_STEP, "step1": z.ZERO_CAP_STEP1, "norm": z.ZERO_CAP_NORM}[fam]
    caps = [int(c) for c in caps.split(",")]
    n = S.n
    if S.clip:
        step_bytes, _ = z.zero_step_traffic(S.L, wl.rank, 1, z.ZERO_F32, True)
        norm_bytes, _ = z.zero_gradnorm_traffic(S.L, wl.rank, n, S.grad_dtype, True)
        job_bytes = step_bytes + norm_bytes
    else:
        job_bytes, _ = z.zero_step_traffic(S.L, wl.rank, n, S.grad_dtype, True)
    t = 0
    for _ in range(args.warmup):
        t += 1
        S.one_step(t)
    res = {c: [] for c in caps}
    for _ in range(args.rounds):
        for c in caps:
            z.zero_set_waves_per_cu(kind, c)
            t += 1
            S.one_step(t)     # one untimed call at the new cap
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(S.stream)
            for _ in range(args.steps):
                t += 1
                S.one_step(t)
            b.record(S.stream)
            torch.cuda.synchronize()
            ms = a.elapsed_time(b) / args.steps
            res[c].append(100.0 * job_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS)
    z.zero_set_waves_per_cu(kind, -1)
    med = {c: float(np.median(v)) for c, v in res.items()}
    print(json.dumps({"sweep": fam, "workload": wl.name, "simulated_ranks": n,
                      "staged": S.staged, "clip": S.clip, "steps_per_point": args.steps,
                      "rounds": args.rounds, "pct_of_8TBps": res, "median": med,
                      "best": max(med, key=med.get),
                      "default": z.zero_get_waves_per_cu_for(kind, n, S.grad_dtype, S.staged)}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the sharded step for N "
              "ranks runs here as N simulated ranks' buffers in one GPU's memory", file=sys.stderr)
        sys.exit(2)
    if args.reshard:
        reshard_bench(args)
        return
    if args.streamed:
        streamed_bench(args)
        return
    if args.offload:
        offload_bench(args)
        return
    if args.host_step:
        host_step_bench(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    import fsdp_sharded_optimizer_flat_amd as z
    from fsdp_sharded_optimizer_flat_amd.workloads import WORKLOADS

    wl = workload_from_args(args)
    if args.grad_dtype != "bf16" and not args.no_cpu_baseline:
        raise SystemExit("--grad-dtype f32 is a variant without the CPU leg: add --no-cpu-baseline")
    if args.norm_only and wl.clip_max_norm is None:
        raise SystemExit("--norm-only needs the clipped workload (llama8b_z3_clip)")
    if args.gap_mib and (args.stagger_kib is None or args.gap_mib < 0 or args.gap_mib % 2):
        raise SystemExit("--gap-mib takes a non-negative multiple of 2, with --stagger-kib")
    if args.toggle and args.stagger_kib is None:
        raise SystemExit("--toggle goes with --stagger-kib")
    S = setup_step(wl, fused=args.fused, stage_chunk=args.stage_chunk, stagger_kib=args.stagger_kib,
                   norm_only=("no_g" if args.no_g else "g") if args.norm_only else None,
                   grad_dtype=args.grad_dtype, gap_mib=args.gap_mib, toggle=args.toggle)
    gdt = z.ZERO_F32 if args.grad_dtype == "f32" else z.ZERO_BF16
    if args.sweep_waves:
        sweep_waves(args, wl, S)
        return
    n, h, L, gidx, sidx, oidx, se = S.n, S.h, S.L, S.gidx, S.sidx, S.oidx, S.se
    clip, staged, ws_elems, stream, one_step = S.clip, S.staged, S.ws_elems, S.stream, S.one_step

    t = 0
    for _ in range(args.warmup):
        t += 1
        one_step(t)
    torch.cuda.synchronize()

    # The clipped workload's dominant kernel (the norm pass) is one part of
    # each step: HIP events around every norm pass.  Otherwise the step is
    # the whole of each iteration: two events bracket the timed region on the
    # launch stream (an event pair around every call would add its own
    # markers to each call's time), and the average call is the span / K.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps if clip else 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if not clip:
        events[0][0].record(stream)
    for k in range(args.steps):
        t += 1
        one_step(t, events[k] if clip else None)
    if not clip:
        events[0][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if clip:
        avg_launch_s = float(np.mean([a.elapsed_time(b) for a, b in events])) / 1e3
        timing = "HIP events on the launch stream around every timed norm pass"
    else:
        avg_launch_s = events[0][0].elapsed_time(events[0][1]) / 1e3 / args.steps
        timing = ("HIP events on the launch stream at the two ends of the timed region; "
                  "average = span / steps")
    elements = se if wl.rank < 0 else L.shard
    fused_bytes, _ = z.zero_step_traffic(L, wl.rank, n, gdt, True)  # 2N + 26 (4N + 26 for fp32)
    if clip:
        step_bytes, _ = z.zero_step_traffic(L, wl.rank, 1, z.ZERO_F32, True)
        norm_bytes, _ = z.zero_gradnorm_traffic(L, wl.rank, n, gdt, not args.no_g)
        if args.norm_only:
            step_bytes = 0.0
        job_bytes = step_bytes + norm_bytes   # 2N + 34: the bytes the two passes need
        dom_bytes, dom_name = norm_bytes, "norm_kernel (rank-sum + divide + fp32 g + binary64 sum of squares)"
    else:
        step_bytes, _ = z.zero_step_traffic(L, wl.rank, n, gdt, True)
        job_bytes = step_bytes
        dom_bytes, dom_name = step_bytes, "step_quad_kernel (fused rank-sum + AdamW + bf16 cast)"
        if staged:
            dom_name = ("staged step: stage_reduce_kernel + step_quad_kernel per workspace chunk "
                        "(all launches of one call; bytes as for the fused step)")
    achieved = dom_bytes / avg_launch_s / 1e9
    ms_per_step = wall / args.steps * 1e3
    value = elements * args.steps / wall

    # per-call spread, after the timed region: an event pair around each of
    # 10 more calls (whole iterations: norm pass, coefficient and step for
    # the clipped workload); reported beside, not in, `value` and `frac`
    per_call = []
    for _ in range(10):
        t += 1
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        one_step(t)
        b.record(stream)
        per_call.append((a, b))
    torch.cuda.synchronize()
    per_ms = sorted(a.elapsed_time(b) for a, b in per_call)

    traffic = None if args.fused or args.norm_only or args.stage_chunk or args.stagger_kib is not None \
        or args.grad_dtype != "bf16" \
        else measured_traffic(wl.name)
    box_copy = None if args.no_box_copy else box_copy_ceiling(z, torch, stream)

    result = {
        "metric": "optimizer-step shard elements/sec and achieved HBM GB/s (% of MI355X peak)",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "description": wl.description,
            "simulated_ranks": n,
            "units": len(wl.unit_numel),
            "params": int(L.numel),
            "elements_per_step": int(elements),
            "grad_dtype": args.grad_dtype,
            "state_dtype": "f32",
            "out_dtype": "bf16",
            "clip_max_norm": wl.clip_max_norm,
            "variant": ", ".join(v for v in (
                "fused step above 32 ranks" if args.fused else "",
                ("norm pass only, " + ("g not written" if args.no_g else "g written")) if args.norm_only else "",
                f"staged chunk {args.stage_chunk} elements" if args.stage_chunk else "",
                f"buffers staggered by {args.stagger_kib} KiB" if args.stagger_kib is not None else "",
                f"{args.gap_mib} MiB more between buffers" if args.gap_mib else "",
                "bases toggled off 4 MiB multiples" if args.toggle else "",
                "fp32 gradients" if args.grad_dtype == "f32" else "") if v)
                or None,
            "algorithmic_bytes_per_step": job_bytes,
            "bytes_per_element": job_bytes / elements,
            "hbm_GBps_whole_step": job_bytes / (wall / args.steps) / 1e9,
            "pct_of_peak_whole_step": 100.0 * job_bytes / (wall / args.steps) / 1e9 / PEAK_HBM_GBPS,
            "fused_convention_bytes_per_step": fused_bytes,
            "pct_of_peak_whole_step_fused_convention":
                100.0 * fused_bytes / (wall / args.steps) / 1e9 / PEAK_HBM_GBPS,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom_name,
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_ms": avg_launch_s * 1e3,
            "timing": timing,
            "per_call_ms": {"median": float(np.median(per_ms)), "min": per_ms[0], "calls": len(per_ms),
                            "timing": "an event pair around each call, 10 calls after the timed region"},
            "launches_per_call": (2 * -(-elements // (ws_elems or 1))) if staged else 1,
            "box_copy_GBps": box_copy,
            "frac_of_box_copy": achieved / box_copy if box_copy else None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del S, one_step   # the step's device buffers
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
