"""The library's launch sequences captured in HIP graphs (torch CUDAGraph)
and replayed: the staged step (compiled and run-time reduction), one rank's
step over several units in shared launches (vector pieces on a shifted wave
grid), that rank's clipped chain (segments of the norm pass in shared
launches, the coefficient and the step on the device), and the same chain
through the no-allocation norm entry point.  Every replay runs between eager
work and synchronizations and is compared bit for bit with the same calls
made eagerly; the eager state is held to the oracle once, after the last
step.  The library allocates nothing and launches only kernels (no memset
nodes), so each sequence can be captured as it stands."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from fsdp_sharded_optimizer_flat_amd.workloads import GPT_HYPER  # noqa: E402
from gpu_common import DEV, assert_same_bf16, assert_same_f32, hyper_args, scalars, to_np  # noqa: E402

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL
H = GPT_HYPER


def log(msg):
    print(msg, flush=True)


def _state(n_elems, seed):
    w0 = np.random.default_rng(seed).normal(0, 0.02, n_elems).astype(np.float32)

    def fresh():
        return [torch.from_numpy(w0).to(DEV), torch.zeros(n_elems, device=DEV),
                torch.zeros(n_elems, device=DEV), torch.zeros(n_elems, dtype=torch.int16, device=DEV)]
    return w0, fresh


def _replay_against_eager(step_fn, fresh, steps=3):
    """Capture step_fn(t, state, stream) once per step count on a side stream,
    then replay step t and run the same step eagerly on a second state after
    it; compare the two after every replay.  Returns the eager state."""
    # one eager step on a throwaway state first: the library's one-time set-up
    # (device properties, code objects loaded on first launch) stays out of
    # the capture
    step_fn(1, fresh(), None)
    torch.cuda.synchronize()
    cap = fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graphs = []
    for t in range(1, steps + 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step_fn(t, cap, s)
        graphs.append(g)
    torch.cuda.synchronize()
    for a, b in zip(cap, fresh()):   # capturing ran nothing: start both from the same state
        a.copy_(b)
    eager = fresh()
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        graphs[t - 1].replay()
        torch.cuda.synchronize()
        step_fn(t, eager, None)
        torch.cuda.synchronize()
        for name, a, b in zip(("master", "exp_avg", "exp_avg_sq"), cap[:3], eager[:3]):
            assert_same_f32(to_np(a), to_np(b), f"replay {t} {name}")
        assert_same_bf16(to_np(cap[3]), to_np(eager[3]), f"replay {t} out")
    return eager


def _oracle_rank(n, numel, rank, grads_np, w0, steps, grad_local, clip_max=None):
    """The oracle's rank step repeated `steps` times on the same gradients,
    LOCAL state and output; with clip_max, each step clipped by the oracle's
    own coefficient of its own reduced gradient."""
    S = w0.size
    w, m, v = w0.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)
    out = np.zeros(S, np.uint16)
    clip = 1.0
    if clip_max is not None:
        og = oracle.reduced_grad(n, numel, rank, grads_np, grad_local=grad_local, divisor=float(n))
        clip = oracle.clip_coef(oracle.sumsq(og), clip_max)
        assert clip < 1.0
    for t in range(1, steps + 1):
        oracle.zero_step_rank(n, numel, rank, grads_np, grad_local=grad_local, divisor=float(n), clip=clip,
                              master=w, m=m, v=v, state_global=False, out=out, out_gather=False, t=t,
                              **hyper_args(H))
    return w, m, v, out


def _check_oracle(state, ref, what):
    for name, a, b in zip(("master", "exp_avg", "exp_avg_sq"), state[:3], ref[:3]):
        assert_same_f32(to_np(a), b, f"{what} {name} vs oracle")
    assert_same_bf16(to_np(state[3]), ref[3], f"{what} out vs oracle")


@pytest.mark.parametrize("n", [48, 64])
def test_staged_step_in_a_graph(n):
    """The staged step (rank-sum chunks through a workspace, then the step on
    them) at a rank count with a compiled reduction (64) and one on the
    run-time kernel (48); a small workspace gives several chunks."""
    numel = [n * 70_001, n * 9_999 + 7, n * 130]
    L = z.zero_pack(n, numel)
    rank = 5
    log(f"graph staged n={n} shard={L.shard}")
    gen = torch.Generator(device=DEV).manual_seed(100 + n)
    grads = [(torch.randn(L.shard, device=DEV, generator=gen) * 1e-3).to(torch.bfloat16) for _ in range(n)]
    gp = z.grad_pointer_array(grads)
    ws = torch.zeros(64 * 1024 + 4, dtype=torch.float32, device=DEV)   # 64K-element chunks
    w0, fresh = _state(L.shard, 200 + n)

    def step(t, st, stream):
        z.zero_step_staged(L, rank, None, Lc, float(n), st[0], st[1], st[2], Lc, st[3], Lc,
                           scalars(t, H), ws, stream, grad_ptrs=gp)

    eager = _replay_against_eager(step, fresh)
    ref = _oracle_rank(n, numel, rank, [to_np(g) for g in grads], w0, 3, grad_local=True)
    _check_oracle(eager, ref, f"staged n={n}")


def _rank_slice_case():
    """One odd rank's slice of several units from full (GLOBAL) gradient
    buffers: unit shards of 2,459,680-like sizes (a multiple of 32 but not of
    64 elements) put the odd ranks' slices half a cache line off, which the
    shared-launch step covers with a shifted wave grid."""
    n = 8
    numel = [8 * 96_032, 8 * 64_032, 8 * 160_000, 8 * 32 + 8 * 5]
    L = z.zero_pack(n, numel)
    rank = 3
    gen = torch.Generator(device=DEV).manual_seed(77)
    grads = [(torch.randn(L.padded, device=DEV, generator=gen) * 3e-2).to(torch.bfloat16) for _ in range(n)]
    return n, numel, L, rank, grads


def test_rank_slice_step_in_a_graph():
    n, numel, L, rank, grads = _rank_slice_case()
    log(f"graph rank-slice step n={n} units={len(numel)} shard={L.shard}")
    gp = z.grad_pointer_array(grads)
    w0, fresh = _state(L.shard, 300)

    def step(t, st, stream):
        z.zero_step(L, rank, None, G, float(n), st[0], st[1], st[2], Lc, st[3], Lc, scalars(t, H), stream,
                    grad_ptrs=gp)

    eager = _replay_against_eager(step, fresh)
    ref = _oracle_rank(n, numel, rank, [to_np(g) for g in grads], w0, 3, grad_local=False)
    _check_oracle(eager, ref, "rank-slice step")


@pytest.mark.parametrize("noalloc", [False, True], ids=["workspace", "noalloc"])
def test_rank_slice_clipped_chain_in_a_graph(noalloc):
    """norm pass (segments in shared launches) -> coefficient -> step on the
    reduced gradient, all on the device, with the norm's partials in a caller
    workspace or in the library's own array (the no-allocation entry point,
    meant for code under capture)."""
    n, numel, L, rank, grads = _rank_slice_case()
    log(f"graph rank-slice clipped chain noalloc={noalloc}")
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8, dtype=torch.float64, device=DEV)
    g_red = torch.zeros(L.shard, device=DEV)
    ssd = torch.zeros(1, dtype=torch.float64, device=DEV)
    coef = torch.zeros(1, dtype=torch.float32, device=DEV)
    w0, fresh = _state(L.shard, 400)
    max_norm = 0.05

    def step(t, st, stream):
        if noalloc:
            z.zero_gradnorm_async_noalloc(L, rank, grads, G, float(n), g_red, Lc, ssd, stream)
        else:
            z.zero_gradnorm_async(L, rank, grads, G, float(n), g_red, Lc, ws, ssd, stream)
        z.zero_clip_coef_async(ssd, max_norm, coef, stream)
        z.zero_step_device_clip(L, rank, [g_red], Lc, 1.0, st[0], st[1], st[2], Lc, st[3], Lc, scalars(t, H),
                                coef, stream)

    if noalloc:   # the library looks up its array's device address on the first call, eagerly
        z.zero_gradnorm_async_noalloc(L, rank, grads, G, float(n), None, Lc, ssd)
        torch.cuda.synchronize()
    eager = _replay_against_eager(step, fresh)
    ref = _oracle_rank(n, numel, rank, [to_np(g) for g in grads], w0, 3, grad_local=False,
                       clip_max=max_norm)
    _check_oracle(eager, ref, f"clipped chain noalloc={noalloc}")
