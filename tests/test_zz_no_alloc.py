"""zero_gradnorm_async_noalloc (no workspace: the partial sums live in the
library's own device array) against zero_gradnorm_async with a caller
workspace, through the C ABI: the same binary64 sum bit for bit and the same
reduced gradient, on calls in a row where a later call selects fewer
elements than the one before (stale partials of an earlier call must not
reach its sum), and both against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from gpu_common import DEV, to_np, bits32  # noqa: E402

Lc = z.ZERO_LOCAL


def _grads(L, n, seed):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    return [(torch.randn(L.shard, device=DEV, generator=gen) * 1e-3).to(torch.bfloat16)
            for _ in range(n)]


def _one_call(n, numel, rank, seed):
    L = z.zero_pack(n, numel)
    grads = _grads(L, n, seed)
    print(f"noalloc case n={n} numel={numel} rank={rank}", flush=True)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, rank) // 8 + 1, dtype=torch.float64, device=DEV)
    s_ref = torch.zeros(1, dtype=torch.float64, device=DEV)
    g_ref = torch.zeros(L.shard, device=DEV)
    z.zero_gradnorm_async(L, rank, grads, Lc, float(n), g_ref, Lc, ws, s_ref)
    s_new = torch.full((1,), float("nan"), dtype=torch.float64, device=DEV)
    g_new = torch.full((L.shard,), float("nan"), device=DEV)
    z.zero_gradnorm_async_noalloc(L, rank, grads, Lc, float(n), g_new, Lc, s_new)
    torch.cuda.synchronize()
    a, b = float(s_new.item()), float(s_ref.item())
    assert np.float64(a).view(np.uint64) == np.float64(b).view(np.uint64), (a, b)
    assert np.array_equal(bits32(to_np(g_new)), bits32(to_np(g_ref)))
    # the oracle: the reduced gradient bit for bit; the sum within the error
    # bound of the oracle's serial binary64 sum (n 2^-53 relative) and within
    # 1e-12 of a pairwise binary64 sum of the oracle's gradient
    hg = [to_np(g) for g in grads]
    og = oracle.reduced_grad(n, numel, rank, hg, grad_local=True, divisor=float(n))
    assert np.array_equal(bits32(to_np(g_new)), bits32(og))
    serial = oracle.sumsq(og)
    pair = float(np.sum(og.astype(np.float64) ** 2))
    assert abs(a - serial) <= og.size * 2.0 ** -53 * serial, (a, serial)
    assert abs(a - pair) <= 1e-12 * pair, (a, pair)
    # no reduced gradient requested: the same sum
    s2 = torch.full((1,), float("nan"), dtype=torch.float64, device=DEV)
    z.zero_gradnorm_async_noalloc(L, rank, grads, Lc, float(n), None, Lc, s2)
    torch.cuda.synchronize()
    assert float(s2.item()) == a
    return a


def test_noalloc_gradnorm_matches_workspace_call():
    big_units = [64 * 500_000, 64 * 77_777 + 5]
    big = _one_call(64, big_units, 5, 11)                 # 577,778 elements, 1,131 partials
    small = _one_call(8, [1000, 77, 8 * 3], 3, 12)        # 138 elements, 3 partials
    assert big != small
    again = _one_call(64, big_units, 5, 11)               # the large case again
    assert again == big


def test_noalloc_gradnorm_empty_selection_writes_zero():
    L = z.zero_pack(4, [0])
    grads = [torch.zeros(1, dtype=torch.bfloat16, device=DEV) for _ in range(4)]
    s = torch.full((1,), 5.0, dtype=torch.float64, device=DEV)
    z.zero_gradnorm_async_noalloc(L, 1, grads, Lc, 4.0, None, Lc, s)
    torch.cuda.synchronize()
    assert float(s.item()) == 0.0

