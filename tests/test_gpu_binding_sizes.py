"""On the GPU, a device buffer shorter than the call's extent is refused by
the binding before the C call: no kernel is launched, nothing is written."""
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from gpu_common import DEV  # noqa: E402

G, Lc = z.ZERO_GLOBAL, z.ZERO_LOCAL


def _sc():
    return z.zero_adamw_scalars_for(1, 1e-3, 0.9, 0.95, 1e-8, 0.1, 1.0)


def _bufs(L, n, ext):
    gs = [torch.ones(ext, dtype=torch.bfloat16, device=DEV) for _ in range(n)]
    st = [torch.full((ext,), 0.5, device=DEV) for _ in range(3)]
    out = torch.zeros(ext, dtype=torch.int16, device=DEV)
    return gs, st, out


@pytest.mark.parametrize("which", ["grad", "master", "exp_avg_sq", "out", "prepared"])
def test_step_short_device_buffer(which):
    n = 4
    L = z.zero_pack(n, [1000, 37])
    gs, st, out = _bufs(L, n, L.shard)
    prepared = None
    if which in ("grad", "prepared"):
        gs[1] = gs[1][:-1]
        if which == "prepared":
            prepared = z.grad_pointer_array(gs)
    elif which == "out":
        out = out[:-1]
    else:
        k = ["master", "exp_avg", "exp_avg_sq"].index(which)
        st[k] = st[k][:-1]
    before = [t.clone() for t in st] + [out.clone()]
    with pytest.raises(ValueError):
        z.zero_step(L, 2, gs, Lc, float(n), *st, Lc, out, Lc, _sc(), grad_ptrs=prepared)
    torch.cuda.synchronize()
    for a, b in zip(st + [out], before):
        assert torch.equal(a, b)


def test_gradnorm_and_reshard_short_device_buffers():
    n = 4
    L = z.zero_pack(n, [1000, 37])
    gs, _, _ = _bufs(L, n, L.padded)
    ws = torch.zeros(z.zero_gradnorm_workspace_bytes(L, -1) // 8, dtype=torch.float64, device=DEV)
    g_out = torch.zeros(L.padded - 1, device=DEV)
    with pytest.raises(ValueError, match="g_out"):
        z.zero_gradnorm(L, -1, gs, G, float(n), g_out, G, ws)
    with pytest.raises(ValueError, match="grad"):
        z.zero_gradnorm(L, -1, gs[:3] + [gs[3][:-5]], G, float(n), None, G, ws)
    B = z.zero_pack(2, [1000, 37])
    src = [torch.zeros(L.shard, device=DEV) for _ in range(n)]
    dst = torch.full((B.shard - 1,), 7.0, device=DEV)
    with pytest.raises(ValueError, match="dst"):
        z.zero_reshard(L, src, B, 0, dst)
    with pytest.raises(ValueError, match="dst"):
        z.zero_pack_copy(L, 0, [torch.zeros(1000, device=DEV), torch.zeros(37, device=DEV)], [0, 1],
                         torch.zeros(L.shard - 1, device=DEV))
    torch.cuda.synchronize()
    assert torch.all(dst == 7.0)
