"""The library's HIP step against golden values that do not come from the
oracle: single AdamW elements whose result bits each alternative association
of the page's AdamW code would change ("ZeRO and FSDP sharding", Code;
tests/golden/adamw_order.json, written by exact rational arithmetic)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import f32exact as F  # noqa: E402
import pins  # noqa: E402
import fsdp_sharded_optimizer_flat_amd as z  # noqa: E402
from gpu_common import DEV  # noqa: E402


@pytest.mark.parametrize("copies", [1, 3, 1024 + 5])
def test_adamw_order_golden_gpu(copies):
    """copies = 1 / 3: the one-element kernel; 1029: the quad kernel plus a
    ragged tail."""
    Lc = z.ZERO_LOCAL
    for c in pins.golden("adamw_order.json")["cases"]:
        hp = [F.value_of(F.from_decimal(c["hyper"][k])) for k in ("lr", "b1", "b2", "eps", "wd")]
        L = z.zero_pack(1, [copies])
        t = {k: torch.from_numpy(np.full(copies, int(c[k], 16), np.uint32).view(np.float32)).to(DEV)
             for k in "wmvg"}
        s = z.zero_adamw_scalars_for(c["t"], *hp, 1.0)
        z.zero_step(L, 0, [t["g"]], Lc, 1.0, t["w"], t["m"], t["v"], Lc, None, Lc, s)
        torch.cuda.synchronize()
        for k in "mvw":
            got = t[k].cpu().view(torch.int32).numpy().view(np.uint32)
            assert np.all(got == int(c["expect"][k], 16)), (c, k, hex(int(got[0])))
