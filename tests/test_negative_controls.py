"""Negative controls: the parity tests can see summation order and FMA
contraction.  Two variants of the oracle, each built on the CPU in a
temporary directory (the oracle itself is never changed), run one N = 8 rank
step on random data:

- the rank sum taken in reverse rank order (visible on fp32 gradients and on
  bf16 gradients spread over many binades; bf16 values of one magnitude
  usually add exactly);
- the same source compiled with FMA contraction allowed (-ffp-contract=fast
  -mfma).

Each must change at least one output bit of the master, m, v or the bf16
copy.  A GPU kernel that summed in another order, or that contracted a
multiply and an add, would therefore fail the bit-exact GPU parity tests."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))

RANK_SUM = ("            float sum = load_grad(grads[0], grad_bf16, gi);\n"
            "            for (int32_t q = 1; q < n_grads; ++q)\n"
            "                sum = sum + load_grad(grads[q], grad_bf16, gi);\n"
            "            float g = sum / divisor;    /* average */")
RANK_SUM_REVERSED = ("            float sum = load_grad(grads[n_grads - 1], grad_bf16, gi);\n"
                     "            for (int32_t q = n_grads - 2; q >= 0; --q)\n"
                     "                sum = sum + load_grad(grads[q], grad_bf16, gi);\n"
                     "            float g = sum / divisor;    /* average */")


def has_fma():
    try:
        return " fma " in open("/proc/cpuinfo").read().replace("\n", " ")
    except OSError:
        return False


def run_step(lib_path, out_npz, kind):
    """One rank step of N = 8 on fixed random data, with the given oracle
    library; results saved to out_npz.  kind "f32": normal fp32 gradients;
    "bf16_wide": bf16 gradients scaled by 2^k, k uniform in [-24, 24], so
    that the ranks' values span many binades.  (Eight bf16 values of similar magnitude, 8
    significant bits each, usually add exactly in binary32 in any order:
    order is visible only where the fp32 sum rounds.)"""
    with oracle.using(lib_path):
        rng = np.random.default_rng(2024)
        n, numel, r = 8, [8 * 40_000 + 5, 8 * 1_001], 3
        L = oracle.Layout(n, numel)
        S = L.total_shard
        if kind == "f32":
            grads = [np.ascontiguousarray(x) for x in
                     (rng.standard_normal((n, S)) * 1e-3).astype(np.float32)]
        else:
            g32 = (rng.standard_normal((n, S)) * 1e-3
                   * np.exp2(rng.integers(-24, 25, (n, S)))).astype(np.float32)
            grads = [np.ascontiguousarray(oracle.bf16(x)) for x in g32]
        w = rng.normal(0, 0.02, S).astype(np.float32)
        m = (rng.standard_normal(S) * 1e-4).astype(np.float32)
        v = (np.abs(rng.standard_normal(S)) * 1e-7).astype(np.float32)
        out = np.zeros(S, np.uint16)
        oracle.zero_step_rank(n, numel, r, grads, grad_local=True, divisor=float(n), clip=1.0,
                              master=w, m=m, v=v, state_global=False, out=out, out_gather=False,
                              t=5, lr=3e-4, b1=0.9, b2=0.95, eps=1e-8, wd=0.1)
    np.savez(out_npz, w=w, m=m, v=v, out=out)


def _child(lib_path, out_npz, kind):
    run_step(lib_path, out_npz, kind)


def results_of(lib_path, tmp_path, tag, kind):
    out = str(tmp_path / f"{tag}_{kind}.npz")
    code = (f"import sys; sys.path[:0] = [{HERE!r}, {os.path.dirname(HERE)!r}]; "
            f"import test_negative_controls as t; t._child({lib_path!r}, {out!r}, {kind!r})")
    subprocess.run([sys.executable, "-c", code], check=True, timeout=600)
    with np.load(out) as f:
        return {k: f[k] for k in f.files}


def differing_bits(a, b):
    return sum(int(np.count_nonzero(a[k].view(np.uint32 if a[k].dtype == np.float32 else np.uint16)
                                    != b[k].view(np.uint32 if b[k].dtype == np.float32 else np.uint16)))
               for k in a)


KINDS = ["f32", "bf16_wide"]


@pytest.fixture(scope="module")
def base(tmp_path_factory):
    tmp = tmp_path_factory.mktemp("base")
    lib = oracle.build(oracle.SRC, str(tmp / "liboracle_base.so"))
    return {k: results_of(lib, tmp, "base", k) for k in KINDS}


@pytest.mark.parametrize("kind", KINDS)
def test_reversed_rank_order_changes_bits(base, tmp_path, kind):
    src = open(oracle.SRC).read()
    assert src.count(RANK_SUM) == 1
    mut = tmp_path / "oracle_reversed.c"
    mut.write_text(src.replace(RANK_SUM, RANK_SUM_REVERSED))
    lib = oracle.build(str(mut), str(tmp_path / "liboracle_reversed.so"))
    res = results_of(lib, tmp_path, "reversed", kind)
    assert differing_bits(base[kind], res) > 0, "reversing the rank order changed no output bit"


@pytest.mark.skipif(not has_fma(), reason="host CPU has no FMA instructions")
@pytest.mark.parametrize("kind", KINDS)
def test_fma_contraction_changes_bits(base, tmp_path, kind):
    lib = oracle.build(oracle.SRC, str(tmp_path / "liboracle_fma.so"),
                       extra=["-ffp-contract=fast", "-mfma"])
    res = results_of(lib, tmp_path, "fma", kind)
    assert differing_bits(base[kind], res) > 0, "FMA contraction changed no output bit"


def test_base_is_reproducible(base, tmp_path):
    lib = oracle.build(oracle.SRC, str(tmp_path / "liboracle_again.so"))
    for k in KINDS:
        assert differing_bits(base[k], results_of(lib, tmp_path, "again", k)) == 0
