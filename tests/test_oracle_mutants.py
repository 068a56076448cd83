"""Mutation tests: plant a plausible mistake in a copy of the oracle and show
that at least one pin catches it.  The copy is built on the CPU in a temporary
directory; the oracle itself is never changed."""
import os
import subprocess
import sys

import pytest

import oracle
import pins

# (name, text in oracle.c, replacement): dropped terms, wrong signs, wrong
# indices, transposed operands, off-by-ones and rounding slips.
MUTANTS = [
    ("drop bias correction 1", "h->bc1 = 1.0f - pow1;", "h->bc1 = 1.0f;"),
    ("drop bias correction 2", "h->bc2 = sqrtf(one_minus_pow2);", "h->bc2 = 1.0f;"),
    ("weight-decay sign", "h->decay = 1.0f - lr_wd;", "h->decay = 1.0f + lr_wd;"),
    ("b1 and 1-b1 swapped in m", "float m_decayed = h->b1 * (*m);", "float m_decayed = h->one_minus_b1 * (*m);"),
    ("b1 used for v", "float v_decayed = h->b2 * (*v);", "float v_decayed = h->b1 * (*v);"),
    ("eps dropped", "float den = root / h->bc2 + h->eps;", "float den = root / h->bc2;"),
    ("m under the square root", "float root = sqrtf(*v);", "float root = sqrtf(fabsf(*m));"),
    ("decay after the update", "*w = w_decayed - update;", "*w = ((*w) - update) * h->decay;"),
    ("t off by one", "for (int32_t i = 0; i < t; ++i) {", "for (int32_t i = 0; i <= t; ++i) {"),
    ("rank 0 counted twice", "            for (int32_t q = 1; q < n_grads; ++q)\n                sum = sum + load_grad(grads[q], grad_bf16, gi);\n            float g = sum / divisor;",
     "            for (int32_t q = 0; q < n_grads; ++q)\n                sum = sum + load_grad(grads[q], grad_bf16, gi);\n            float g = sum / divisor;"),
    ("wrong divisor", "float g = sum / divisor;    /* average */", "float g = sum / (divisor + 1.0f);"),
    ("ranks' slices reversed", "int64_t j = L.offset[u] + (int64_t)r * L.shard[u] + i;\n            int64_t gi = grad_local ? k : j;\n            /* reduce-scatter",
     "int64_t j = L.offset[u] + (int64_t)(n - 1 - r) * L.shard[u] + i;\n            int64_t gi = grad_local ? k : j;\n            /* reduce-scatter"),
    ("local offset not accumulated",
     "shard[u] = p / n;\n        offset[u] = next_offset;\n        local_offset[u] = next_local;\n"
     "        next_offset += padded[u];\n        next_local += shard[u];",
     "shard[u] = p / n;\n        offset[u] = next_offset;\n        local_offset[u] = next_local;\n"
     "        next_offset += padded[u];\n        next_local += 0;"),
    ("row layout's local offset not accumulated",
     "shard[u] = padded[u] / n;\n        offset[u] = next_offset;\n        local_offset[u] = next_local;\n"
     "        next_offset += padded[u];\n        next_local += shard[u];",
     "shard[u] = padded[u] / n;\n        offset[u] = next_offset;\n        local_offset[u] = next_local;\n"
     "        next_offset += padded[u];\n        next_local += 0;"),
    ("padding rounds up one extra", "while (p % n != 0)     /* pad one element at a time: obviously minimal */\n            p += 1;",
     "do                      /* pad one element at a time: obviously minimal */\n            p += 1;\n        while (p % n != 0);"),
    ("bf16 ties away from zero", "pick = (below & 1u) ? above : below;", "pick = above;"),
    ("bf16 truncates", "else if (d_above < d_below)\n        pick = above;", "else if (0)\n        pick = above;"),
    ("clip coefficient not capped", "if (coef > 1.0)\n        coef = 1.0;", ""),
    ("clip eps dropped", "double coef = max_norm / (norm + 1e-6);", "double coef = max_norm / norm;"),
    ("sum of squares in binary32", "double acc = 0.0;\n    for (int64_t i = 0; i < n; ++i) {\n        double x = (double)g[i];",
     "float acc = 0.0f;\n    for (int64_t i = 0; i < n; ++i) {\n        float x = g[i];"),
    ("ledger stage 2 forgets the gradients", "if (stage >= 2)\n        grads = grads / n;", ""),
    ("ledger stage 3 communication 2 psi", "double passes = (stage >= 3) ? 3.0 : 2.0;", "double passes = 2.0;"),
    ("rows padded by elements", "while (rows % n != 0)   /* pad one row at a time */",
     "while ((rows * row_len[u]) % n != 0)   /* pad one row at a time */"),
    ("reshard reads the destination layout's offset", "A.local_offset, A.offset[w] + stream, &q, &ka);",
     "A.local_offset, B.offset[w] + stream, &q, &ka);"),
    ("reshard ignores the unit's stream start", "stream += numel_b[u];\n            ++u;",
     "++u;"),
    ("reshard reads the destination rank's shard", "memcpy(d, (const char *)src[q] + ka * elem",
     "memcpy(d, (const char *)src[dst_rank < n_a ? dst_rank : 0] + ka * elem"),
    ("footprint forgets the output", "    if (with_out)\n        per += 2.0;\n", ""),
    # the reduced gradient (the norm pass's reference) and the association of
    # the AdamW update that the page's code fixes
    ("reduced gradient: wrong divisor", "g_out[k] = sum / divisor;", "g_out[k] = sum / (divisor + 1.0f);"),
    ("reduced gradient: index spaces swapped", "int64_t gi = grad_local ? k : j;\n            float sum",
     "int64_t gi = grad_local ? j : k;\n            float sum"),
    ("v increment as (1-b2)*(g*g)", "float v_incr = (h->one_minus_b2 * g) * g;",
     "float v_incr = h->one_minus_b2 * (g * g);"),
    ("update as (lr/bc1)*(m/den)", "float numer = h->lr_over_bc1 * (*m);\n    float update = numer / den;",
     "float numer = (*m) / den;\n    float update = h->lr_over_bc1 * numer;"),
    ("denominator by the reciprocal of bc2", "float den = root / h->bc2 + h->eps;",
     "float den = root * (1.0f / h->bc2) + h->eps;"),
    ("denominator as sqrt(v / bc2^2)", "float den = root / h->bc2 + h->eps;",
     "float den = sqrtf(*v / (h->bc2 * h->bc2)) + h->eps;"),
]


def run_all_pins():
    failed = []
    for pin in pins.ALL_PINS:
        try:
            if pin is pins.pin_bf16_vs_torch:
                pin(patterns=pins.bf16_probe_patterns(n_random=1 << 14))
            else:
                pin()
        except (AssertionError, ValueError) as e:
            failed.append((pin.__name__, str(e)[:120]))
    return failed


def _child(lib_path):
    with oracle.using(lib_path):
        failed = run_all_pins()
    for name, msg in failed:
        print("PIN FAILED:", name, msg)
    sys.exit(1 if failed else 0)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name!r} not unique in oracle.c"
    mut_src = tmp_path / "oracle_mutant.c"
    mut_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mut_src), str(tmp_path / "liboracle_mutant.so"))
    # The pins run in a child process: a mutant may also corrupt memory and
    # crash, which counts as caught but must not take the test runner down.
    here = os.path.dirname(os.path.abspath(__file__))
    code = f"import sys; sys.path[:0] = [{here!r}, {os.path.dirname(here)!r}]; " \
           f"import test_oracle_mutants as t; t._child({lib!r})"
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert res.returncode != 0, f"no pin caught the planted mistake: {name}\n{res.stdout[-2000:]}"
