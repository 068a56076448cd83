"""bench.py's output contract on the GPU: one JSON line with the metric, the
throughput, the timing fields, the workload, the roofline object (live HIP
event timing of the dominant kernel) and the oracle baseline, for a short
run of the small workload (one GPT-2-Large-shaped block) and of the
reshard."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
        "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic", "avg_launch_ms", "timing", "per_call_ms"}


def _run(args):
    print("bench", *args, flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    return json.loads(lines[0])


def _check(d, steps, warmup):
    assert KEYS <= d.keys()
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and d["vs_baseline"] is None
    assert "workload" in d["config"]
    r = d["roofline"]
    assert ROOF <= r.keys()
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] < 1.0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] == 1 and cb["sample"]


@pytest.mark.gpu
def test_step_line():
    d = _run(["--workload", "gpt2l_block", "--steps", "5", "--warmup", "2", "--cpu-seconds", "0.5"])
    _check(d, 5, 2)
    assert d["config"]["workload"] == "gpt2l_block" and d["unit"] == "elements/s"
    # the block's 19.7M elements, 2N + 26 bytes each at N = 8
    assert d["config"]["bytes_per_element"] == pytest.approx(42.0)


@pytest.mark.gpu
def test_reshard_line():
    d = _run(["--reshard", "gpt2l_reshard", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5"])
    _check(d, 3, 1)
    assert d["config"]["workload"] == "gpt2l_reshard"
