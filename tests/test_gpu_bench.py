"""bench.py end to end on the GPU, on the tiny workload: the JSON line keeps
its contract (the fields and their types, the roofline and CPU-baseline
objects, value consistent with ms_per_step), and the loss it reports is the
oracle's on the same seeded batch."""
import json
import math
import os
import subprocess
import sys

import pytest

import oracle
import workloads
from gpu_support import LOSS_TOL, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_tiny():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--cpu-seconds", "0.5", "--no-power-context"]
    say("bench", " ".join(cmd[1:]))
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.strip().splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["higher_is_better"] is True
    assert d["unit"] == "tokens/s" and d["dtype"] == "bf16" and d["data"] == "synthetic" and d["vs_baseline"] is None
    w = workloads.WORKLOADS["tiny"]
    assert d["config"]["workload"] == "tiny" and d["config"]["n_tokens"] == w.n_tokens
    assert d["value"] > 0 and abs(d["value"] - w.n_tokens / (d["ms_per_step"] / 1e3)) <= 2e-3 * d["value"]
    roof = d["roofline"]
    assert roof["bound"] in ("mfma", "hbm") and roof["unit"] in ("TFLOP/s", "GB/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) <= 1e-3
    assert "traffic" in roof  # null: no counters were taken for the tiny workload
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    # the loss the benchmark measured is the oracle's on the same seeded batch
    b = workloads.make(w, seed=0)
    ref = oracle.cross_entropy(oracle.bf16_to_f64(b.hidden), oracle.bf16_to_f64(b.weight), b.targets, grad=False)
    assert math.isfinite(d["loss"]) and abs(d["loss"] - ref.loss) <= LOSS_TOL, (d["loss"], ref.loss)
