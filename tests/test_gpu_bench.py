"""bench.py's output contract on the GPU (needs an MI355X): one JSON line with
the driver's keys, the roofline and CPU-baseline objects, and the extra legs,
on the tiny workload (a child process, so this test's own GPU state does not
matter; it prints what it runs before it starts)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_on_tiny_workload():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "20", "--warmup", "5",
           "--prerun", "0.5", "--no-bf16"]
    print("[gpu-case] " + " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5 and d["higher_is_better"] is True
    assert d["unit"] == "TFLOP/s" and d["value"] > 0 and d["ms_per_step"] > 0
    assert d["config"]["workload"] == "tiny" and d["vs_baseline"] is None
    # value is the useful work over the measured time per step
    flops = 2 * 512 * 128 * 256
    assert abs(d["value"] - flops / (d["ms_per_step"] * 1e-3) / 1e12) <= 0.01 * d["value"] + 0.01
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 5000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-4
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    for leg in ("sustained", "plain_entry", "padded_rows", "cold_caches", "graph_replay"):
        assert leg in d, leg
    assert d["graph_replay"]["ms_per_call"] > 0 and d["cold_caches"]["cold_median_ms"] > 0
