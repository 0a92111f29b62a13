"""bench.py's contract pieces that run without a GPU (CPU only)."""
import os
import subprocess
import sys

import numpy as np

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_cpu_baselines_on_tiny_workloads():
    cfg = W.make_config("tiny")
    host = [cfg[k].numpy() for k in ("A", "sA", "B", "sB", "offs")]
    res = bench.cpu_baseline(cfg, *host, budget_s=1.0)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1 and "tiny" in res["sample"]
    b = W.make_bf16(4, 128, 256, 512, [96, 0, 160, 256], seed=5)
    u16 = lambda t: t.view(__import__("torch").int16).numpy().view(np.uint16)
    rb = bench.cpu_baseline_bf16(b, u16(b["A"]), u16(b["B"]), b["offs"].numpy(), budget_s=1.0)
    assert rb["kind"] == "oracle" and rb["value"] > 0
    r = W.make_rows(3, 700, 256, 272, [300, 0, 290], seed=6)
    rr = bench.cpu_baseline_rows(dict(r, name="rows"), *(r[k].numpy() for k in ("A", "sA", "B", "sB", "offs")),
                                 budget_s=0.5)
    assert rr["kind"] == "oracle" and rr["value"] > 0
