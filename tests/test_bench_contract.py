"""Host-side parts of bench.py's output contract (CPU only)."""
from __future__ import annotations

import math
import os
import subprocess
import sys

import torch

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a configuration that is not run


def test_cpu_baseline_fields_and_repeated_passes():
    # a small GQA shape whose single pass takes well under the budget, so
    # the baseline must pass over the workload again until the budget is spent
    w = workloads.Workload(name="tiny_gqa", B=2, Hq=4, Hkv=2, N=64, d=64, dtype="bf16", seed=3)
    q, k, v = workloads.random_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, torch.bfloat16, seed=3)
    rec = bench.cpu_baseline(w, q, k, v, 1 / math.sqrt(w.d), budget_s=0.5)
    assert set(rec) >= {"value", "unit", "cores", "kind", "sample"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert rec["seconds"] >= 0.5
    passes = float(rec["sample"].split("(")[2].split()[0])
    assert passes > 1.0, rec["sample"]
