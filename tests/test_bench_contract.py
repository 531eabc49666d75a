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
    rec = bench.cpu_baseline(w, q, k, v, 1 / math.sqrt(w.d), budget_s=0.5, threads=2)
    assert set(rec) >= {"value", "unit", "cores", "kind", "sample", "host_cpus", "cpu_model"}
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] == 2
    assert rec["host_cpus"] >= 1 and rec["cpu_model"]
    assert rec["seconds"] >= 0.5
    passes = float(rec["sample"].split("(")[1].split()[0])
    assert passes > 1.0, rec["sample"]


def test_cpu_baseline_splits_long_heads_into_row_blocks():
    """A long head is sampled in blocks of query rows, each block's rows
    against all of the head's keys."""
    w = workloads.Workload(name="long1", B=1, Hq=1, Hkv=1, N=4096, d=128, dtype="bf16", seed=4)
    q, k, v = workloads.random_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, torch.bfloat16, seed=4)
    rec = bench.cpu_baseline(w, q, k, v, 1 / math.sqrt(w.d), budget_s=0.3, threads=2)
    assert "up to 512 query rows x all 4096 keys" in rec["sample"], rec["sample"]
    assert rec["value"] > 0


def test_default_workload_is_the_largest_single_gpu_configuration():
    big = max((w for w in workloads.WORKLOADS.values() if w.dtype == "bf16"),
              key=lambda w: 4 * w.B * w.Hq * w.N * w.N * w.d)
    assert workloads.DEFAULT_BENCH == big.name == "long_context_b1_h8_n32768_d128"
    assert not workloads.WORKLOADS[workloads.DEFAULT_BENCH].materialized


def test_sequence_length_sweep_fixes_everything_but_n():
    """The sweep of the measurement section: one configuration at every
    length, the comparison path wherever its S and P fit the bench's 64 GiB
    cap, and none of it among the configurations the default is chosen from."""
    sw = list(workloads.SWEEP.values())
    assert [w.N for w in sw] == sorted(w.N for w in sw) and len(sw) >= 5
    assert {(w.B, w.Hq, w.Hkv, w.d, w.dtype) for w in sw} == {(4, 32, 32, 128, "bf16")}
    for w in sw:
        sp = w.B * w.Hq * w.N * w.N * (4 + w.elem_bytes)
        assert w.materialized == (sp < (64 << 30)), w.name
        assert w.name in workloads.ALL and w.name not in workloads.WORKLOADS
    assert set(workloads.WORKLOADS) <= set(workloads.ALL)
