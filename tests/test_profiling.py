"""Host logic of the profile summaries and the bench's counter matching (CPU only)."""
from __future__ import annotations

import csv
import json
import os

import pytest

from exact_io_aware_73_amd import profiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRACE_FIELDS = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for name, start, dur in rows:
            w.writerow({"Kind": "KERNEL_DISPATCH", "Kernel_Name": name,
                        "Start_Timestamp": start, "End_Timestamp": start + dur})


def test_last_k_takes_the_latest_dispatches(tmp_path):
    # warm-up dispatches are slow (900 us), the timed ones ~100 us, written out of order
    rows = [("fused", 10_000_000 + 1_000_000 * i, 900_000) for i in range(5)]
    rows += [("fused", 20_000_000 + 1_000_000 * i, 100_000 + 1000 * i) for i in range(3)]
    rows += [("other", 5_000_000, 50_000)]
    path = tmp_path / "trace.csv"
    _write_trace(path, list(reversed(rows)))
    text = profiling.last_k_table(str(path), 3)
    line = next(ln for ln in text.splitlines() if ln.startswith("fused"))
    calls, avg, lo, hi = line.split()[1:]
    assert int(calls) == 3
    assert float(avg) == pytest.approx(101.0)                  # microseconds
    assert float(lo) == pytest.approx(100.0) and float(hi) == pytest.approx(102.0)
    other = next(ln for ln in text.splitlines() if ln.startswith("other"))
    assert int(other.split()[1]) == 1                          # fewer dispatches than K


def _counter_csv(path, kernel, values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for v in values:
            w.writerow({"Kernel_Name": kernel, "Counter_Value": v})


def test_counters_scale_by_the_copy_calibration(tmp_path):
    # a 1 MiB copy reads as 512 KiB fetched and 1024 KiB written: fetch x2, write x1
    _counter_csv(tmp_path / "cf.csv", profiling.COPY_KERNEL, [512.0, 512.0, 512.0])
    _counter_csv(tmp_path / "cw.csv", profiling.COPY_KERNEL, [1024.0])
    _counter_csv(tmp_path / "f.csv", profiling.FUSED_KERNEL + "_kernel<64>", [100.0, 101.0, 99.0])
    _counter_csv(tmp_path / "w.csv", profiling.FUSED_KERNEL + "_kernel<64>", [50.0])
    rec = profiling.counters_summary("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                     str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1,
                                     "cmd", "sha")
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_read_bytes_per_launch"] == 100 * 1024 * 2      # the median dispatch
    assert rec["hbm_write_bytes_per_launch"] == 50 * 1024
    assert rec["hbm_bytes_per_launch"] == 100 * 1024 * 2 + 50 * 1024


def test_counter_summary_matches_only_its_own_kernel_sources(tmp_path):
    import bench

    w = "gpt2_medium_b64_h16_n1024_d64"
    rec = {"kernel_source_sha": bench.kernel_source_hash(w), "hbm_bytes_per_launch": 12345}
    path = tmp_path / f"attn_fwd_{w}_counters.json"
    path.write_text(json.dumps(rec))
    assert bench.traffic_from_profiles(w, 0, str(tmp_path)) == 12345
    path.write_text(json.dumps(dict(rec, kernel_source_sha="stale")))
    assert bench.traffic_from_profiles(w, 0, str(tmp_path)) is None
    assert bench.traffic_from_profiles("long_b4_h32_n4096_d128", 0, str(tmp_path)) is None
    # the d = 64 and d = 128 kernels are built from different sources
    assert bench.kernel_source_hash(w) != bench.kernel_source_hash("long_b4_h32_n4096_d128")


def test_counters_sum_the_kernels_of_one_call(tmp_path):
    """The materialising path's three kernels: one call's bytes are the sum of
    each kernel's median dispatch, every one scaled by the copy calibration."""
    _counter_csv(tmp_path / "cf.csv", profiling.COPY_KERNEL, [512.0])
    _counter_csv(tmp_path / "cw.csv", profiling.COPY_KERNEL, [1024.0])
    rows_f = [("qk_bf16_kernel<128>", 10.0), ("softmax_rows_wave_kernel<bf16>", 20.0),
              ("pv_bf16_kernel<128, true>", 30.0)] * 2
    rows_w = [("qk_bf16_kernel<128>", 1.0), ("softmax_rows_wave_kernel<bf16>", 2.0),
              ("pv_bf16_kernel<128, true>", 3.0)] * 2
    for name, rows in (("f.csv", rows_f), ("w.csv", rows_w)):
        with open(tmp_path / name, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
            w.writeheader()
            for k, v in rows:
                w.writerow({"Kernel_Name": k, "Counter_Value": v})
    rec = profiling.counters_summary("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                     str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1,
                                     "cmd", "sha", ("qk_bf16", "softmax_rows", "pv_bf16"))
    assert rec["hbm_read_bytes_per_launch"] == (10 + 20 + 30) * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == (1 + 2 + 3) * 1024
    assert rec["per_kernel"]["softmax_rows"]["read_bytes"] == 20 * 1024 * 2
    with pytest.raises(ValueError):
        profiling.counters_summary("wl", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                   str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 1,
                                   "cmd", "sha", ("no_such_kernel",))


def test_materialized_counters_match_their_own_sources(tmp_path):
    import bench

    w = "long_b4_h32_n4096_d128"
    rec = {"kernel_source_sha": bench.materialized_source_hash(),
           "hbm_read_bytes_per_launch": 7, "hbm_write_bytes_per_launch": 5}
    path = tmp_path / f"attn_fwd_materialized_{w}_counters.json"
    path.write_text(json.dumps(rec))
    assert bench.materialized_traffic_from_profiles(w, str(tmp_path)) == (7, 5)
    path.write_text(json.dumps(dict(rec, kernel_source_sha="stale")))
    assert bench.materialized_traffic_from_profiles(w, str(tmp_path)) is None


def test_backward_counters_match_their_own_sources(tmp_path):
    import bench

    w = "long_b4_h32_n4096_d128"
    rec = {"kernel_source_sha": bench.backward_source_hash(),
           "hbm_read_bytes_per_launch": 11, "hbm_write_bytes_per_launch": 3}
    path = tmp_path / f"attn_bwd_{w}_counters.json"
    path.write_text(json.dumps(rec))
    assert bench.backward_traffic_from_profiles(w, str(tmp_path)) == (11, 3)
    path.write_text(json.dumps(dict(rec, kernel_source_sha="stale")))
    assert bench.backward_traffic_from_profiles(w, str(tmp_path)) is None
    assert bench.backward_source_hash() != bench.materialized_source_hash()


def test_committed_backward_counters_are_current():
    # every committed backward byte count was taken on the backward's current sources
    import glob
    import bench

    paths = glob.glob(os.path.join(ROOT, "profiles", "attn_bwd_*_counters.json"))
    assert paths
    for p in paths:
        rec = json.load(open(p))
        assert rec["kernel_source_sha"] == bench.backward_source_hash(), p


def test_backward_minimum_bytes():
    from exact_io_aware_73_amd import accounting as acc

    # one head, N = 1, d = 1: Q K V O dO read (5 x 2 bytes), lse (4), dQ dK dV (3 x 2)
    assert acc.bwd_min_bytes(1, 1, 1, 1, 1, 2) == 10 + 4 + 6
    # GQA 4:1: the K/V-sized tensors (K, V, dK, dV) scale with Hkv, the rest with Hq
    assert acc.bwd_min_bytes(1, 4, 1, 8, 2, 2) == 2 * (4 * 4 * 8 * 2 + 4 * 1 * 8 * 2) + 4 * 4 * 8


def test_committed_forward_counters_are_current():
    # every committed byte count of the fused and materialising paths was
    # taken on the sources the kernel it describes is built from now
    import glob
    import bench

    paths = glob.glob(os.path.join(ROOT, "profiles", "attn_fwd_*_counters.json"))
    assert paths
    for p in paths:
        rec = json.load(open(p))
        if "_materialized_" in os.path.basename(p):
            want = bench.materialized_source_hash()
        else:
            want = bench.kernel_source_hash(rec["workload"])
        assert rec["kernel_source_sha"] == want, p
