"""FLOP / byte accounting against the numbers the pages print (no GPU)."""
import json
import os

import pytest

from exact_io_aware_73_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))
MIB = 1024 * 1024


def _close(x, ref, rel):
    return abs(x - ref) <= rel * abs(ref) + 1e-12


def test_sp_sweep():
    g = GOLD["sp_fp16_mib_sweep"]
    for n, mib in zip(g["n"], g["mib"]):
        assert acc.sp_bytes(n, 2) == 4 * n * n
        assert acc.sp_bytes(n, 2) / MIB == mib


def test_worked_example_n4096():
    g = GOLD["qk_worked_example"]
    n, d = g["n"], g["d"]
    assert _close(acc.qk_flops(n, d), g["qk_flops"], g["qk_flops_rel"])
    assert _close(acc.softmax_flops(n), g["softmax_flops"], g["softmax_flops_rel"])
    assert _close(acc.softmax_bytes(n, 2), g["softmax_bytes"], g["softmax_bytes_rel"])
    assert acc.softmax_flops(n) / acc.softmax_bytes(n, 2) == g["softmax_ai"]
    # the page's own formula for the Q K^T bytes: read Q and K, write S
    qk_bytes = 2 * n * d * 2 + acc.nn_matrix_bytes(n, 2)
    assert qk_bytes == 100_663_296
    assert not _close(qk_bytes, g["qk_bytes_printed"], 0.05)   # the printed 1.3e8 is a slip


def test_a100_balance():
    g = GOLD["a100_balance"]
    assert g["flops"] / g["bytes_per_s"] == g["balance"]


def test_d128_footprint():
    g = GOLD["d128_footprint"]
    n, d = g["n"], g["d"]
    assert _close(acc.nn_matrix_bytes(n, 2) / 1e6, g["s_mb"], g["rel"])
    assert _close(acc.sp_bytes(n, 2) / 1e6, g["sp_mb"], g["rel"])
    assert _close(n * d * 2 / 1e6, g["o_mb"], 0.05)
    assert _close(acc.sp_bytes(8192, 2) / 1e6, g["sp_mb_8192"], g["rel"])


def test_fp32_score_matrix():
    g = GOLD["fp32_score_matrix"]
    assert acc.nn_matrix_bytes(g["n"], 4) / MIB == g["mb"]


def test_128k_context():
    g = GOLD["context_128k"]
    assert _close(g["n"] ** 2, g["elements"], g["rel"])


def test_score_matrix_2n2():
    g = GOLD["score_matrix_2n2"]
    for n, b in zip(g["n"], g["bytes"]):
        assert _close(acc.nn_matrix_bytes(n, 2), b, g["rel"])


def test_dao_ratios():
    g = GOLD["dao_fig2_ratios"]
    assert _close(g["fa_gflops"] / g["std_gflops"] - 1, 0.13, 0.05)
    assert _close(1 - g["fa_hbm_gb"] / g["std_hbm_gb"], 0.89, 0.01)
    assert _close(1 - g["fa_ms"] / g["std_ms"], 0.82, 0.01)
    assert _close(g["std_hbm_gb"] / g["std_ms"] * 1e3, g["std_gbps"], 0.005)
    assert _close(g["fa_hbm_gb"] / g["fa_ms"] * 1e3, g["fa_gbps"], 0.005)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,flops,minb", [
    (1, 1, 1, 256, 64, 16_777_216, None),
    (64, 16, 16, 1024, 64, 274_877_906_944, 536_870_912),
    (4, 32, 32, 4096, 128, 1_099_511_627_776, 536_870_912),
    (2, 32, 8, 8192, 128, 2_199_023_255_552, 335_544_320),
    (1, 8, 8, 32768, 128, 4_398_046_511_104, 268_435_456),
])
def test_workload_accounting(B, Hq, Hkv, N, d, flops, minb):
    assert acc.attn_fwd_flops(B, Hq, N, d) == flops
    if minb is not None:
        assert acc.min_bytes(B, Hq, Hkv, N, d, 2) == minb


def test_materialized_prediction_long_config():
    # S fp32 and P bf16 each written and read once, plus Q, K, V, O
    b = acc.materialized_bytes(4, 32, 32, 4096, 128, 2)
    assert b == 2 * 4 * 32 * 4096 * 4096 * 4 + 2 * 4 * 32 * 4096 * 4096 * 2 + 536_870_912
    assert abs(b / 1e9 - 26.31) < 0.01


def test_peak():
    assert abs(acc.peak_bf16_tflops() - acc.PEAK_BF16_TFLOPS) < 0.1
