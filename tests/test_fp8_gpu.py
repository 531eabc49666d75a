"""GPU parity of the 8-bit forward (attn_fwd_fp8, through the C ABI) against
the fp64 oracle on the dequantised inputs (oracle/fp8.py).

Three kinds of check:
  * exact weights: q and k rows of three +-1 entries make every score an
    integer, and scale = ln 2 makes every weight a power of two within the
    range E4M3 holds exactly, so the rounding of the weights loses nothing and
    O must match to the bf16 output rounding (plus fp32), lse to 1e-5;
  * general inputs: every element within the oracle's bound for rounding the
    weights to E4M3 and for the matrix core's score error (plus the bf16
    output rounding), lse within the score error bound (it uses the
    unrounded weights), and the mean square error within the bound for
    independent roundings;
  * structure: NaN codes in V^T's padding never reach O, negative and zero
    scales, GQA groups, ragged N, determinism, a full-size workload sampled.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.parity import half_ulp

pytestmark = pytest.mark.gpu

LN2 = math.log(2.0)


@pytest.fixture(scope="module")
def attn():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from exact_io_aware_73_amd import attn as a
    return a


def _say(msg):
    print(msg, flush=True)


def _run(attn, q8, k8, vt8, qs, ks, vs, scale):
    o, lse = attn.fwd_fp8(q8.cuda(), k8.cuda(), vt8.cuda(), qs, ks, vs, scale)
    torch.cuda.synchronize()
    return workloads.to_f64(o), lse.cpu().numpy().astype(np.float64)


def _refs(q8, k8, vt8, qs, ks, vs, scale):
    args = (q8.numpy(), k8.numpy(), vt8.numpy(), qs, ks, vs, scale)
    O, lse = oracle.attention_fp8_ref(*args)
    return (O, lse, oracle.fp8_error_bound(*args), oracle.fp8_mean_square_bound(*args),
            oracle.fp8_lse_bound(*args))


def _check_exact(attn, B, Hq, Hkv, N, d, seed):
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(B, Hq, Hkv, N, d, seed, kind="exact")
    _say(f"[fp8] exact weights {(B, Hq, Hkv, N, d)}")
    o, lse = _run(attn, q8, k8, vt8, qs, ks, vs, LN2)
    O, lse_ref, _, _, _ = _refs(q8, k8, vt8, qs, ks, vs, LN2)
    tol = half_ulp(O, "bf16") + 1e-5 * np.max(np.abs(O))
    err = np.abs(o - O)
    assert np.all(np.isfinite(o)) and np.all(err <= tol), float(np.max(err - tol))
    assert np.max(np.abs(lse - lse_ref)) <= 1e-5


def _check_general(attn, q8, k8, vt8, qs, ks, vs, scale, label):
    _say(f"[fp8] {label} q8={tuple(q8.shape)} vt8={tuple(vt8.shape)} scale={scale}")
    o, lse = _run(attn, q8, k8, vt8, qs, ks, vs, scale)
    O, lse_ref, bound, ms, lb = _refs(q8, k8, vt8, qs, ks, vs, scale)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    err = np.abs(o - O)
    allow = bound + half_ulp(O, "bf16") + 1e-6
    assert np.all(err <= allow), (label, float(np.max(err - allow)))
    assert np.mean(err ** 2) <= 2.0 * np.mean(ms) + 2.0 * np.mean((2.0 ** -9 * O) ** 2), label
    assert np.all(np.abs(lse - lse_ref) <= lb + 1e-5), label
    return float(np.max(err)), float(np.max(bound))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 100, 128, 300, 1000])
def test_fp8_exact_weights(attn, N, d):
    _check_exact(attn, 1, 2, 1, N, d, 101 * N + d)


@pytest.mark.parametrize("B,Hq,Hkv,N", [(2, 8, 2, 129), (1, 16, 1, 33), (2, 12, 3, 200)])
def test_fp8_exact_weights_gqa(attn, B, Hq, Hkv, N):
    _check_exact(attn, B, Hq, Hkv, N, 128, 7 * N + Hq)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 64, 65, 257, 1000])
@pytest.mark.parametrize("B,Hq,Hkv", [(1, 1, 1), (2, 4, 2)])
def test_fp8_general(attn, B, Hq, Hkv, N, d):
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(B, Hq, Hkv, N, d, 13 * N + d + Hq)
    _check_general(attn, q8, k8, vt8, qs, ks, vs, 1.0 / math.sqrt(d), "general")


@pytest.mark.parametrize("scale", [0.0, -0.09, 0.5])
def test_fp8_scales(attn, scale):
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(1, 4, 2, 300, 128, 55)
    _check_general(attn, q8, k8, vt8, qs, ks, vs, scale, "scale")


def test_fp8_zero_scale_is_mean(attn):
    """scale 0: every weight is 1 (exact in E4M3), O = the mean of V's rows."""
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(1, 2, 1, 77, 128, 8)
    o, _ = _run(attn, q8, k8, vt8, qs, ks, vs, 0.0)
    _, _, v = oracle.dequantize(q8.numpy(), k8.numpy(), vt8.numpy(), qs, ks, vs, 77)
    want = np.broadcast_to(v[0, 0].mean(axis=0), o[0, 0].shape)
    assert np.all(np.abs(o[0, 0] - want) <= half_ulp(want, "bf16") + 1e-6)


def test_fp8_padding_nan_ignored(attn):
    """NaN codes in V^T's padding keys (N .. Np-1) and beyond N in the last
    64-key tile change nothing."""
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(2, 4, 2, 37, 128, 21)
    o1, l1 = _run(attn, q8, k8, vt8, qs, ks, vs, 0.1)
    vt_nan = vt8.clone()
    vt_nan[..., 37:] = 0x7F
    o2, l2 = _run(attn, q8, k8, vt_nan, qs, ks, vs, 0.1)
    assert np.all(np.isfinite(o2)) and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fp8_deterministic(attn):
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(2, 8, 2, 700, 128, 4)
    a = _run(attn, q8, k8, vt8, qs, ks, vs, 0.09)
    b = _run(attn, q8, k8, vt8, qs, ks, vs, 0.09)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_fp8_full_size_sampled(attn):
    """The long-sequence shape (B=4, H=32, N=4096, d=128) in 8 bits: sampled
    rows against the oracle's rows and bound."""
    B, H, N, d = 4, 32, 4096, 128
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(B, H, H, N, d, 3000)
    _say(f"[fp8] full size {(B, H, N, d)}")
    o, lse = _run(attn, q8, k8, vt8, qs, ks, vs, 1.0 / math.sqrt(d))
    q, k, v = oracle.dequantize(q8.numpy(), k8.numpy(), vt8.numpy(), qs, ks, vs, N)
    rng = np.random.default_rng(0)
    scale = 1.0 / math.sqrt(d)
    for b, h in [(0, 0), (1, 17), (3, 31)]:
        rows = np.sort(rng.choice(N, 24, replace=False))
        O, lse_ref = oracle.attention_ref_rows(q, k, v, b, h, rows, scale)
        bound, ds = oracle.fp8_bounds_rows(q, k, v, b, h, rows, scale)
        err = np.abs(o[b, h, rows] - O)
        assert np.all(err <= bound + half_ulp(O, "bf16") + 1e-6), (b, h)
        assert np.all(np.abs(lse[b, h, rows] - lse_ref) <= ds + 1e-5), (b, h)


def test_fp8_rejects(attn):
    q8, k8, vt8, qs, ks, vs = workloads.fp8_inputs(1, 2, 1, 40, 128, 1)
    q8, k8, vt8 = q8.cuda(), k8.cuda(), vt8.cuda()
    with pytest.raises(ValueError):          # V not transposed / padded
        attn.fwd_fp8(q8, k8, k8, qs, ks, vs)
    with pytest.raises(ValueError):          # a non-finite scale
        attn.fwd_fp8(q8, k8, vt8, float("inf"), ks, vs)
