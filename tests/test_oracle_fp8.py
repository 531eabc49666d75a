"""Pins of the 8-bit oracle (oracle/fp8.py), CPU only.

The E4M3 decoder is checked against the values the OCP format fixes and
against torch's float8_e4m3fn conversion for all 256 codes; the transposed,
padded V layout against closed forms (constant V, padding holding NaN
codes); the error bound against a direct emulation of what the bound
assumes -- weights rounded to E4M3 (torch's round-to-nearest-even cast)
relative to a running maximum at most 2 (log2) below the true one and
scaled by 2^6 -- on score distributions that exercise the normal range,
the subnormal range and flushed weights.  Bounds with a term planted out
fail those emulations.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F


def test_decode_fixed_values():
    """Values the E4M3 format fixes: zero, the subnormal and normal ends, one, NaN."""
    codes = np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0xB8, 0x3C, 0x7E, 0xFE, 0x7F, 0xFF],
                     dtype=np.uint8)
    want = [0.0, -0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, -1.0, 1.5, 448.0, -448.0,
            np.nan, np.nan]
    got = F.e4m3_decode(codes)
    np.testing.assert_array_equal(got, np.array(want))
    assert np.signbit(got[1])


def test_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(F.e4m3_decode(codes), ref)


def test_decode_monotone_positive():
    v = F.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_padded_keys():
    assert [F.padded_keys(n) for n in (1, 15, 16, 17, 32, 100)] == [16, 16, 16, 32, 32, 112]


def _codes(x):
    return torch.from_numpy(np.ascontiguousarray(x)).float().to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def _random_fp8(B, Hq, Hkv, N, d, seed):
    rng = np.random.default_rng(seed)
    q8 = _codes(rng.standard_normal((B, Hq, N, d)))
    k8 = _codes(rng.standard_normal((B, Hkv, N, d)))
    Np = F.padded_keys(N)
    vt = np.zeros((B, Hkv, d, Np))
    vt[..., :N] = rng.standard_normal((B, Hkv, d, N))
    return q8, k8, _codes(vt)


def test_constant_v_and_padding_ignored():
    """Constant V over the keys gives O = v_scale * that constant; NaN codes in
    the padding keys (N .. Np-1) do not reach the result."""
    B, Hq, Hkv, N, d = 1, 2, 1, 21, 8
    q8, k8, vt8 = _random_fp8(B, Hq, Hkv, N, d, 3)
    col = _codes(np.linspace(-3, 3, d))
    vt8 = np.broadcast_to(col[None, None, :, None], (B, Hkv, d, F.padded_keys(N))).copy()
    vt8[..., N:] = 0x7F                                   # NaN codes in the padding
    O, lse = F.attention_fp8_ref(q8, k8, vt8, 0.5, 2.0, 0.25, 0.3)
    want = 0.25 * F.e4m3_decode(col)
    np.testing.assert_allclose(O[0, 0], np.broadcast_to(want, (N, d)), rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_dequantize_layout():
    """v comes back as [B, Hkv, N, d] with v[..., j, c] from vt[..., c, j]."""
    vt8 = np.arange(2 * 3 * 16, dtype=np.uint8).reshape(1, 1, 6, 16) % 0x70
    q8 = np.zeros((1, 1, 5, 6), dtype=np.uint8)
    k8 = np.zeros((1, 1, 5, 6), dtype=np.uint8)
    _, _, v = F.dequantize(q8, k8, vt8, 1.0, 1.0, 2.0, 5)
    assert v.shape == (1, 1, 5, 6)
    for j in range(5):
        for c in range(6):
            assert v[0, 0, j, c] == 2.0 * F.e4m3_decode(vt8[0, 0, c, j])


def test_scales_enter_scores_and_values():
    """The scales multiply the decoded codes: scaling q_scale by t equals scaling
    the score scale by t; v_scale multiplies O."""
    q8, k8, vt8 = _random_fp8(1, 1, 1, 40, 16, 5)
    O1, l1 = F.attention_fp8_ref(q8, k8, vt8, 0.5, 1.0, 1.0, 0.2)
    O2, l2 = F.attention_fp8_ref(q8, k8, vt8, 1.0, 1.0, 3.0, 0.1)
    np.testing.assert_allclose(3.0 * O1, O2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# the error bound against an emulation of the rounding it describes

def _emulate(S, V, rng, below=2.0):
    """O' = sum_j round(2^6 e^(S_j - m)) v_j / sum_j 2^6 e^(S_j - m), m drawn
    in [M - below * ln 2, M] per row, rounding by torch's E4M3 cast."""
    M = S.max(axis=1, keepdims=True)
    m = M - rng.uniform(0.0, below * math.log(2.0), size=M.shape)
    p = 64.0 * np.exp(S - m)
    pt = _codes(p)
    pr = F.e4m3_decode(pt)
    return (pr @ V) / p.sum(axis=1, keepdims=True)


def _bound_from(S, V, u=F.U_E4M3, e=F.E_ABS, slack=F.FP32_SLACK):
    W, _ = oracle.softmax_rows(S)
    av = np.abs(V)
    return (u + slack) * (W @ av) + e * W.max(axis=1, keepdims=True) * av.sum(axis=0, keepdims=True)


def _cases():
    rng = np.random.default_rng(11)
    N, d = 2048, 16
    V = rng.standard_normal((N, d))
    yield "normal", 0.3 * rng.standard_normal((64, N)), V
    yield "wide", 4.0 * rng.standard_normal((64, N)), V
    # one dominant key; every other weight ~2^-16.5 of it after the 2^6 scale
    # lands below half the smallest subnormal and is flushed to zero
    S = np.full((8, N), -(16.5 * math.log(2.0)))
    S[:, 0] = 0.0
    Vf = np.abs(V) + 1.0
    Vf[0] = 0.0                  # the dominant key's own rounding adds nothing
    yield "flushed", S, Vf
    # weights spread over the subnormal range
    S = -math.log(2.0) * rng.uniform(0.0, 14.0, size=(32, N))
    S[:, 5] = 0.0
    yield "subnormal", S, V


@pytest.mark.parametrize("name,S,V", list(_cases()), ids=lambda x: x if isinstance(x, str) else "")
def test_bound_holds_under_emulation(name, S, V):
    rng = np.random.default_rng(7)
    O = oracle.softmax_rows(S)[0] @ V
    bound = _bound_from(S, V)
    worst = 0.0
    for _ in range(4):
        err = np.abs(_emulate(S, V, rng) - O)
        assert np.all(err <= bound), (name, float(np.max(err - bound)))
        worst = max(worst, float(np.max(err / bound)))
    assert worst > 0.02, (name, worst)     # the bound is not vacuous


def test_bound_fails_without_flush_term():
    """Planted: no absolute (subnormal / flush) term -> the flushed case, with
    the running maximum at the true one, breaks it."""
    rng = np.random.default_rng(7)
    name, S, V = [c for c in _cases() if c[0] == "flushed"][0]
    O = oracle.softmax_rows(S)[0] @ V
    err = np.abs(_emulate(S, V, rng, below=0.0) - O)
    assert np.all(err <= _bound_from(S, V))
    assert np.any(err > _bound_from(S, V, e=0.0))


def test_bound_fails_with_halved_u():
    """Planted: u = 2^-5 (a 4-bit mantissa) -> the wide case breaks it somewhere."""
    rng = np.random.default_rng(7)
    name, S, V = [c for c in _cases() if c[0] == "wide"][0]
    O = oracle.softmax_rows(S)[0] @ V
    assert np.any(np.abs(_emulate(S, V, rng) - O) > _bound_from(S, V, u=2.0 ** -5, slack=0.0))


def test_oracle_bound_matches_direct_form():
    """fp8_error_bound on 8-bit inputs equals the direct formula on the decoded
    values, with the score term 2 eps_s max_j |scale| sum_c |q_ic k_jc| added
    to the relative part; fp8_lse_bound is that score term's half."""
    q8, k8, vt8 = _random_fp8(1, 2, 1, 50, 32, 9)
    b = F.fp8_error_bound(q8, k8, vt8, 0.7, 1.1, 0.5, -0.2)
    lb = F.fp8_lse_bound(q8, k8, vt8, 0.7, 1.1, 0.5, -0.2)
    q, k, v = F.dequantize(q8, k8, vt8, 0.7, 1.1, 0.5, 50)
    for h in range(2):
        S = -0.2 * q[0, h] @ k[0, 0].T
        A = 0.2 * np.abs(q[0, h]) @ np.abs(k[0, 0]).T          # >= |S| entrywise
        assert np.all(A >= np.abs(S) - 1e-12)
        ds = F.EPS_S * A.max(axis=1)
        W = oracle.softmax_rows(S)[0]
        want = _bound_from(S, v[0, 0]) + 2.0 * ds[:, None] * (W @ np.abs(v[0, 0]))
        np.testing.assert_allclose(b[0, h], want, rtol=1e-12)
        np.testing.assert_allclose(lb[0, h], ds, rtol=1e-12)


def test_score_perturbation_within_bound():
    """Scores perturbed by up to eps_s * A_ij (the contract's score error) move O
    by less than the score term of the bound."""
    rng = np.random.default_rng(3)
    q8, k8, vt8 = _random_fp8(1, 1, 1, 300, 64, 4)
    q, k, v = F.dequantize(q8, k8, vt8, 1.0, 1.0, 1.0, 300)
    S = 0.125 * q[0, 0] @ k[0, 0].T
    A = 0.125 * np.abs(q[0, 0]) @ np.abs(k[0, 0]).T
    dS = F.EPS_S * A * rng.choice([-1.0, 1.0], size=A.shape)
    W0, l0 = oracle.softmax_rows(S)
    W1, l1 = oracle.softmax_rows(S + dS)
    ds = F.EPS_S * A.max(axis=1)
    assert np.all(np.abs(l1 - l0) <= ds)
    assert np.all(np.abs(W1 @ v[0, 0] - W0 @ v[0, 0]) <= 2.0 * ds[:, None] * (W0 @ np.abs(v[0, 0])) * 1.01)


def test_mean_square_bound_holds_under_emulation():
    """The mean square of the emulated error stays under the predicted bound."""
    rng = np.random.default_rng(5)
    N, d = 1024, 16
    V = rng.standard_normal((N, d))
    S = 1.5 * rng.standard_normal((256, N))
    O = oracle.softmax_rows(S)[0] @ V
    W = oracle.softmax_rows(S)[0]
    pred = (F.U_E4M3 ** 2 / 3.0) * ((W * W) @ (V * V))
    err = _emulate(S, V, rng) - O
    assert np.mean(err ** 2) <= np.mean(pred)


def _f32_toward_zero(x):
    """Round float64 values to float32 toward zero (a directed rounding)."""
    r = x.astype(np.float32)
    over = np.abs(r.astype(np.float64)) > np.abs(x)
    r[over] = np.nextafter(r[over], np.float32(0.0))
    return r


def _sum_f32(prod, order, toward_zero):
    """Sum the rows of `prod` (exact products) in fp32 in the given order:
    'forward', 'reverse' (sequential) or 'tree' (pairwise), each addition
    rounded once, to nearest or toward zero."""
    rnd = _f32_toward_zero if toward_zero else (lambda x: x.astype(np.float32))
    p = prod[:, ::-1] if order == "reverse" else prod
    if order == "tree":
        cur = p.astype(np.float32)
        while cur.shape[1] > 1:
            cur = rnd(cur[:, 0::2].astype(np.float64) + cur[:, 1::2].astype(np.float64))
        return cur[:, 0].astype(np.float64)
    acc = p[:, 0].astype(np.float32)
    for c in range(1, p.shape[1]):
        acc = rnd(acc.astype(np.float64) + p[:, c])
    return acc.astype(np.float64)


@pytest.mark.parametrize("d", [64, 128])
def test_score_error_constant_covers_fp32_summation(d):
    """Size of eps_s: E4M3 x E4M3 products are exact in fp32 (at most 8
    significant bits); summing d of them in fp32 -- sequentially either way
    or as a pairwise tree, rounding to nearest or toward zero -- stays within
    (d - 1) 2^-23 sum_c |q_c k_c|, and eps_s is four times that bound at
    d = 128.  Inputs span the E4M3 range, with mixed signs so the sums cancel."""
    rng = np.random.default_rng(d)
    codes = rng.integers(0, 256, size=(2, 4000, d)).astype(np.uint8)
    vals = F.e4m3_decode(codes)
    vals = np.where(np.isnan(vals), 0.0, vals)
    prod = vals[0] * vals[1]
    assert np.all(prod.astype(np.float32).astype(np.float64) == prod)   # exact in fp32
    exact = prod.sum(axis=1)                                             # exact in fp64 here
    mag = np.abs(prod).sum(axis=1)
    bound = (d - 1) * 2.0 ** -23 * mag
    worst = 0.0
    for order in ("forward", "reverse", "tree"):
        for tz in (False, True):
            err = np.abs(_sum_f32(prod, order, tz) - exact)
            assert np.all(err <= bound), (order, tz)
            worst = max(worst, float(np.max(err / np.maximum(mag, 1e-300))))
    assert worst > 0.0
    assert F.EPS_S == 4 * 2.0 ** -16 and 127 * 2.0 ** -23 < 2.0 ** -16


def test_bounds_rows_equal_the_whole_tensor_bounds():
    """fp8_bounds_rows on selected rows of one head equals the rows of the
    whole-tensor fp8_error_bound and fp8_lse_bound."""
    q8, k8, vt8 = _random_fp8(2, 4, 2, 70, 64, 13)
    args = (q8, k8, vt8, 0.6, 1.3, 0.4, 0.11)
    b = F.fp8_error_bound(*args)
    lb = F.fp8_lse_bound(*args)
    q, k, v = F.dequantize(q8, k8, vt8, 0.6, 1.3, 0.4, 70)
    rows = [0, 5, 33, 69]
    for (bb, h) in [(0, 0), (1, 3), (0, 2)]:
        got, ds = F.fp8_bounds_rows(q, k, v, bb, h, rows, 0.11)
        np.testing.assert_allclose(got, b[bb, h, rows], rtol=1e-12)
        np.testing.assert_allclose(ds, lb[bb, h, rows], rtol=1e-12)
