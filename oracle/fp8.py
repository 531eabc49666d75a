"""CPU oracle for the 8-bit floating-point forward, in float64.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run this module.  It shares no code with the GPU path and never
imports it.

The pages name FP8 among the features of the third FlashAttention version
and give nothing of its arithmetic (blog "attention 的显存线性化", section 五).
The reading taken here, stated as the contract of the 8-bit entry point:

  * Inputs are OCP 8-bit floating point E4M3 codes (the OCP "8-bit Floating
    Point Specification", format E4M3: one sign bit, four exponent bits with
    bias 7, three mantissa bits; exponent field 0 holds the subnormals
    m/8 * 2^-6; the code with all exponent and mantissa bits set is NaN;
    there is no infinity; the largest finite value is 448), one float scale
    per tensor:  q = q_scale * decode(q8),  k = k_scale * decode(k8),
    v = v_scale * decode(v8).  V comes transposed, [B, Hkv, d, Np] with
    Np = N rounded up to a multiple of 16; keys N .. Np-1 are not data.
  * The reference result is the plain definition (``attention_ref``) on the
    decoded, scaled inputs, so the scores and lse are those of exact
    attention of those values.
  * The one step that loses precision: each weight is rounded to E4M3 before
    the PV product.  A weight is p_j = exp(S_j - m), m a running row maximum
    that is never above the row's true maximum M and never more than
    2 (in log2 units) below it when the row's largest weights are met; it is
    multiplied by 2^6 before rounding (so e^M - m <= 2^8 < 448 never
    overflows).  The exp-sum l adds the unrounded weights.
  * Error bound (derived here, not on the pages).  Rounding to nearest on
    E4M3 has relative error <= u = 2^-4 on normal values and absolute error
    <= 2^-10 (half the subnormal spacing 2^-9) below them, i.e. <= 2^-16 in
    units of e^m, hence <= 2^-16 * e^M.  With w_j = e^{S_j} / sum_k e^{S_k}
    the exact weights and O = sum_j w_j v_j, the path's
    O' = sum_j p~_j v_j / sum_j p_j differs from O by
        sum_j (p~_j - p_j) v_j / sum_j p_j,
    so per output element (i, c)
        |O'_ic - O_ic| <= sum_j (u * w_ij + e * w_i,max) * |v_jc|,
    e = 2^-16.  ``fp8_error_bound`` returns that, plus two slack terms on
    the relative part: 2^-12 for the fp32 arithmetic (exp2, the sums), and
    2 * eps_s * max_j A_ij for the scores, A_ij = |scale| * sum_c |q_ic| |k_jc|:
    the matrix core sums the exact 8-bit products into fp32 with an error
    the contract bounds by eps_s * A_ij (a score error dS_j moves the
    normalised weight w_j by a factor within exp(+-2 max_j |dS_j|)).  The
    same eps_s * max_j A_ij bounds the error of lse (``fp8_lse_bound``).
    The final rounding of O to bf16 is the caller's to add.
  * eps_s.  A product of two E4M3 values has at most 8 significant bits, so
    every product is exact in fp32; only the d - 1 additions round.  Summed
    in ANY order (any tree of pairwise additions), each addition rounded
    once, even toward zero (relative error < 2^-23 each), the sum differs
    from the exact one by at most (d - 1) 2^-23 sum_c |q_c k_c|: at d = 128
    that is 127 * 2^-23 < 2^-16.  The matrix core's internal order and
    rounding are not documented, so the contract takes four times that,
    eps_s = 2^-14, for the steps around it (the fp32 multiply by the scale,
    any wider internal partial sums rounded more than once).  The largest
    error seen on the GPU was about 2^-17 of the same sum.
  * For a statistical check: with independent rounding errors of relative
    size <= u (mean square <= u^2 / 3), the mean square of O' - O is at most
    (u^2 / 3) * sum_j w_ij^2 v_jc^2 per element; ``fp8_mean_square_bound``.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_ref, head_scores, kv_head, softmax_rows

U_E4M3 = 2.0 ** -4          # relative rounding error bound of E4M3 (3 mantissa bits)
E_ABS = 2.0 ** -16          # absolute weight error bound, relative to the row's largest
FP32_SLACK = 2.0 ** -12     # fp32 arithmetic around the 8-bit products
EPS_S = 2.0 ** -14          # score error allowed per unit of sum_c |q_c k_c| * |scale|:
                            # 4 x the any-order, toward-zero fp32 summation bound at d = 128


def padded_keys(N: int) -> int:
    """Row length of the transposed V: N rounded up to a multiple of 16."""
    return (N + 15) // 16 * 16


def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) as float64; NaN for the NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def dequantize(q8, k8, vt8, q_scale: float, k_scale: float, v_scale: float, N: int):
    """Decoded, scaled q, k, v (float64); v back in [B, Hkv, N, d] order."""
    q = q_scale * e4m3_decode(q8)
    k = k_scale * e4m3_decode(k8)
    vt = e4m3_decode(np.asarray(vt8)[..., :N])          # [B, Hkv, d, N]
    v = v_scale * np.ascontiguousarray(np.swapaxes(vt, -1, -2))
    return q, k, v


def attention_fp8_ref(q8, k8, vt8, q_scale, k_scale, v_scale, scale):
    """(O, lse) of exact attention on the dequantised inputs."""
    N = np.asarray(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, q_scale, k_scale, v_scale, N)
    return attention_ref(q, k, v, scale)


def _heads(q8, k8, vt8, q_scale, k_scale, v_scale, scale):
    """Per (b, h): exact weights W, the K/V head's v, and each row's
    score-error bound eps_s * max_j |scale| sum_c |q_ic| |k_jc|."""
    N = np.asarray(q8).shape[2]
    q, k, v = dequantize(q8, k8, vt8, q_scale, k_scale, v_scale, N)
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    for b in range(B):
        for h in range(Hq):
            kv = kv_head(h, Hq, Hkv)
            W, _ = softmax_rows(head_scores(q[b, h], k[b, kv], scale))
            ds = EPS_S * abs(scale) * (np.abs(q[b, h]) @ np.abs(k[b, kv]).T).max(axis=1)
            yield b, h, W, v[b, kv], ds


def _bound(W, v, ds):
    """The per-element bound of rows with exact weights W [rows, N], the K/V
    head's v [N, d] and score-error bounds ds [rows]."""
    av = np.abs(v)
    rel = U_E4M3 + FP32_SLACK + 2.0 * ds[:, None]
    return rel * (W @ av) + E_ABS * W.max(axis=1, keepdims=True) * av.sum(axis=0, keepdims=True)


def fp8_error_bound(q8, k8, vt8, q_scale, k_scale, v_scale, scale) -> np.ndarray:
    """Per-element bound on |O_path - O| (before the output's bf16 rounding)."""
    q8 = np.asarray(q8)
    out = np.zeros(q8.shape, dtype=np.float64)
    for b, h, W, v, ds in _heads(q8, k8, vt8, q_scale, k_scale, v_scale, scale):
        out[b, h] = _bound(W, v, ds)
    return out


def fp8_bounds_rows(q, k, v, b: int, h: int, rows, scale):
    """The same two bounds for selected query rows of one head, from the
    dequantised q, k, v (``dequantize``): (per-element bound [rows, d],
    lse bound [rows]).  For sampled checks of shapes too large for the
    whole-tensor functions."""
    kv = kv_head(h, q.shape[1], k.shape[1])
    qr = np.asarray(q[b, h])[np.asarray(rows)]
    W, _ = softmax_rows(head_scores(qr, k[b, kv], scale))
    ds = EPS_S * abs(scale) * (np.abs(qr) @ np.abs(k[b, kv]).T).max(axis=1)
    return _bound(W, v[b, kv], ds), ds


def fp8_lse_bound(q8, k8, vt8, q_scale, k_scale, v_scale, scale) -> np.ndarray:
    """Per-row bound on |lse_path - lse|: the score error bound of the row."""
    q8 = np.asarray(q8)
    out = np.zeros(q8.shape[:3], dtype=np.float64)
    for b, h, _, _, ds in _heads(q8, k8, vt8, q_scale, k_scale, v_scale, scale):
        out[b, h] = ds
    return out


def fp8_mean_square_bound(q8, k8, vt8, q_scale, k_scale, v_scale, scale) -> np.ndarray:
    """Per-element bound on the mean square of O_path - O from independent
    weight roundings: (u^2 / 3) * sum_j w_ij^2 v_jc^2."""
    q8 = np.asarray(q8)
    out = np.zeros(q8.shape, dtype=np.float64)
    for b, h, W, v, _ in _heads(q8, k8, vt8, q_scale, k_scale, v_scale, scale):
        out[b, h] = (U_E4M3 ** 2 / 3.0) * ((W * W) @ (v * v))
    return out
