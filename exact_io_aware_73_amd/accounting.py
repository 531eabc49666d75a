"""FLOP and byte accounting for attention forward (measurement helpers).

Pure integer arithmetic about tensor sizes; no attention arithmetic.

* FLOPs: each of the two products S = Q K^T and O = P V costs n*n*d
  multiply-adds per head (aiknowledge.cn "1.1 注意力计算的计算与显存瓶颈",
  section 1.1.3), i.e. 2*n*n*d FLOPs (section 1.1.5 counts Q K^T as
  2*n^2*d).  Forward total per head: 4*n^2*d.  exp / max / sum are not
  counted.
* Materialised S and P: n*n elements each (section 1.1.2 counts both in
  fp16, 4*n^2 bytes together).
* Minimum HBM bytes of the fused forward: read Q, K, V once and write O once
  (blog "attention 的显存线性化", section 四: only the O(N) inputs and
  outputs are kept).
"""
from __future__ import annotations


def attn_fwd_flops(B: int, Hq: int, N: int, d: int) -> int:
    """Algorithmic FLOPs of one attention forward: 4 * B * Hq * N^2 * d."""
    return 4 * B * Hq * N * N * d


def qk_flops(n: int, d: int) -> int:
    """FLOPs of S = Q K^T for one [n, d] head: 2 * n^2 * d."""
    return 2 * n * n * d


def min_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elem: int) -> int:
    """Q, K, V read once and O written once: elem * (2*B*Hq*N*d + 2*B*Hkv*N*d)."""
    return elem * (2 * B * Hq * N * d + 2 * B * Hkv * N * d)


def bwd_min_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elem: int) -> int:
    """The backward's least traffic: Q, K, V, O, dO and the fp32 lse read
    once, dQ, dK, dV written once."""
    return elem * (3 * B * Hq * N * d + 2 * B * Hkv * N * d) + 4 * B * Hq * N \
        + elem * (B * Hq * N * d + 2 * B * Hkv * N * d)


def lse_bytes(B: int, Hq: int, N: int) -> int:
    """The fp32 log-sum-exp output, B*Hq*N values."""
    return 4 * B * Hq * N


def nn_matrix_bytes(n: int, elem: int) -> int:
    """One [n, n] matrix of ``elem``-byte elements."""
    return n * n * elem


def sp_bytes(n: int, elem: int = 2) -> int:
    """S and P together, one head: 2 * n^2 * elem (4 n^2 bytes in fp16)."""
    return 2 * nn_matrix_bytes(n, elem)


def softmax_flops(n: int) -> int:
    """About 3 operations per score (subtract max, exp, divide): 3 * n^2."""
    return 3 * n * n


def softmax_bytes(n: int, elem: int = 2) -> int:
    """Read S and write P once each: 2 * n^2 * elem."""
    return 2 * n * n * elem


def materialized_bytes(B: int, Hq: int, Hkv: int, N: int, d: int, elem: int,
                       s_elem: int = 4, include_lse: bool = False) -> int:
    """Predicted HBM bytes of the three-kernel materialising path.

    S (``s_elem`` bytes per score) is written once and read once, P (I/O
    dtype) is written once and read once, and Q, K, V, O move once each.
    """
    nn = B * Hq * N * N
    total = 2 * nn * s_elem + 2 * nn * elem + min_bytes(B, Hq, Hkv, N, d, elem)
    if include_lse:
        total += lse_bytes(B, Hq, N)
    return total


# ---------------------------------------------------------------------------
# MI355X (gfx950) peaks, from AMD's published specification.
CU_COUNT = 256
XCD_COUNT = 8
PEAK_CLOCK_GHZ = 2.4
BF16_DENSE_FLOP_PER_CLK_PER_CU = 4096
PEAK_BF16_TFLOPS = 2516.6          # 256 CU * 2.4 GHz * 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2           # dense FP8 MFMA: twice the bf16 rate
# fp32 vector FMA without the packed (two-per-lane) instructions, which the
# library is built without: 256 CU * 2.4 GHz * 64 FMA lanes * 2 FLOP.  The
# published 157.3 TFLOP/s counts the packed form.
PEAK_FP32_VECTOR_TFLOPS = 78.6
PEAK_HBM_GBPS = 8000.0


def peak_bf16_tflops(cus: int = CU_COUNT, ghz: float = PEAK_CLOCK_GHZ) -> float:
    return cus * ghz * 1e9 * BF16_DENSE_FLOP_PER_CLK_PER_CU / 1e12
