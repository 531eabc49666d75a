"""CPU oracle: exact scaled-dot-product attention forward, in float64.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run this module.  It shares no code with the GPU path (no tiling,
no running max, no exp2, no common helpers) and never imports it.

What it computes is the plain full-matrix definition, because the pages say
the tiled method reaches exactly that result, only with less memory traffic
(blog "attention 的显存线性化", section 二: the result is mathematically
identical; course chapter "efficient attention" (deeplearning.wizardwu.top),
table of the three classes of fixes: zero loss, mathematically equivalent).
For every batch b and query head h, with kv = h // (Hq / Hkv):

    S[i, j]   = scale * sum_c Q[b,h,i,c] * K[b,kv,j,c]
    m_i       = max_j S[i, j]
    E[i, j]   = exp(S[i, j] - m_i),   l_i = sum_j E[i, j]
    P[i, j]   = E[i, j] / l_i
    O[b,h,i,:] = sum_j P[i, j] * V[b,kv,j,:]
    lse[b,h,i] = m_i + ln(l_i)

Sources for each line:
  * S, P = softmax(S), O = P V with the 1/sqrt(d) scale:
    aiknowledge.cn "1.1 注意力计算的计算与显存瓶颈", section 1.1.1 (the
    materialising listing) and the blog "attention 的显存线性化", section 一
    (Attention(Q,K,V) = softmax(QK^T / sqrt(d_k)) V).  ``scale`` is a caller
    value; it defaults to 1/sqrt(d).
  * The row softmax with the row maximum subtracted before exp:
    aiknowledge.cn "1.1 ...", section 1.1.8 (first of the two sections so
    numbered).
  * Rows are independent (same section), so splitting the query rows into
    chunks of whole rows changes nothing; every chunk still sees its full
    key range.
  * Grouped-query attention (several query heads share one K/V head): the
    "efficient attention" chapter, class 3 and its methods table.  The pages
    give no index rule; the reading used is contiguous groups,
    kv = h // (Hq / Hkv).
  * lse, the natural log of each row's exp-sum, is not on the pages; it is
    part of this library's output contract (a backward pass needs it).

Inputs are NumPy float64 arrays (the exact upcast of the bf16 / fp32 tensors
the GPU sees): q [B, Hq, N, d], k and v [B, Hkv, N, d].
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# bytes of float64 scores allowed per row chunk (whole rows only)
_CHUNK_BYTES = 64 << 20


def default_scale(d: int) -> float:
    """1/sqrt(d): the scale of the scores in the pages' definition."""
    return 1.0 / math.sqrt(d)


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """K/V head shared by query head ``h``: contiguous groups of Hq/Hkv heads."""
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def softmax_rows(S: np.ndarray):
    """Row-wise softmax of a score block and each row's log-sum-exp.

    P_i = exp(S_i - max S_i) / sum_j exp(S_ij - max S_i); lse_i = max S_i + ln sum_j ...
    (aiknowledge.cn "1.1 ...", section 1.1.8).  Returns (P, lse), float64.
    """
    S = np.asarray(S, dtype=np.float64)
    m = S.max(axis=-1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=-1, keepdims=True)
    P = E / l
    lse = (m + np.log(l))[..., 0]
    return P, lse


def head_scores(q_h: np.ndarray, k_h: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one head: q_h [n_rows, d], k_h [N, d] -> [n_rows, N]."""
    return scale * (q_h @ k_h.T)


def attention_head(q_h, k_h, v_h, scale: float, rows=None):
    """(O, lse) of one head, for all rows or for the given row indices.

    Rows are processed in chunks of whole rows; each chunk forms its full
    score rows, takes the row softmax and multiplies by V.
    """
    q_h = np.asarray(q_h, dtype=np.float64)
    k_h = np.asarray(k_h, dtype=np.float64)
    v_h = np.asarray(v_h, dtype=np.float64)
    if rows is not None:
        q_h = q_h[np.asarray(rows)]
    n_rows, N = q_h.shape[0], k_h.shape[0]
    O = np.empty((n_rows, v_h.shape[1]), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    chunk = max(1, min(n_rows, _CHUNK_BYTES // (8 * max(N, 1))))
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        S = head_scores(q_h[r0:r1], k_h, scale)
        P, lse[r0:r1] = softmax_rows(S)
        O[r0:r1] = P @ v_h
    return O, lse


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k, v must be [B, Hkv, N, d] matching q")
    Hkv = k.shape[1]
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return B, Hq, Hkv, N, d


def attention_ref(q, k, v, scale=None, workers: int = 1):
    """Full forward: (O [B,Hq,N,d], lse [B,Hq,N]), float64.

    ``workers`` > 1 runs the (b, h) slices on a thread pool (NumPy's matmul
    and exp release the GIL); BLAS is then held to one thread per worker.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, N, d = _check(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    O = np.empty((B, Hq, N, d), dtype=np.float64)
    lse = np.empty((B, Hq, N), dtype=np.float64)

    def one(bh):
        b, h = divmod(bh, Hq)
        kv = kv_head(h, Hq, Hkv)
        O[b, h], lse[b, h] = attention_head(q[b, h], k[b, kv], v[b, kv], scale)

    if workers <= 1:
        for bh in range(B * Hq):
            one(bh)
    else:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one, range(B * Hq)))
    return O, lse


def attention_ref_rows(q, k, v, b: int, h: int, rows, scale=None):
    """(O, lse) for selected query rows of one (b, h): for sampled checks at full size."""
    q = np.asarray(q)
    k = np.asarray(k)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = default_scale(d) if scale is None else float(scale)
    kv = kv_head(h, Hq, Hkv)
    return attention_head(q[b, h], k[b, kv], np.asarray(v)[b, kv], scale, rows=rows)


def attention_ref_sp(q, k, v, scale=None):
    """Full forward that also returns the score and weight matrices.

    (O, lse, S, P) with S, P [B, Hq, N, N] in float64: the standard,
    materialising computation the pages compare against (aiknowledge.cn
    "1.1 ...", section 1.1.1).  Small sizes only.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Hkv, N, d = _check(q, k, v)
    scale = default_scale(d) if scale is None else float(scale)
    S = np.empty((B, Hq, N, N), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kv = kv_head(h, Hq, Hkv)
            S[b, h] = head_scores(q[b, h], k[b, kv], scale)
    P, lse = softmax_rows(S)
    O = np.empty((B, Hq, N, d), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            O[b, h] = P[b, h] @ v[b, kv_head(h, Hq, Hkv)]
    return O, lse, S, P
