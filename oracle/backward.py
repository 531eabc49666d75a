"""CPU oracle: gradients of exact attention, in float64.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT (same rules as attention.py:
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may use it; it never touches the GPU path).

The pages say the IO-aware method also speeds up the backward pass by
recomputing the blocks it needs instead of storing the [n, n] matrices
(blog "attention 的显存线性化", section 五; "efficient attention" chapter,
the interactive online-softmax section: recomputation instead of keeping the
attention matrix).  Recomputation changes where the numbers come from, not
what they are, so the oracle is the plain definition's gradient: for a
scalar loss L with dL/dO = dO given, dQ, dK, dV are the derivatives of

    O = softmax(scale * Q K^T) V        (per head, kv = h // (Hq / Hkv))

taken by reverse-mode automatic differentiation of exactly the forward the
forward oracle writes out (a library primitive used as one step), in
float64.  A K/V head's gradient sums those of the query heads that share it.
Each head is differentiated on its own, so memory stays at one [N, N]
matrix per head.
"""
from __future__ import annotations

import numpy as np

from .attention import _check, default_scale, kv_head


def attention_bwd_head(q_h, k_h, v_h, do_h, scale: float):
    """(dQ, dK, dV) of one head: q_h, do_h [N, d]; k_h, v_h [N, d]; float64."""
    import torch

    tq = torch.tensor(np.asarray(q_h, dtype=np.float64), requires_grad=True)
    tk = torch.tensor(np.asarray(k_h, dtype=np.float64), requires_grad=True)
    tv = torch.tensor(np.asarray(v_h, dtype=np.float64), requires_grad=True)
    S = scale * (tq @ tk.T)
    P = torch.softmax(S, dim=-1)
    O = P @ tv
    O.backward(torch.tensor(np.asarray(do_h, dtype=np.float64)))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def attention_bwd_ref(q, k, v, do, scale=None):
    """(dQ [B,Hq,N,d], dK [B,Hkv,N,d], dV [B,Hkv,N,d]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq, Hkv, N, d = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have q's shape")
    scale = default_scale(d) if scale is None else float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv = kv_head(h, Hq, Hkv)
            gq, gk, gv = attention_bwd_head(q[b, h], k[b, kv], v[b, kv], do[b, h], scale)
            dq[b, h] = gq
            dk[b, kv] += gk
            dv[b, kv] += gv
    return dq, dk, dv
