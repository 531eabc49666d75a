"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm).

No entry point allocates, synchronises or clears memory with a memset, so a
caller may capture them.  Each graph is replayed several times with eager
work (new inputs written in place) and synchronisations between replays, and
every replay must equal the eager call bit for bit (the kernels are
deterministic).
"""
from __future__ import annotations

import math
import sys

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from exact_io_aware_73_amd import attn as a   # fails loudly if libattn.so is missing
    return a


def _inputs(B, Hq, Hkv, N, d, seed):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=seed)
    return q.cuda(), k.cuda(), v.cuda()


def _capture(fn):
    """Warm fn up on a side stream, then capture it into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _refill(ts, seed):
    """Eager work between replays: new inputs written into the captured tensors."""
    for i, t in enumerate(ts):
        gen = torch.Generator(device="cuda").manual_seed(seed + i)
        t.copy_(torch.randn(t.shape, device="cuda", generator=gen).to(t.dtype))


@pytest.mark.parametrize("d", [64, 128])
def test_graph_fwd(attn, d):
    print(f"[graph] attn_fwd d={d}", file=sys.stderr, flush=True)
    q, k, v = _inputs(2, 8, 2, 300, d, seed=31 + d)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    g = _capture(lambda: attn.attn_fwd(q, k, v, o, lse, scale))
    for rep in range(3):
        _refill((q, k, v), seed=100 * rep + d)
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = attn.fwd(q, k, v, scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {rep}"


def test_graph_split_and_bwd(attn):
    print("[graph] attn_fwd_split + attn_bwd d=128", file=sys.stderr, flush=True)
    q, k, v = _inputs(1, 4, 2, 500, 128, seed=77)
    scale = 1.0 / math.sqrt(128)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(attn.attn_fwd_split_workspace_bytes(1, 4, 500, 128, 3), dtype=torch.uint8,
                     device="cuda")
    dout = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    wsb = torch.empty(attn.attn_bwd_workspace_bytes(1, 4, 500), dtype=torch.uint8, device="cuda")

    def step():
        attn.attn_fwd_split(q, k, v, o, lse, ws, 3, scale)
        attn.attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, wsb, scale)

    g = _capture(step)
    for rep in range(3):
        _refill((q, k, v, dout), seed=500 + 10 * rep)
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = attn.fwd_split(q, k, v, 3, scale)
        grads = attn.bwd(q, k, v, o_ref, lse_ref, dout, scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"split replay {rep}"
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
            assert torch.equal(got, ref), f"{name} replay {rep}"
