"""GPU parity of the backward (attn_bwd, through the C ABI) against the fp64
oracle (oracle/backward.py), on the same seeded bf16 inputs.

Tolerance: the kernels round P and dS to bf16 (relative error 2^-9) before
the products that consume them and the gradients to bf16 on output, and
take D = rowsum(dO * O) from the forward's bf16 O; with fp32 accumulation
the error of each gradient stays near a few 2^-9 of its largest entry.  The
test allows 1 % of that entry (plus 1e-4 absolute, for gradients that are
exactly zero in the reference).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from exact_io_aware_73_amd import attn as a
    return a


def _grads(attn, q, k, v, do, scale):
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = attn.fwd(qd, kd, vd, scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, o, lse, dod, scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


def _check(attn, q, k, v, do, scale, label):
    got = _grads(attn, q, k, v, do, scale)
    ref = oracle.attention_bwd_ref(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                   workloads.to_f64(do), scale)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = float(np.max(np.abs(workloads.to_f64(g) - r)))
        tol = 1e-2 * float(np.max(np.abs(r))) + 1e-4
        assert err <= tol, (label, name, err, tol)


def _inputs(B, Hq, Hkv, N, d, seed):
    q, k, v = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=seed)
    do, _, _ = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed=seed + 7)
    return q, k, v, do


@pytest.mark.parametrize("d", [64, 128])
# 300, 400, 520: several dK/dV workgroups (256 keys each at d = 128), the
# last one with whole, partial and empty waves and key blocks
@pytest.mark.parametrize("N", [1, 17, 64, 65, 127, 128, 129, 300, 400, 520])
@pytest.mark.parametrize("B,Hq,Hkv", [(1, 1, 1), (2, 4, 2)])
def test_bwd_small(attn, B, Hq, Hkv, N, d):
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, 31 * N + d + Hq)
    _check(attn, q, k, v, do, 1 / math.sqrt(d), f"bwd {B},{Hq},{Hkv},{N},{d}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,Hq,Hkv,N", [(1, 16, 1, 1), (1, 16, 1, 33), (2, 12, 3, 100), (1, 32, 4, 77)])
def test_bwd_gqa_packed(attn, B, Hq, Hkv, N, d):
    """Query tiles shared by the heads of a K/V group, crossing head boundaries."""
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, 37 * N + d + Hq)
    _check(attn, q, k, v, do, 1 / math.sqrt(d), f"bwd packed {B},{Hq},{Hkv},{N},{d}")


@pytest.mark.parametrize("scale", [0.0, -0.1, 0.4])
def test_bwd_scales(attn, scale):
    q, k, v, do = _inputs(1, 2, 1, 200, 64, 77)
    _check(attn, q, k, v, do, scale, f"scale {scale}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_very_negative_logits_ragged(attn, d):
    """Every score near -150 (lse the same), N = 100 (a partial last key
    tile): a key past N would weigh exp(-lse) = e^150, past fp32 range, in
    the dQ kernel, which takes such keys without a mask (their K rows are
    zero); the clamped weight keeps them finite, so no inf or NaN reaches dQ."""
    N = 100
    q, k, v, do = _inputs(1, 2, 1, N, d, 400 + d)
    a = math.sqrt(150.0 / d)
    q = (a + 0.05 * q.float()).to(torch.bfloat16)
    k = (-a + 0.05 * k.float()).to(torch.bfloat16)
    got = _grads(attn, q, k, v, do, 1.0)
    assert all(torch.isfinite(g.float()).all() for g in got)
    ref = oracle.attention_bwd_ref(workloads.to_f64(q), workloads.to_f64(k), workloads.to_f64(v),
                                   workloads.to_f64(do), 1.0)
    # dV has no cancellation: the usual bound
    err = float(np.max(np.abs(workloads.to_f64(got[2]) - ref[2])))
    assert err <= 1e-2 * float(np.max(np.abs(ref[2]))) + 1e-4, ("dv", err)
    # dQ = dS K and dK = dS^T Q sum terms that nearly cancel (K and Q share a
    # large common part here), so the bf16 rounding of P and dS (2^-9 each)
    # is bounded per entry by the sum of the terms' magnitudes, not by the result
    Q, K, V, dO = (workloads.to_f64(x)[0] for x in (q, k, v, do))
    K, V = np.repeat(K, 2, axis=0), np.repeat(V, 2, axis=0)
    S = Q @ K.transpose(0, 2, 1)
    P = np.exp(S - S.max(-1, keepdims=True))
    P /= P.sum(-1, keepdims=True)
    dS = P * (dO @ V.transpose(0, 2, 1) - (dO * (P @ V)).sum(-1, keepdims=True))
    bound_q = 2.0 ** -7 * (np.abs(dS) @ np.abs(K)) + 1e-4
    bound_k = 2.0 ** -7 * np.abs(dS).transpose(0, 2, 1) @ np.abs(Q)
    bound_k = bound_k.reshape(1, 2, N, d).sum(1) + 1e-4
    assert np.all(np.abs(workloads.to_f64(got[0])[0] - ref[0][0]) <= bound_q), "dq"
    assert np.all(np.abs(workloads.to_f64(got[1])[0] - ref[1][0]) <= bound_k[0]), "dk"


def test_bwd_longer_gqa(attn):
    q, k, v, do = _inputs(1, 4, 1, 1024, 128, 91)
    _check(attn, q, k, v, do, 1 / math.sqrt(128), "N=1024 GQA 4:1")


def test_bwd_deterministic(attn):
    q, k, v, do = _inputs(2, 8, 2, 700, 128, 5)
    a = _grads(attn, q, k, v, do, 0.09)
    b = _grads(attn, q, k, v, do, 0.09)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_single_key(attn):
    """N = 1: dV = dO (summed over the group), dQ = dK = 0 up to rounding."""
    q, k, v, do = _inputs(2, 4, 2, 1, 64, 3)
    dq, dk, dv = _grads(attn, q, k, v, do, 0.3)
    assert dq.abs().max().item() <= 1e-4 and dk.abs().max().item() <= 1e-4
    want = workloads.to_f64(do).reshape(2, 2, 2, 1, 64).sum(axis=2)
    assert np.max(np.abs(workloads.to_f64(dv) - want)) <= 2 ** -7 * np.max(np.abs(want))


def test_python_bwd_rejects(attn):
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    o, lse = attn.fwd(q, q, q)
    ws = torch.empty(4, dtype=torch.uint8, device="cuda")   # too small
    with pytest.raises(ValueError):
        attn.attn_bwd(q, q, q, o, lse, q, torch.empty_like(q), torch.empty_like(q),
                      torch.empty_like(q), ws, 0.125)
    with pytest.raises(ValueError):
        attn.bwd(q.float(), q.float(), q.float(), o, lse, q)


# ---------------------------------------------------------------------------
# the shapes the backward is timed on, at full size: the whole batch runs on
# the GPU; sampled heads are checked element by element against the oracle
# (a K/V head's dK and dV against the sum over every query head of its group)
TIMED = {
    "gpt2_medium_b64_h16_n1024_d64": 3,
    "long_b4_h32_n4096_d128": 2,
    "gqa_b2_hq32_hkv8_n8192_d128": 1,
}


@pytest.mark.parametrize("name", list(TIMED))
def test_bwd_timed_workload(attn, name):
    w = workloads.WORKLOADS[name]
    print(f"[bwd] full workload {name}", flush=True)
    q, k, v = workloads.make_inputs(w)
    do = workloads.random_inputs(w.B, w.Hq, w.Hkv, w.N, w.d, torch.bfloat16, seed=w.seed + 9)[0]
    scale = 1 / math.sqrt(w.d)
    dq, dk, dv = (t.cpu() for t in _grads(attn, q, k, v, do, scale))
    g = w.Hq // w.Hkv
    rng = np.random.default_rng(w.seed)
    groups = {(0, 0), (w.B - 1, w.Hkv - 1)}
    while len(groups) < TIMED[name]:
        groups.add((int(rng.integers(w.B)), int(rng.integers(w.Hkv))))
    for (b, kvh) in sorted(groups)[:TIMED[name]]:
        kk, vv = workloads.to_f64(k[b, kvh]), workloads.to_f64(v[b, kvh])
        dk_ref = np.zeros_like(kk)
        dv_ref = np.zeros_like(vv)
        for h in range(kvh * g, (kvh + 1) * g):
            gq, gk, gv = oracle.attention_bwd_head(workloads.to_f64(q[b, h]), kk, vv,
                                                   workloads.to_f64(do[b, h]), scale)
            dk_ref += gk
            dv_ref += gv
            err = float(np.max(np.abs(workloads.to_f64(dq[b, h]) - gq)))
            tol = 1e-2 * float(np.max(np.abs(gq))) + 1e-4
            assert err <= tol, (name, (b, h), "dq", err, tol)
        for gname, got, ref in (("dk", dk[b, kvh], dk_ref), ("dv", dv[b, kvh], dv_ref)):
            err = float(np.max(np.abs(workloads.to_f64(got) - ref)))
            tol = 1e-2 * float(np.max(np.abs(ref))) + 1e-4
            assert err <= tol, (name, (b, kvh), gname, err, tol)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
