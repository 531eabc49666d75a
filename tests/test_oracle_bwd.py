"""Pins of the backward oracle (oracle/backward.py), CPU only.

The oracle differentiates the plain forward by reverse-mode autodiff; these
checks tie it to things that do not use autodiff: central finite
differences of the pinned forward oracle on tiny inputs, closed forms
(one key; scale 0; constant V), invariants that follow from softmax's
shift invariance, and grouped-query heads as sums over repeated heads.
Each plausible mistake planted in a copy of the oracle below fails one.
"""
import numpy as np
import pytest

import oracle
from oracle import backward as bwd


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(B, Hq, Hkv, N, d, seed):
    return (_rand((B, Hq, N, d), seed), _rand((B, Hkv, N, d), seed + 1),
            _rand((B, Hkv, N, d), seed + 2), _rand((B, Hq, N, d), seed + 3))


def _loss(q, k, v, do, scale):
    O, _ = oracle.attention_ref(q, k, v, scale)
    return float(np.sum(O * do))


def _fd_grads(q, k, v, do, scale, h=1e-5):
    """Central differences of L = sum(O * dO) through the forward oracle."""
    out = []
    for which in range(3):
        arrs = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(arrs[which])
        it = np.nditer(arrs[which], flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            x0 = arrs[which][i]
            arrs[which][i] = x0 + h
            lp = _loss(*arrs, do, scale)
            arrs[which][i] = x0 - h
            lm = _loss(*arrs, do, scale)
            arrs[which][i] = x0
            g[i] = (lp - lm) / (2 * h)
        out.append(g)
    return out


FD_CASES = [(1, 1, 1, 1, 2, 0.7), (1, 1, 1, 3, 2, 0.7), (1, 2, 1, 4, 3, -0.3),
            (2, 4, 2, 3, 2, 1.3), (1, 2, 2, 5, 1, 0.5)]


def fd_pin(ref, B, Hq, Hkv, N, d, scale, seed=0):
    q, k, v, do = _inputs(B, Hq, Hkv, N, d, seed)
    got = ref(q, k, v, do, scale)
    want = _fd_grads(q, k, v, do, scale)
    return all(np.max(np.abs(a - b)) <= 1e-7 for a, b in zip(got, want))


@pytest.mark.parametrize("case", FD_CASES)
def test_finite_differences(case):
    assert fd_pin(oracle.attention_bwd_ref, *case)


def test_one_key():
    """N = 1: O = V_0 whatever Q, K: dV = dO (summed over the group), dQ = dK = 0."""
    q, k, v, do = _inputs(2, 4, 2, 1, 8, 5)
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, 0.4)
    assert np.max(np.abs(dq)) == 0.0 and np.max(np.abs(dk)) <= 1e-15
    want = do.reshape(2, 2, 2, 1, 8).sum(axis=2)
    assert np.max(np.abs(dv - want)) <= 1e-12


def test_scale_zero():
    """scale = 0: P is uniform 1/N, so dV_j = mean_i dO_i and dQ = dK = 0."""
    q, k, v, do = _inputs(1, 2, 1, 7, 4, 6)
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, 0.0)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    want = np.broadcast_to(do.sum(axis=1, keepdims=True).mean(axis=2, keepdims=True), dv.shape)
    assert np.max(np.abs(dv - want)) <= 1e-12


def test_constant_v():
    """Every V row equal: O does not depend on the weights, dQ = dK = 0."""
    q, k, _, do = _inputs(1, 2, 1, 6, 3, 7)
    v = np.broadcast_to(_rand((1, 1, 1, 3), 8), (1, 1, 6, 3)).copy()
    dq, dk, _ = oracle.attention_bwd_ref(q, k, v, do, 0.9)
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12


def test_key_gradients_sum_to_zero():
    """Each row of the score gradient sums to 0 (shift invariance), so the
    key gradients of a K/V head sum to zero over the keys."""
    q, k, v, do = _inputs(2, 4, 2, 9, 5, 9)
    _, dk, _ = oracle.attention_bwd_ref(q, k, v, do, 0.6)
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12


def test_key_shift_invariance():
    """K + 1 u^T shifts every score of a row by q.u: P, and so dQ, dK, dV, stay."""
    q, k, v, do = _inputs(1, 2, 1, 6, 4, 10)
    u = _rand((4,), 11)
    a = oracle.attention_bwd_ref(q, k, v, do, 0.5)
    b = oracle.attention_bwd_ref(q, k + u, v, do, 0.5)
    for x, y in zip(a, b):
        assert np.max(np.abs(x - y)) <= 1e-10


def test_gqa_is_sum_over_repeated_heads():
    q, k, v, do = _inputs(1, 4, 2, 5, 3, 12)
    dq, dk, dv = oracle.attention_bwd_ref(q, k, v, do, 0.8)
    rk, rv = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_bwd_ref(q, rk, rv, do, 0.8)
    assert np.max(np.abs(dq - dq2)) <= 1e-12
    assert np.max(np.abs(dk - dk2.reshape(1, 2, 2, 5, 3).sum(axis=2))) <= 1e-12
    assert np.max(np.abs(dv - dv2.reshape(1, 2, 2, 5, 3).sum(axis=2))) <= 1e-12


# ---------------------------------------------------------------------------
# plausible mistakes, each in a copy of the oracle: a pin above must fail
def _mutant(head_fn=None, overwrite=False):
    def ref(q, k, v, do, scale):
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(B):
            for h in range(Hq):
                kv = h // (Hq // Hkv)
                gq, gk, gv = (head_fn or bwd.attention_bwd_head)(q[b, h], k[b, kv], v[b, kv], do[b, h], scale)
                dq[b, h] = gq
                if overwrite:
                    dk[b, kv], dv[b, kv] = gk, gv
                else:
                    dk[b, kv] += gk
                    dv[b, kv] += gv
        return dq, dk, dv
    return ref


def _head(mistake):
    def fn(q_h, k_h, v_h, do_h, scale):
        import torch
        tq = torch.tensor(q_h, requires_grad=True)
        tk = torch.tensor(k_h, requires_grad=True)
        tv = torch.tensor(v_h, requires_grad=True)
        s = 1.0 if mistake == "no_scale" else scale
        S = s * (tq @ tk.T)
        P = torch.softmax(S, dim=0 if mistake == "softmax_dim" else -1)
        if mistake == "no_softmax_grad":
            P = P.detach()
        O = (P.T if mistake == "transposed_p" else P) @ tv
        O.backward(torch.tensor(do_h.T.copy() if mistake == "transposed_do" and do_h.shape[0] == do_h.shape[1] else do_h))
        gq, gk, gv = (t.grad.numpy() if t.grad is not None else np.zeros(tuple(t.shape))
                      for t in (tq, tk, tv))
        if mistake == "swap_kv":
            return gq, gv, gk
        return gq, gk, gv
    return fn


MUTANTS = {
    "no_scale": _mutant(_head("no_scale")),
    "softmax_dim": _mutant(_head("softmax_dim")),
    "no_softmax_grad": _mutant(_head("no_softmax_grad")),
    "transposed_p": _mutant(_head("transposed_p")),
    "swap_kv": _mutant(_head("swap_kv")),
    "gqa_overwrite": _mutant(overwrite=True),
}


def _caught(ref):
    return not all(fd_pin(ref, *case) for case in FD_CASES)


def test_unmutated_copy_passes():
    assert not _caught(_mutant())


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name])
