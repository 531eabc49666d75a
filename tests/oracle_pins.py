"""Pins for the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes an implementation and raises AssertionError if it
disagrees with a fact that does not come from the implementation itself:

* ``ref(q, k, v, scale) -> (O, lse)`` with q [B,Hq,N,d], k/v [B,Hkv,N,d]
  float64 arrays;
* ``softmax(S) -> (P, lse)`` for a score block [..., n].

``tests/test_oracle.py`` runs every pin on the real oracle;
``tests/test_oracle_mutants.py`` plants plausible mistakes in copies of the
oracle and checks that some pin catches each one.
"""
from __future__ import annotations

import math

import numpy as np
import torch

RNG = np.random.default_rng(12345)


def _rand(*shape, rng=None, std=1.0):
    rng = RNG if rng is None else rng
    return rng.standard_normal(shape) * std


# --- (1) rows of P are probability vectors -------------------------------
def pin_rows_stochastic(softmax):
    """P >= 0 and each row sums to 1 (aiknowledge.cn "1.1 ...", section 1.1.8:
    each row is normalised by its own exp-sum).  Scores up to +-1000 also
    check that the maximum is subtracted before exp (no overflow)."""
    rng = np.random.default_rng(1)
    for scale in (1.0, 30.0, 1000.0):
        S = rng.standard_normal((3, 7, 33)) * scale
        P, lse = softmax(S)
        assert np.all(np.isfinite(P)) and np.all(np.isfinite(lse))
        assert np.all(P >= 0.0)
        assert np.max(np.abs(P.sum(-1) - 1.0)) <= 1e-12


# --- (2) shift invariance on the scores ----------------------------------
def pin_shift_scores(softmax):
    """Adding c_i to every score of row i leaves P unchanged and adds c_i to
    lse (course chapter "efficient attention": subtracting one number from
    all scores leaves softmax unchanged; the basis of the rescale)."""
    rng = np.random.default_rng(2)
    S = rng.standard_normal((5, 40)) * 3
    c = rng.standard_normal((5, 1)) * 50
    P0, l0 = softmax(S)
    P1, l1 = softmax(S + c)
    assert np.max(np.abs(P0 - P1)) <= 1e-12
    assert np.max(np.abs((l1 - l0) - c[:, 0])) <= 1e-9


# --- (3) shift invariance through K --------------------------------------
def pin_shift_keys(ref):
    """K' = K + 1 u^T adds scale * q_i . u to every score of row i, so O is
    unchanged and lse grows by scale * q_i . u."""
    rng = np.random.default_rng(3)
    B, Hq, Hkv, N, d = 1, 2, 1, 37, 8
    q, k, v = _rand(B, Hq, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng)
    u = rng.standard_normal(d) * 2
    scale = 0.3
    O0, l0 = ref(q, k, v, scale)
    O1, l1 = ref(q, k + u, v, scale)
    assert np.max(np.abs(O0 - O1)) <= 1e-11
    shift = scale * (q @ u)                      # [B, Hq, N]
    assert np.max(np.abs((l1 - l0) - shift)) <= 1e-10


# --- (4) constant V -------------------------------------------------------
def pin_constant_v(ref):
    """V_j = v for every key => O_i = v (the weights of a row sum to 1)."""
    rng = np.random.default_rng(4)
    B, Hq, Hkv, N, d = 2, 4, 2, 29, 6
    q, k = _rand(B, Hq, N, d, rng=rng, std=2), _rand(B, Hkv, N, d, rng=rng, std=2)
    vrow = rng.standard_normal((B, Hkv, 1, d))
    v = np.broadcast_to(vrow, (B, Hkv, N, d)).copy()
    O, _ = ref(q, k, v, 0.7)
    expect = np.repeat(vrow, Hq // Hkv, axis=1)
    assert np.max(np.abs(O - expect)) <= 1e-12


# --- (5) a dominant score selects its V row ------------------------------
def pin_one_hot(ref):
    """If S[i, j*] exceeds every other score of row i by Delta, then
    |O_i - V_j*| <= 2 (N - 1) exp(-Delta) max|V|.  Scores near 1000 also
    require the row maximum to be subtracted before exp."""
    rng = np.random.default_rng(5)
    N, d = 16, 4
    k = rng.uniform(-0.5, 0.5, size=(1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    q = np.zeros((1, 1, N, d))
    for c in range(d):
        k[0, 0, c, :] = 0.0
        k[0, 0, c, c] = 26.0                    # key c wins for queries along e_c
    for i in range(N):
        q[0, 0, i, i % d] = 40.0                # winner score 40 * 26 = 1040
    O, lse = ref(q, k, v, 1.0)
    # every other score is at most 40 * 0.5 = 20, so Delta >= 1020
    for i in range(N):
        assert np.max(np.abs(O[0, 0, i] - v[0, 0, i % d])) <= 1e-12
        assert abs(lse[0, 0, i] - 1040.0) <= 1e-9


# --- (6) brute force on tiny inputs --------------------------------------
def brute_force(q, k, v, scale):
    """Pure-Python loops with math.exp / math.fsum; query head h reads K/V
    head (h * Hkv) // Hq, which is the contiguous-group rule written another
    way."""
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    O = np.zeros((B, Hq, N, d))
    lse = np.zeros((B, Hq, N))
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            for i in range(N):
                s = [scale * math.fsum(float(q[b, h, i, c]) * float(k[b, g, j, c]) for c in range(d))
                     for j in range(N)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = math.fsum(e)
                for c in range(d):
                    O[b, h, i, c] = math.fsum(e[j] * float(v[b, g, j, c]) for j in range(N)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return O, lse


def pin_brute(ref):
    rng = np.random.default_rng(6)
    for (B, Hq, Hkv, N, d) in [(1, 1, 1, 1, 1), (1, 1, 1, 5, 3), (2, 2, 1, 8, 4),
                               (1, 4, 2, 7, 4), (1, 3, 3, 6, 2)]:
        q, k, v = _rand(B, Hq, N, d, rng=rng, std=1.5), _rand(B, Hkv, N, d, rng=rng, std=1.5), _rand(B, Hkv, N, d, rng=rng)
        scale = float(rng.uniform(0.2, 1.5))
        O, lse = ref(q, k, v, scale)
        Ob, lb = brute_force(q, k, v, scale)
        assert np.max(np.abs(O - Ob)) <= 1e-12, (B, Hq, Hkv, N, d)
        assert np.max(np.abs(lse - lb)) <= 1e-12, (B, Hq, Hkv, N, d)


# --- (7) closed forms -----------------------------------------------------
def pin_closed_forms(ref):
    rng = np.random.default_rng(7)
    d = 5
    # N = 1: O = V_0, lse = scale * q . k_0
    q, k, v = _rand(1, 2, 1, d, rng=rng), _rand(1, 1, 1, d, rng=rng), _rand(1, 1, 1, d, rng=rng)
    O, lse = ref(q, k, v, 0.8)
    assert np.max(np.abs(O - v)) <= 1e-12
    assert np.max(np.abs(lse[0, :, 0] - 0.8 * (q[0, :, 0] @ k[0, 0, 0]))) <= 1e-12
    # N = 2: O = sigma(s0 - s1) V0 + sigma(s1 - s0) V1, lse = logaddexp(s0, s1)
    q, k, v = _rand(1, 1, 2, d, rng=rng), _rand(1, 1, 2, d, rng=rng), _rand(1, 1, 2, d, rng=rng)
    O, lse = ref(q, k, v, 0.6)
    for i in range(2):
        s0 = 0.6 * float(q[0, 0, i] @ k[0, 0, 0])
        s1 = 0.6 * float(q[0, 0, i] @ k[0, 0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        assert np.max(np.abs(O[0, 0, i] - (w0 * v[0, 0, 0] + w1 * v[0, 0, 1]))) <= 1e-12
        assert abs(lse[0, 0, i] - np.logaddexp(s0, s1)) <= 1e-12
    # scale = 0: uniform weights, O_i = mean_j V_j, lse = ln N
    N = 23
    q, k, v = _rand(1, 2, N, d, rng=rng), _rand(1, 1, N, d, rng=rng), _rand(1, 1, N, d, rng=rng)
    O, lse = ref(q, k, v, 0.0)
    assert np.max(np.abs(O - v.mean(axis=2, keepdims=True))) <= 1e-12
    assert np.max(np.abs(lse - math.log(N))) <= 1e-12


# --- (8) the pages' online softmax, run by hand, equals the full softmax -
def online_softmax_blocks(s, vals, blocks):
    """The recurrences of the blog "attention 的显存线性化", section 三
    (running max m and exp-sum l per row), with the accumulator rescaled by
    exp(m_old - m_new) whenever the max grows (course chapter "efficient
    attention", online-softmax paragraph) and divided by l once at the end.
    ``s``: one row of scores; ``vals``: [n, d]; ``blocks``: list of index
    ranges covering the row in order."""
    m = -math.inf
    l = 0.0
    acc = np.zeros(vals.shape[1])
    for lo, hi in blocks:
        blk = s[lo:hi]
        m_new = max(m, max(blk))
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        e = np.array([math.exp(x - m_new) for x in blk])
        l = alpha * l + math.fsum(e)
        acc = alpha * acc + e @ vals[lo:hi]
        m = m_new
    return acc / l, m + math.log(l)


def pin_two_block_example(ref):
    """One row of scores [1, 3 | 2, 5] in two blocks with values [1, 2, 3, 4]:
    the hand-run recurrence and the oracle's full softmax must agree.  The
    scores are fed as q = 1, k_j = s_j, d = 1, scale = 1."""
    s = [1.0, 3.0, 2.0, 5.0]
    vals = np.array([[1.0], [2.0], [3.0], [4.0]])
    o_online, lse_online = online_softmax_blocks(s, vals, [(0, 2), (2, 4)])
    # the same quantities from the definition, in exact-sum arithmetic
    e = [math.exp(x) for x in s]
    o_def = math.fsum(ei * vi for ei, vi in zip(e, [1, 2, 3, 4])) / math.fsum(e)
    lse_def = math.log(math.fsum(e))
    assert abs(o_online[0] - o_def) <= 1e-14 and abs(lse_online - lse_def) <= 1e-14
    q = np.ones((1, 1, 1, 1))
    k = np.array(s).reshape(1, 1, 4, 1)
    v = vals.reshape(1, 1, 4, 1)
    O, lse = ref(np.repeat(q, 4, axis=2), k, v, 1.0)
    assert abs(O[0, 0, 0, 0] - o_def) <= 1e-14
    assert abs(lse[0, 0, 0] - lse_def) <= 1e-14


def pin_random_partitions(ref, n_cases: int = 25):
    """Any split of a row into consecutive blocks gives the full result."""
    rng = np.random.default_rng(8)
    for _ in range(n_cases):
        N = int(rng.integers(1, 60))
        d = int(rng.integers(1, 6))
        q = rng.standard_normal((1, 1, 1, d)) * 3
        k = rng.standard_normal((1, 1, N, d)) * 3
        v = rng.standard_normal((1, 1, N, d))
        cuts = sorted(set(rng.integers(1, N, size=int(rng.integers(0, 5))).tolist())) if N > 1 else []
        edges = [0] + cuts + [N]
        blocks = list(zip(edges[:-1], edges[1:]))
        s = [float(x) for x in (0.9 * (k[0, 0] @ q[0, 0, 0]))]
        o_on, lse_on = online_softmax_blocks(s, v[0, 0], blocks)
        O, lse = ref(np.repeat(q, N, axis=2), k, v, 0.9)
        assert np.max(np.abs(O[0, 0, 0] - o_on)) <= 1e-12
        assert abs(lse[0, 0, 0] - lse_on) <= 1e-12


# --- (9) GQA equals MHA with each K/V head repeated ----------------------
def pin_gqa_repeat(ref):
    """Several query heads sharing one K/V head (course chapter "efficient
    attention", class 3) equals ordinary multi-head attention on K/V with
    each head repeated Hq/Hkv times in place."""
    rng = np.random.default_rng(9)
    B, Hq, Hkv, N, d = 2, 8, 2, 19, 4
    q, k, v = _rand(B, Hq, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng)
    O, lse = ref(q, k, v, 0.5)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    O2, lse2 = ref(q, kr, vr, 0.5)
    assert np.max(np.abs(O - O2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13


# --- (10) an independent library implementation --------------------------
def pin_torch_sdpa(ref):
    """torch.nn.functional.scaled_dot_product_attention on the CPU in float64
    (the route the "efficient attention" chapter's cost table names), with
    enable_gqa for shared K/V heads."""
    rng = np.random.default_rng(10)
    for (B, Hq, Hkv, N, d, scale) in [(2, 4, 4, 64, 16, None), (1, 8, 2, 200, 32, 0.2),
                                      (1, 4, 1, 1024, 64, None), (2, 6, 3, 33, 8, -0.4)]:
        q, k, v = _rand(B, Hq, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng), _rand(B, Hkv, N, d, rng=rng)
        sc = 1.0 / math.sqrt(d) if scale is None else scale
        O, _ = ref(q, k, v, sc)
        Ot = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
            scale=sc, enable_gqa=(Hq != Hkv)).numpy()
        assert np.max(np.abs(O - Ot)) <= 1e-10, (B, Hq, Hkv, N, d)


REF_PINS = [pin_shift_keys, pin_constant_v, pin_one_hot, pin_brute, pin_closed_forms,
            pin_two_block_example, pin_random_partitions, pin_gqa_repeat, pin_torch_sdpa]
SOFTMAX_PINS = [pin_rows_stochastic, pin_shift_scores]
