"""Plant plausible mistakes in copies of the oracle and check a pin catches each.

Every mutant below is the plain definition with one deliberate error; the
pins of ``tests/oracle_pins.py`` must reject all of them, which shows they
can tell a wrong oracle from a right one.  (CPU only.)
"""
import math

import numpy as np
import pytest

from tests import oracle_pins as pins


def _make(score=None, softmax=None, combine=None, kvmap=None, lse_fn=None):
    def ref(q, k, v, scale):
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        O = np.zeros((B, Hq, N, d))
        L = np.zeros((B, Hq, N))
        for b in range(B):
            for h in range(Hq):
                g = kvmap(h, Hq, Hkv) if kvmap else h // (Hq // Hkv)
                S = score(q[b, h], k[b, g], scale) if score else scale * q[b, h] @ k[b, g].T
                m = S.max(-1, keepdims=True)
                E = np.exp(S - m)
                l = E.sum(-1, keepdims=True)
                P = softmax(S) if softmax else E / l
                O[b, h] = combine(P, v[b, g]) if combine else P @ v[b, g]
                L[b, h] = lse_fn(m, l)[:, 0] if lse_fn else (m + np.log(l))[:, 0]
        return O, L
    return ref


def _sm(fn):
    def softmax(S):
        return fn(np.asarray(S, dtype=np.float64))
    return softmax


MUTANTS = {
    "scale_ignored": _make(score=lambda q, k, s: q @ k.T),
    "scale_squared": _make(score=lambda q, k, s: s * s * (q @ k.T)),
    "score_sign": _make(score=lambda q, k, s: -s * (q @ k.T)),
    "score_transposed": _make(score=lambda q, k, s: s * (k @ q.T)),
    "last_key_dropped": _make(score=lambda q, k, s: np.concatenate(
        [s * (q @ k[:-1].T), np.full((q.shape[0], 1), -np.inf)], axis=1)),
    "kv_head_modulo": _make(kvmap=lambda h, Hq, Hkv: h % Hkv),
    "no_normalise": _make(softmax=lambda S: np.exp(S - S.max(-1, keepdims=True))),
    "no_max_subtracted": _make(softmax=lambda S: np.exp(S) / np.exp(S).sum(-1, keepdims=True)),
    "column_softmax": _make(softmax=lambda S: np.exp(S - S.max(0, keepdims=True)) /
                            np.exp(S - S.max(0, keepdims=True)).sum(0, keepdims=True)),
    "p_transposed": _make(combine=lambda P, v: P.T @ v),
    "lse_log2": _make(lse_fn=lambda m, l: m + np.log2(l)),
    "lse_without_max": _make(lse_fn=lambda m, l: np.log(l)),
    "lse_base2_max": _make(lse_fn=lambda m, l: m * math.log2(math.e) + np.log(l)),
}

SOFTMAX_MUTANTS = {
    "sm_no_max": _sm(lambda S: (np.exp(S) / np.exp(S).sum(-1, keepdims=True),
                                np.log(np.exp(S).sum(-1)))),
    "sm_no_normalise": _sm(lambda S: (np.exp(S - S.max(-1, keepdims=True)),
                                      S.max(-1) + np.log(np.exp(S - S.max(-1, keepdims=True)).sum(-1)))),
    "sm_lse_no_max": _sm(lambda S: (np.exp(S - S.max(-1, keepdims=True)) /
                                    np.exp(S - S.max(-1, keepdims=True)).sum(-1, keepdims=True),
                                    np.log(np.exp(S - S.max(-1, keepdims=True)).sum(-1)))),
}


def _caught(impl, pin_list):
    failed = []
    for pin in pin_list:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    return failed


def test_unmutated_copy_passes():
    assert _caught(_make(), pins.REF_PINS) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert _caught(MUTANTS[name], pins.REF_PINS), f"no pin catches mutant {name}"


@pytest.mark.parametrize("name", sorted(SOFTMAX_MUTANTS))
def test_softmax_mutant_is_caught(name):
    assert _caught(SOFTMAX_MUTANTS[name], pins.SOFTMAX_PINS), f"no pin catches {name}"
