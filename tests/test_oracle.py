"""The CPU oracle against its pins (no GPU)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as pins


def _ref(q, k, v, scale):
    return oracle.attention_ref(q, k, v, scale)


@pytest.mark.parametrize("pin", pins.REF_PINS, ids=lambda f: f.__name__)
def test_ref_pin(pin):
    pin(_ref)


@pytest.mark.parametrize("pin", pins.SOFTMAX_PINS, ids=lambda f: f.__name__)
def test_softmax_pin(pin):
    pin(oracle.softmax_rows)


def test_threaded_equals_serial():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 4, 70, 8))
    k = rng.standard_normal((2, 2, 70, 8))
    v = rng.standard_normal((2, 2, 70, 8))
    O1, l1 = oracle.attention_ref(q, k, v, 0.3)
    O2, l2 = oracle.attention_ref(q, k, v, 0.3, workers=4)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2)


def test_row_chunking_equals_whole(monkeypatch):
    """Chunks of whole rows give the same result as one block."""
    from oracle import attention as A
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal((1, 1, 50, 4)) for _ in range(3))
    O1, l1 = A.attention_ref(q, k, v, 0.5)
    monkeypatch.setattr(A, "_CHUNK_BYTES", 8 * 50 * 3)   # 3 rows per chunk
    O2, l2 = A.attention_ref(q, k, v, 0.5)
    assert np.max(np.abs(O1 - O2)) <= 1e-15 and np.max(np.abs(l1 - l2)) <= 1e-15


def test_rows_subset_matches_full():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((2, 4, 40, 8))
    k = rng.standard_normal((2, 2, 40, 8))
    v = rng.standard_normal((2, 2, 40, 8))
    O, l = oracle.attention_ref(q, k, v, 0.4)
    rows = [0, 7, 39]
    Or, lr = oracle.attention_ref_rows(q, k, v, 1, 3, rows, 0.4)
    assert np.max(np.abs(Or - O[1, 3, rows])) <= 1e-15
    assert np.max(np.abs(lr - l[1, 3, rows])) <= 1e-15


def test_sp_variant_consistent():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 4, 30, 8))
    k = rng.standard_normal((1, 2, 30, 8))
    v = rng.standard_normal((1, 2, 30, 8))
    O, l = oracle.attention_ref(q, k, v, 0.4)
    O2, l2, S, P = oracle.attention_ref_sp(q, k, v, 0.4)
    assert np.max(np.abs(O - O2)) <= 1e-14 and np.max(np.abs(l - l2)) <= 1e-14
    # S is the scaled score matrix and P its row softmax
    assert np.max(np.abs(S[0, 3] - 0.4 * q[0, 3] @ k[0, 1].T)) <= 1e-14
    assert np.max(np.abs(P.sum(-1) - 1)) <= 1e-12


def test_rejects_bad_gqa():
    q = np.zeros((1, 3, 4, 2)); k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention_ref(q, k, k, 1.0)
