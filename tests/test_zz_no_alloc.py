"""attn_bwd_noalloc (through the C ABI): the backward with no workspace
argument, its row sums in the library's fixed scratch buffer, against
attn_bwd with a caller workspace on the same inputs -- two calls in a row,
the second on a smaller problem, each bit-identical to attn_bwd; and the
size limit, rejected before any HIP call."""
import ctypes
import math

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def attn():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    from exact_io_aware_73_amd import attn as a
    return a


def _case(attn, B, Hq, Hkv, N, d, seed):
    q, k, v = (t.cuda() for t in workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed))
    do = workloads.random_inputs(B, Hq, Hkv, N, d, torch.bfloat16, seed + 7)[0].cuda()
    scale = 1 / math.sqrt(d)
    o, lse = attn.fwd(q, k, v, scale)
    ref = attn.bwd(q, k, v, o, lse, do, scale)
    got = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")),
           torch.full_like(v, float("nan")))
    attn.attn_bwd_noalloc(q, k, v, o, lse, do, *got, scale)
    torch.cuda.synchronize()
    for name, r, g in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(r, g), (name, (B, Hq, Hkv, N, d))


@pytest.mark.parametrize("d", [64, 128])
def test_noalloc_matches_workspace_entry_two_calls(attn, d):
    # the first call fills more of the scratch buffer than the second uses
    _case(attn, 2, 8, 2, 1000, d, seed=50 + d)
    _case(attn, 1, 4, 1, 77, d, seed=60 + d)


def test_noalloc_largest_accepted_size(attn):
    rows = attn.attn_bwd_noalloc_max_rows()
    assert rows == (16 << 20) // 4
    _case(attn, 1, rows // 16384, rows // 16384, 16384, 64, seed=70)   # exactly the limit
    _case(attn, 1, 2, 1, 129, 128, seed=71)


def test_noalloc_rejects_beyond_the_limit(attn):
    rows = attn.attn_bwd_noalloc_max_rows()
    lib = ctypes.CDLL(attn.LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, P]
    A = 1 << 40
    ptrs = [A * (i + 1) for i in range(9)]   # never dereferenced: the size check comes first
    st = lib.attn_bwd_noalloc(*ptrs, 1, 1, 1, rows + 1, 64, F(0.125), None)
    assert st == attn.ATTN_ERR_SCRATCH
    with pytest.raises(ValueError):
        q = torch.zeros(1, 1, rows + 1, 64, dtype=torch.bfloat16, device="cuda")
        o, lse = torch.zeros_like(q), torch.zeros(1, 1, rows + 1, device="cuda")
        attn.attn_bwd_noalloc(q, q, q, o, lse, q, torch.empty_like(q), torch.empty_like(q),
                              torch.empty_like(q), 0.125)
