"""The C-ABI library: it loads, exports every declared symbol, and rejects
bad arguments with the documented status before any HIP call (no GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")
LIB = os.path.join(ROOT, "exact_io_aware_73_amd", "libattn.so")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"ATTN_API\s+[\w\s\*]+?\b(attn_\w+)\s*\(", text)


def _status_codes():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"(ATTN_\w+)\s*=\s*(\d+)", text)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    l = ctypes.CDLL(LIB)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    l.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P]
    l.attn_fwd_f32.argtypes = [P, P, P, P, P, I, I, I, I, I, F, P]
    l.attn_fwd_materialized.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, P]
    l.attn_fwd_materialized_f32.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, F, P]
    l.attn_fwd_split.argtypes = [P, P, P, P, P, P, ctypes.c_ulonglong, I, I, I, I, I, I, F, P]
    l.attn_fwd_split_workspace_bytes.argtypes = [I, I, I, I, I]
    l.attn_fwd_split_workspace_bytes.restype = ctypes.c_ulonglong
    l.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, ctypes.c_ulonglong, I, I, I, I, I, F, P]
    l.attn_bwd_workspace_bytes.argtypes = [I, I, I]
    l.attn_bwd_workspace_bytes.restype = ctypes.c_ulonglong
    l.attn_fwd_fp8.argtypes = [P, P, P, P, P, F, F, F, I, I, I, I, I, F, P]
    l.attn_strerror.argtypes = [I]
    l.attn_strerror.restype = ctypes.c_char_p
    l.attn_fwd_plan.argtypes = [I, I, I, I, I, ctypes.POINTER(I)]
    l.attn_fwd_plan.restype = I
    return l


def test_header_declares_the_entry_points():
    assert set(_declared()) == {"attn_fwd", "attn_fwd_f32", "attn_fwd_materialized",
                                "attn_fwd_materialized_f32", "attn_fwd_split",
                                "attn_fwd_split_workspace_bytes", "attn_bwd",
                                "attn_bwd_workspace_bytes", "attn_bwd_noalloc",
                                "attn_bwd_noalloc_max_rows", "attn_fwd_fp8", "attn_device_info",
                                "attn_fwd_plan", "attn_strerror"}


def test_status_numbering_is_pinned():
    """The status values are part of the ABI: 0 - 7 as the boundary was
    specified (ATTN_ERR_HIP = 7), the three codes added with the alias check,
    the split-KV and the workspace arguments after them, then the fixed
    scratch buffer's limit.  The binding's
    constants carry the same values."""
    want = {"ATTN_OK": 0, "ATTN_ERR_NULL": 1, "ATTN_ERR_SHAPE": 2, "ATTN_ERR_GQA": 3,
            "ATTN_ERR_HEADDIM": 4, "ATTN_ERR_SCALE": 5, "ATTN_ERR_ALIGN": 6, "ATTN_ERR_HIP": 7,
            "ATTN_ERR_ALIAS": 8, "ATTN_ERR_SPLIT": 9, "ATTN_ERR_WORKSPACE": 10,
            "ATTN_ERR_SCRATCH": 11}
    assert _status_codes() == want
    src = open(os.path.join(ROOT, "exact_io_aware_73_amd", "attn.py")).read()
    m = re.findall(r"^(ATTN_[\w, ]+?)\s*=\s*([\d, ]+)$", src, re.M)
    got = {}
    for names, vals in m:
        for n, v in zip(names.split(","), vals.split(",")):
            got[n.strip()] = int(v)
    assert {k: got[k] for k in want} == want
    kern = {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define (ATTN_KERNEL_\w+) (\d+)", open(HEADER).read())}
    assert kern == {"ATTN_KERNEL_ROWS32": got["ATTN_KERNEL_ROWS32"],
                    "ATTN_KERNEL_ROWS64": got["ATTN_KERNEL_ROWS64"]}


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_strerror_names_every_code(lib):
    codes = _status_codes()
    assert codes["ATTN_OK"] == 0
    texts = {lib.attn_strerror(c).decode() for c in codes.values()}
    assert len(texts) == len(codes)          # a distinct message per code
    assert lib.attn_strerror(999) == b"unknown status"


# Fake, never-dereferenced device addresses, far apart so nothing overlaps.
# Every call below fails validation, which runs before any HIP call.
A = 1 << 40
Q, K, V, O, L, S, Pp = (A * (i + 1) for i in range(7))


def _fwd(lib, fn, q=Q, k=K, v=V, o=O, lse=L, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125):
    return getattr(lib, fn)(q, k, v, o, lse, B, Hq, Hkv, N, d, ctypes.c_float(scale), None)


def _mat(lib, fn, q=Q, k=K, v=V, o=O, lse=L, s=S, p=Pp, B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125):
    return getattr(lib, fn)(q, k, v, o, lse, s, p, B, Hq, Hkv, N, d, ctypes.c_float(scale), None)


FWD = ["attn_fwd", "attn_fwd_f32"]
MAT = ["attn_fwd_materialized", "attn_fwd_materialized_f32"]


@pytest.mark.parametrize("fn", FWD)
@pytest.mark.parametrize("kw,code", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(k=None), "ATTN_ERR_NULL"), (dict(v=None), "ATTN_ERR_NULL"),
    (dict(o=None), "ATTN_ERR_NULL"), (dict(lse=None), "ATTN_ERR_NULL"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(Hq=0), "ATTN_ERR_SHAPE"), (dict(Hkv=0), "ATTN_ERR_SHAPE"),
    (dict(N=0), "ATTN_ERR_SHAPE"), (dict(N=-5), "ATTN_ERR_SHAPE"),
    (dict(Hq=3, Hkv=2), "ATTN_ERR_GQA"),
    (dict(d=32), "ATTN_ERR_HEADDIM"), (dict(d=96), "ATTN_ERR_HEADDIM"), (dict(d=256), "ATTN_ERR_HEADDIM"),
    (dict(scale=math.inf), "ATTN_ERR_SCALE"), (dict(scale=-math.inf), "ATTN_ERR_SCALE"),
    (dict(scale=math.nan), "ATTN_ERR_SCALE"),
    (dict(q=Q + 8), "ATTN_ERR_ALIGN"), (dict(k=K + 4), "ATTN_ERR_ALIGN"), (dict(v=V + 2), "ATTN_ERR_ALIGN"),
    (dict(o=O + 8), "ATTN_ERR_ALIGN"), (dict(lse=L + 2), "ATTN_ERR_ALIGN"),
    (dict(o=Q), "ATTN_ERR_ALIAS"), (dict(o=K + 16), "ATTN_ERR_ALIAS"), (dict(lse=V + 64), "ATTN_ERR_ALIAS"),
    (dict(lse=O + 1024), "ATTN_ERR_ALIAS"),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, N=1 << 10), "ATTN_ERR_SHAPE"),
])
def test_fwd_rejects(lib, fn, kw, code):
    assert _fwd(lib, fn, **kw) == _status_codes()[code]


@pytest.mark.parametrize("fn", MAT)
@pytest.mark.parametrize("kw,code", [
    (dict(s=None), "ATTN_ERR_NULL"), (dict(p=None), "ATTN_ERR_NULL"), (dict(q=None), "ATTN_ERR_NULL"),
    (dict(s=S + 4), "ATTN_ERR_ALIGN"), (dict(p=Pp + 8), "ATTN_ERR_ALIGN"),
    (dict(s=Pp), "ATTN_ERR_ALIAS"), (dict(p=Q), "ATTN_ERR_ALIAS"), (dict(s=O), "ATTN_ERR_ALIAS"),
    (dict(Hq=4, Hkv=3), "ATTN_ERR_GQA"), (dict(d=80), "ATTN_ERR_HEADDIM"),
    (dict(scale=math.nan), "ATTN_ERR_SCALE"), (dict(N=0), "ATTN_ERR_SHAPE"),
    (dict(B=64, Hq=64, Hkv=64, N=1 << 14), "ATTN_ERR_SHAPE"),   # softmax grid too large
])
def test_materialized_rejects(lib, fn, kw, code):
    assert _mat(lib, fn, **kw) == _status_codes()[code]


@pytest.mark.parametrize("args,code", [
    ((0, 2, 1, 16, 64), "ATTN_ERR_SHAPE"), ((1, 2, 0, 16, 64), "ATTN_ERR_SHAPE"),
    ((1, 2, 1, 0, 128), "ATTN_ERR_SHAPE"), ((1, 3, 2, 16, 64), "ATTN_ERR_GQA"),
    ((1, 2, 1, 16, 96), "ATTN_ERR_HEADDIM"), ((1 << 20, 1 << 10, 1 << 10, 1 << 10, 64), "ATTN_ERR_SHAPE"),
])
def test_plan_rejects(lib, args, code):
    """attn_fwd_plan checks its sizes as attn_fwd does, before any HIP call."""
    out = ctypes.c_int(-1)
    assert lib.attn_fwd_plan(*args, ctypes.byref(out)) == _status_codes()[code]
    assert out.value == -1
    assert lib.attn_fwd_plan(1, 2, 1, 16, 64, None) == _status_codes()["ATTN_ERR_NULL"]


def test_python_binding_signatures_match_header():
    """The binding's entry points carry the C names declared in the header."""
    src = open(os.path.join(ROOT, "exact_io_aware_73_amd", "attn.py")).read()
    for name in _declared():
        assert re.search(rf"^def {name}\(", src, re.M), name


# ---------------------------------------------------------------------------
# split-KV entry point
W = A * 9     # fake workspace address, apart from the others


def _split(lib, q=Q, k=K, v=V, o=O, lse=L, ws=W, ws_bytes=1 << 40, n_split=4, B=1, Hq=2, Hkv=1,
           N=16, d=64, scale=0.125):
    return lib.attn_fwd_split(q, k, v, o, lse, ws, ws_bytes, n_split, B, Hq, Hkv, N, d,
                              ctypes.c_float(scale), None)


@pytest.mark.parametrize("B,Hq,N,d,S", [(1, 1, 1, 64, 1), (2, 8, 1000, 128, 4), (1, 1, 32768, 128, 64),
                                         (3, 5, 17, 64, 7)])
def test_split_workspace_bytes(lib, B, Hq, N, d, S):
    assert lib.attn_fwd_split_workspace_bytes(B, Hq, N, d, S) == S * B * Hq * N * (d + 1) * 4


@pytest.mark.parametrize("args", [(0, 1, 16, 64, 2), (1, 0, 16, 64, 2), (1, 1, 0, 64, 2),
                                  (1, 1, 16, 96, 2), (1, 1, 16, 64, 0), (1, 1, 16, 64, 65)])
def test_split_workspace_bytes_rejects(lib, args):
    assert lib.attn_fwd_split_workspace_bytes(*args) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(n_split=0), "ATTN_ERR_SPLIT"), (dict(n_split=65), "ATTN_ERR_SPLIT"),
    (dict(n_split=-1), "ATTN_ERR_SPLIT"),
    (dict(ws=None), "ATTN_ERR_WORKSPACE"), (dict(ws=W + 8), "ATTN_ERR_WORKSPACE"),
    (dict(ws_bytes=4 * 2 * 16 * 65 * 4 - 1), "ATTN_ERR_WORKSPACE"),
    (dict(ws=Q), "ATTN_ERR_ALIAS"), (dict(ws=O - 64), "ATTN_ERR_ALIAS"), (dict(ws=L), "ATTN_ERR_ALIAS"),
    (dict(q=None), "ATTN_ERR_NULL"), (dict(o=None), "ATTN_ERR_NULL"),
    (dict(Hq=3, Hkv=2), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEADDIM"),
    (dict(scale=math.nan), "ATTN_ERR_SCALE"), (dict(N=0), "ATTN_ERR_SHAPE"),
    (dict(o=Q), "ATTN_ERR_ALIAS"), (dict(q=Q + 8), "ATTN_ERR_ALIGN"),
])
def test_split_rejects(lib, kw, code):
    assert _split(lib, **kw) == _status_codes()[code]


# ---------------------------------------------------------------------------
# backward entry point
DO_, DQ_, DK_, DV_, WB = (A * (i + 10) for i in range(5))


def _bwd(lib, q=Q, k=K, v=V, o=O, lse=L, do=DO_, dq=DQ_, dk=DK_, dv=DV_, ws=WB, ws_bytes=1 << 40,
         B=1, Hq=2, Hkv=1, N=16, d=64, scale=0.125):
    return lib.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, N, d,
                        ctypes.c_float(scale), None)


def _bwd_noalloc(lib, q=Q, k=K, v=V, o=O, lse=L, do=DO_, dq=DQ_, dk=DK_, dv=DV_, B=1, Hq=2, Hkv=1,
                N=16, d=64, scale=0.125):
    return lib.attn_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, N, d,
                                ctypes.c_float(scale), None)


def test_bwd_noalloc_limit(lib):
    lib.attn_bwd_noalloc_max_rows.restype = ctypes.c_ulonglong
    assert lib.attn_bwd_noalloc_max_rows() == (16 << 20) // 4


@pytest.mark.parametrize("kw,code", [
    (dict(N=(16 << 20) // 4 + 1, Hq=1), "ATTN_ERR_SCRATCH"),
    (dict(B=2, Hq=8, Hkv=8, N=(16 << 20) // 64 + 1), "ATTN_ERR_SCRATCH"),
    (dict(do=None), "ATTN_ERR_NULL"), (dict(dq=None), "ATTN_ERR_NULL"), (dict(lse=None), "ATTN_ERR_NULL"),
    (dict(dk=DK_ + 2), "ATTN_ERR_ALIGN"), (dict(dq=Q), "ATTN_ERR_ALIAS"), (dict(dv=DK_ + 64), "ATTN_ERR_ALIAS"),
    (dict(Hq=3, Hkv=2), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEADDIM"), (dict(N=0), "ATTN_ERR_SHAPE"),
    (dict(scale=math.nan), "ATTN_ERR_SCALE"),
])
def test_bwd_noalloc_rejects(lib, kw, code):
    lib.attn_bwd_noalloc.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 5 + [ctypes.c_float,
                                                                                   ctypes.c_void_p]
    assert _bwd_noalloc(lib, **kw) == _status_codes()[code]


def test_bwd_workspace_bytes(lib):
    assert lib.attn_bwd_workspace_bytes(2, 8, 1000) == 2 * 8 * 1000 * 4
    assert lib.attn_bwd_workspace_bytes(0, 8, 1000) == 0
    assert lib.attn_bwd_workspace_bytes(1, 1, 0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), "ATTN_ERR_NULL"), (dict(dq=None), "ATTN_ERR_NULL"), (dict(dk=None), "ATTN_ERR_NULL"),
    (dict(dv=None), "ATTN_ERR_NULL"), (dict(o=None), "ATTN_ERR_NULL"), (dict(lse=None), "ATTN_ERR_NULL"),
    (dict(ws=None), "ATTN_ERR_WORKSPACE"), (dict(ws=WB + 4), "ATTN_ERR_WORKSPACE"),
    (dict(ws_bytes=2 * 16 * 4 - 1), "ATTN_ERR_WORKSPACE"),
    (dict(do=DO_ + 8), "ATTN_ERR_ALIGN"), (dict(dk=DK_ + 2), "ATTN_ERR_ALIGN"),
    (dict(dq=Q), "ATTN_ERR_ALIAS"), (dict(dk=V + 32), "ATTN_ERR_ALIAS"), (dict(dv=DO_), "ATTN_ERR_ALIAS"),
    (dict(dv=DK_ + 64), "ATTN_ERR_ALIAS"), (dict(ws=DQ_), "ATTN_ERR_ALIAS"), (dict(dq=L), "ATTN_ERR_ALIAS"),
    (dict(Hq=3, Hkv=2), "ATTN_ERR_GQA"), (dict(d=32), "ATTN_ERR_HEADDIM"), (dict(N=0), "ATTN_ERR_SHAPE"),
    (dict(scale=math.inf), "ATTN_ERR_SCALE"),
])
def test_bwd_rejects(lib, kw, code):
    assert _bwd(lib, **kw) == _status_codes()[code]


# ---------------------------------------------------------------------------
# 8-bit entry point (host-side checks only: every case is rejected before any
# HIP call).  Inputs: q8 / k8 1 byte per element, vt8 [B, Hkv, d, Np].
Q8, K8, VT8, O8, L8 = (A * (i + 20) for i in range(5))


def _fp8(lib, q=Q8, k=K8, vt=VT8, o=O8, lse=L8, qs=0.5, ks=0.5, vs=0.25, B=1, Hq=2, Hkv=1, N=17,
         d=128, scale=0.125):
    return lib.attn_fwd_fp8(q, k, vt, o, lse, ctypes.c_float(qs), ctypes.c_float(ks),
                            ctypes.c_float(vs), B, Hq, Hkv, N, d, ctypes.c_float(scale), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), "ATTN_ERR_NULL"), (dict(vt=None), "ATTN_ERR_NULL"), (dict(lse=None), "ATTN_ERR_NULL"),
    (dict(Hq=3, Hkv=2), "ATTN_ERR_GQA"), (dict(d=96), "ATTN_ERR_HEADDIM"), (dict(N=0), "ATTN_ERR_SHAPE"),
    (dict(B=0), "ATTN_ERR_SHAPE"), (dict(scale=math.nan), "ATTN_ERR_SCALE"),
    (dict(qs=math.inf), "ATTN_ERR_SCALE"), (dict(vs=math.nan), "ATTN_ERR_SCALE"),
    (dict(qs=3e38, ks=3e38), "ATTN_ERR_SCALE"),        # the combined multiplier overflows
    (dict(N=1 << 24), "ATTN_ERR_SHAPE"),               # d * Np reaches 2^31
    (dict(vt=VT8 + 8), "ATTN_ERR_ALIGN"), (dict(o=O8 + 2), "ATTN_ERR_ALIGN"),
    (dict(lse=L8 + 2), "ATTN_ERR_ALIGN"),
    (dict(o=Q8), "ATTN_ERR_ALIAS"), (dict(o=VT8 + 128 * 32 - 16), "ATTN_ERR_ALIAS"),
    (dict(lse=K8 + 16), "ATTN_ERR_ALIAS"), (dict(lse=O8 + 64), "ATTN_ERR_ALIAS"),
])
def test_fp8_rejects(lib, kw, code):
    assert _fp8(lib, **kw) == _status_codes()[code]
