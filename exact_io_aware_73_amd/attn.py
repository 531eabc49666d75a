"""Thin ctypes binding over libattn.so (include/attn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory and the stream.
There is no fallback: if the library is missing this module fails to import.

Entry points carry the C names and take tensors instead of raw pointers:

    attn_fwd(q, k, v, o, lse, scale, stream=None)                 bf16
    attn_fwd_f32(q, k, v, o, lse, scale, stream=None)             fp32
    attn_fwd_materialized(q, k, v, o, lse, s, p, scale, stream=None)
    attn_fwd_materialized_f32(q, k, v, o, lse, s, p, scale, stream=None)
    attn_fwd_split(q, k, v, o, lse, workspace, n_split, scale, stream=None)   bf16
    attn_fwd_split_workspace_bytes(B, Hq, N, d, n_split)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, stream=None)   bf16
    attn_bwd_workspace_bytes(B, Hq, N)
    attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale, stream=None)   bf16, no workspace
    attn_bwd_noalloc_max_rows()
    attn_fwd_fp8(q8, k8, vt8, o, lse, q_scale, k_scale, v_scale, scale, stream=None)
    attn_device_info(device=None) -> (compute units, XCDs, L2 bytes)
    attn_fwd_plan(B, Hq, Hkv, N, d, device=None) -> ATTN_KERNEL_ROWS32 / _ROWS64
    attn_strerror(status)

plus ``fwd`` / ``fwd_materialized`` / ``fwd_split`` / ``bwd``, which allocate
the outputs (and the workspaces) and pick the
entry point by dtype.  q: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; contiguous
CUDA (HIP) tensors.  Argument errors raise ValueError, launch errors
RuntimeError.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m exact_io_aware_73_amd.build` "
        "(or __graft_entry__.build()) first.  There is no fallback path.")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_lib.attn_fwd.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_fwd_f32.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_fwd_materialized.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_fwd_materialized_f32.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
for _fn in ("attn_fwd", "attn_fwd_f32", "attn_fwd_materialized", "attn_fwd_materialized_f32"):
    getattr(_lib, _fn).restype = _I
_U64 = ctypes.c_ulonglong
_lib.attn_fwd_split.argtypes = [_P, _P, _P, _P, _P, _P, _U64, _I, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_fwd_split.restype = _I
_lib.attn_fwd_split_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
_lib.attn_fwd_split_workspace_bytes.restype = _U64
_lib.attn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _U64, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_bwd.restype = _I
_lib.attn_bwd_workspace_bytes.argtypes = [_I, _I, _I]
_lib.attn_bwd_workspace_bytes.restype = _U64
_lib.attn_fwd_fp8.argtypes = [_P, _P, _P, _P, _P, _F, _F, _F, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_fwd_fp8.restype = _I
_lib.attn_strerror.argtypes = [_I]
_lib.attn_strerror.restype = ctypes.c_char_p

_lib.attn_bwd_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]
_lib.attn_bwd_noalloc.restype = _I
_lib.attn_bwd_noalloc_max_rows.argtypes = []
_lib.attn_bwd_noalloc_max_rows.restype = _U64
_lib.attn_device_info.argtypes = [ctypes.POINTER(_I), ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.attn_device_info.restype = _I
_lib.attn_fwd_plan.argtypes = [_I, _I, _I, _I, _I, ctypes.POINTER(_I)]
_lib.attn_fwd_plan.restype = _I

ATTN_OK, ATTN_ERR_NULL, ATTN_ERR_SHAPE, ATTN_ERR_GQA, ATTN_ERR_HEADDIM = 0, 1, 2, 3, 4
ATTN_ERR_SCALE, ATTN_ERR_ALIGN, ATTN_ERR_HIP, ATTN_ERR_ALIAS = 5, 6, 7, 8
ATTN_ERR_SPLIT, ATTN_ERR_WORKSPACE, ATTN_ERR_SCRATCH = 9, 10, 11
ATTN_MAX_SPLIT = 64
ATTN_KERNEL_ROWS32, ATTN_KERNEL_ROWS64 = 1, 2


def attn_strerror(status: int) -> str:
    return _lib.attn_strerror(int(status)).decode()


def _raise(status: int, fn: str):
    if status == ATTN_OK:
        return
    msg = f"{fn}: {attn_strerror(status)} (status {status})"
    if status == ATTN_ERR_HIP:
        raise RuntimeError(msg)
    raise ValueError(msg)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream))


def _dims(q, k, v):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError(f"k, v must be [B, Hkv, N, d] matching q {tuple(q.shape)}; "
                         f"got {tuple(k.shape)} and {tuple(v.shape)}")
    if q.device != k.device or q.device != v.device:
        raise ValueError("q, k, v must be on one device")
    return B, Hq, k.shape[1], N, d


def _call(fn_name, dtype, q, k, v, o, lse, s, p, scale, stream):
    B, Hq, Hkv, N, d = _dims(q, k, v)
    for name, t, dt in (("q", q, dtype), ("k", k, dtype), ("v", v, dtype), ("o", o, dtype),
                        ("lse", lse, torch.float32), ("s", s, torch.float32), ("p", p, dtype)):
        if t is None:
            continue
        if t.dtype != dt:
            raise ValueError(f"{fn_name}: {name} must be {dt}, got {t.dtype}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be contiguous on {q.device}")
    if o.shape != q.shape or lse.shape != (B, Hq, N):
        raise ValueError(f"{fn_name}: o must be {tuple(q.shape)} and lse {(B, Hq, N)}")
    for name, t in (("s", s), ("p", p)):
        if t is not None and t.shape != (B, Hq, N, N):
            raise ValueError(f"{fn_name}: {name} must be {(B, Hq, N, N)}")
    fn = getattr(_lib, fn_name)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse)]
    if fn_name.startswith("attn_fwd_materialized"):
        args += [_ptr(s), _ptr(p)]
    with torch.cuda.device(q.device):
        st = fn(*args, B, Hq, Hkv, N, d, ctypes.c_float(float(scale)),
                _stream_handle(stream, q.device))
    _raise(st, fn_name)


def attn_fwd(q, k, v, o, lse, scale, stream=None):
    """Fused tiled forward, bf16 I/O (C: attn_fwd)."""
    _call("attn_fwd", torch.bfloat16, q, k, v, o, lse, None, None, scale, stream)


def attn_fwd_f32(q, k, v, o, lse, scale, stream=None):
    """Fused tiled forward, fp32 I/O (C: attn_fwd_f32)."""
    _call("attn_fwd_f32", torch.float32, q, k, v, o, lse, None, None, scale, stream)


def attn_fwd_materialized(q, k, v, o, lse, s, p, scale, stream=None):
    """Three-kernel path that writes S (fp32) and P (bf16) (C: attn_fwd_materialized)."""
    _call("attn_fwd_materialized", torch.bfloat16, q, k, v, o, lse, s, p, scale, stream)


def attn_fwd_materialized_f32(q, k, v, o, lse, s, p, scale, stream=None):
    """Three-kernel path, fp32 throughout (C: attn_fwd_materialized_f32)."""
    _call("attn_fwd_materialized_f32", torch.float32, q, k, v, o, lse, s, p, scale, stream)


def attn_fwd_split_workspace_bytes(B, Hq, N, d, n_split) -> int:
    """Workspace bytes attn_fwd_split needs (0 for arguments it would reject)."""
    return int(_lib.attn_fwd_split_workspace_bytes(int(B), int(Hq), int(N), int(d), int(n_split)))


def attn_fwd_split(q, k, v, o, lse, workspace, n_split, scale, stream=None):
    """Split-KV forward, bf16 I/O (C: attn_fwd_split); workspace: a contiguous
    device tensor of at least attn_fwd_split_workspace_bytes(...) bytes."""
    fn_name = "attn_fwd_split"
    B, Hq, Hkv, N, d = _dims(q, k, v)
    for name, t, dt in (("q", q, torch.bfloat16), ("k", k, torch.bfloat16), ("v", v, torch.bfloat16),
                        ("o", o, torch.bfloat16), ("lse", lse, torch.float32)):
        if t.dtype != dt:
            raise ValueError(f"{fn_name}: {name} must be {dt}, got {t.dtype}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be contiguous on {q.device}")
    if o.shape != q.shape or lse.shape != (B, Hq, N):
        raise ValueError(f"{fn_name}: o must be {tuple(q.shape)} and lse {(B, Hq, N)}")
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError(f"{fn_name}: workspace must be contiguous on {q.device}")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = _lib.attn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                 ws_bytes, int(n_split), B, Hq, Hkv, N, d,
                                 ctypes.c_float(float(scale)), _stream_handle(stream, q.device))
    _raise(st, fn_name)


_FP8_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def fp8_padded_keys(N: int) -> int:
    """Row length of the transposed V of attn_fwd_fp8: N rounded up to 16."""
    return (int(N) + 15) // 16 * 16


def attn_fwd_fp8(q8, k8, vt8, o, lse, q_scale, k_scale, v_scale, scale, stream=None):
    """8-bit forward (C: attn_fwd_fp8).  q8 [B,Hq,N,d], k8 [B,Hkv,N,d] and
    vt8 [B,Hkv,d,Np] (V transposed, Np = fp8_padded_keys(N)) hold OCP E4M3
    codes (uint8 or float8_e4m3fn); o bf16 [B,Hq,N,d]; lse fp32 [B,Hq,N]."""
    fn_name = "attn_fwd_fp8"
    for name, t in (("q8", q8), ("k8", k8), ("vt8", vt8)):
        if t.dim() != 4 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be a contiguous 4-D device tensor")
        if t.dtype not in _FP8_DTYPES:
            raise ValueError(f"{fn_name}: {name} must be uint8 or float8_e4m3fn, got {t.dtype}")
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    want = {"k8": (B, Hkv, N, d), "vt8": (B, Hkv, d, fp8_padded_keys(N)), "o": (B, Hq, N, d),
            "lse": (B, Hq, N)}
    for name, t, dt in (("k8", k8, None), ("vt8", vt8, None), ("o", o, torch.bfloat16),
                        ("lse", lse, torch.float32)):
        if tuple(t.shape) != want[name]:
            raise ValueError(f"{fn_name}: {name} must be {want[name]}, got {tuple(t.shape)}")
        if dt is not None and t.dtype != dt:
            raise ValueError(f"{fn_name}: {name} must be {dt}, got {t.dtype}")
        if t.device != q8.device or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be contiguous on {q8.device}")
    with torch.cuda.device(q8.device):
        st = _lib.attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(o), _ptr(lse),
                               ctypes.c_float(float(q_scale)), ctypes.c_float(float(k_scale)),
                               ctypes.c_float(float(v_scale)), B, Hq, Hkv, N, d,
                               ctypes.c_float(float(scale)), _stream_handle(stream, q8.device))
    _raise(st, fn_name)


def attn_bwd_workspace_bytes(B, Hq, N) -> int:
    """Workspace bytes attn_bwd needs (0 for arguments it would reject)."""
    return int(_lib.attn_bwd_workspace_bytes(int(B), int(Hq), int(N)))


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, scale, stream=None):
    """Gradients of attn_fwd, bf16 I/O (C: attn_bwd)."""
    fn_name = "attn_bwd"
    B, Hq, Hkv, N, d = _dims(q, k, v)
    for name, t, dt, shape in (("q", q, torch.bfloat16, q.shape), ("o", o, torch.bfloat16, q.shape),
                               ("dout", dout, torch.bfloat16, q.shape),
                               ("dq", dq, torch.bfloat16, q.shape), ("dk", dk, torch.bfloat16, k.shape),
                               ("dv", dv, torch.bfloat16, k.shape), ("k", k, torch.bfloat16, k.shape),
                               ("v", v, torch.bfloat16, k.shape), ("lse", lse, torch.float32, (B, Hq, N))):
        if t.dtype != dt:
            raise ValueError(f"{fn_name}: {name} must be {dt}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn_name}: {name} must be {tuple(shape)}, got {tuple(t.shape)}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be contiguous on {q.device}")
    if workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError(f"{fn_name}: workspace must be contiguous on {q.device}")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        st = _lib.attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                           _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, B, Hq, Hkv, N, d,
                           ctypes.c_float(float(scale)), _stream_handle(stream, q.device))
    _raise(st, fn_name)


def attn_device_info(device=None):
    """(compute units, XCDs, L2 bytes of one XCD) of a device as the library
    reads them (C: attn_device_info)."""
    cu, xcd, l2 = _I(0), _I(0), _I(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        st = _lib.attn_device_info(ctypes.byref(cu), ctypes.byref(xcd), ctypes.byref(l2))
    _raise(st, "attn_device_info")
    return cu.value, xcd.value, l2.value


def attn_fwd_plan(B, Hq, Hkv, N, d, device=None) -> int:
    """ATTN_KERNEL_ROWS32 or ATTN_KERNEL_ROWS64: the kernel attn_fwd launches for
    these sizes on ``device`` (C: attn_fwd_plan)."""
    kern = _I(0)
    with torch.cuda.device(device if device is not None else torch.cuda.current_device()):
        st = _lib.attn_fwd_plan(int(B), int(Hq), int(Hkv), int(N), int(d), ctypes.byref(kern))
    _raise(st, "attn_fwd_plan")
    return kern.value


def attn_bwd_noalloc_max_rows() -> int:
    """Largest B * Hq * N that attn_bwd_noalloc accepts."""
    return int(_lib.attn_bwd_noalloc_max_rows())


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, scale, stream=None):
    """Gradients of attn_fwd with no workspace argument: the library's fixed
    scratch buffer holds the row sums (C: attn_bwd_noalloc).  Calls that may
    overlap on one device race on that buffer."""
    fn_name = "attn_bwd_noalloc"
    B, Hq, Hkv, N, d = _dims(q, k, v)
    for name, t, dt, shape in (("q", q, torch.bfloat16, q.shape), ("o", o, torch.bfloat16, q.shape),
                               ("dout", dout, torch.bfloat16, q.shape),
                               ("dq", dq, torch.bfloat16, q.shape), ("dk", dk, torch.bfloat16, k.shape),
                               ("dv", dv, torch.bfloat16, k.shape), ("k", k, torch.bfloat16, k.shape),
                               ("v", v, torch.bfloat16, k.shape), ("lse", lse, torch.float32, (B, Hq, N))):
        if t.dtype != dt:
            raise ValueError(f"{fn_name}: {name} must be {dt}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{fn_name}: {name} must be {tuple(shape)}, got {tuple(t.shape)}")
        if t.device != q.device or not t.is_contiguous():
            raise ValueError(f"{fn_name}: {name} must be contiguous on {q.device}")
    with torch.cuda.device(q.device):
        st = _lib.attn_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                   _ptr(dq), _ptr(dk), _ptr(dv), B, Hq, Hkv, N, d,
                                   ctypes.c_float(float(scale)), _stream_handle(stream, q.device))
    _raise(st, fn_name)


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def fwd(q, k, v, scale=None, stream=None):
    """(o, lse) = attention forward; bf16 or fp32 by q's dtype; scale defaults to 1/sqrt(d)."""
    B, Hq, _, N, d = _dims(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    if q.dtype == torch.bfloat16:
        attn_fwd(q, k, v, o, lse, _scale(scale, d), stream)
    elif q.dtype == torch.float32:
        attn_fwd_f32(q, k, v, o, lse, _scale(scale, d), stream)
    else:
        raise ValueError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    return o, lse


def fwd_materialized(q, k, v, scale=None, stream=None):
    """(o, lse, s, p) through the materialising three-kernel path."""
    B, Hq, _, N, d = _dims(q, k, v)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    s = torch.empty((B, Hq, N, N), dtype=torch.float32, device=q.device)
    p = torch.empty((B, Hq, N, N), dtype=q.dtype, device=q.device)
    if q.dtype == torch.bfloat16:
        attn_fwd_materialized(q, k, v, o, lse, s, p, _scale(scale, d), stream)
    elif q.dtype == torch.float32:
        attn_fwd_materialized_f32(q, k, v, o, lse, s, p, _scale(scale, d), stream)
    else:
        raise ValueError(f"unsupported dtype {q.dtype}; use bfloat16 or float32")
    return o, lse, s, p


def fwd_split(q, k, v, n_split, scale=None, stream=None):
    """(o, lse) through the split-KV path (bf16); allocates its workspace."""
    B, Hq, _, N, d = _dims(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError(f"the split-KV path takes bfloat16, got {q.dtype}")
    need = attn_fwd_split_workspace_bytes(B, Hq, N, d, n_split)
    if need == 0:
        raise ValueError(f"attn_fwd_split: invalid arguments (n_split={n_split}, d={d})")
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    attn_fwd_split(q, k, v, o, lse, ws, n_split, _scale(scale, d), stream)
    return o, lse


def bwd(q, k, v, o, lse, dout, scale=None, stream=None):
    """(dq, dk, dv) of the forward (o, lse) = fwd(q, k, v, scale); bf16."""
    B, Hq, _, N, d = _dims(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError(f"the backward takes bfloat16, got {q.dtype}")
    ws = torch.empty(attn_bwd_workspace_bytes(B, Hq, N), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, _scale(scale, d), stream)
    return dq, dk, dv


def fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, scale=None, stream=None):
    """(o, lse) of the 8-bit forward; o is bf16; scale defaults to 1/sqrt(d)."""
    B, Hq, N, d = q8.shape
    o = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    attn_fwd_fp8(q8, k8, vt8, o, lse, q_scale, k_scale, v_scale, _scale(scale, d), stream)
    return o, lse
