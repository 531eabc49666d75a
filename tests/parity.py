"""Comparison helpers for GPU-vs-oracle parity (shared by the GPU tests,
``__graft_entry__.smoke()`` and ``bench.py``)."""
from __future__ import annotations

import numpy as np

# Tolerances: max-abs on O of 1e-2 for bf16 I/O and 1e-4 for fp32 I/O; lse
# within 1e-3.  A bf16 output cannot be closer to the exact value than half
# a bf16 spacing at that value (rounding the exact O to bf16 alone costs up
# to 0.0156 where |O| is in [4, 8)), so each element may also use that half
# spacing on top of the tolerance.  On the i.i.d. workloads |O| < 0.5 and
# the extra term stays below 0.001.
O_TOL = {"bf16": 1e-2, "f32": 1e-4}
LSE_TOL = 1e-3
MANTISSA_BITS = {"bf16": 7, "f32": 23}


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the I/O format at |x| (normal range)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(ax, 1e-30)))
    return 0.5 * np.exp2(e - MANTISSA_BITS[dtype])


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str) -> dict:
    """Element-wise comparison; returns error figures and pass flags."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref)
    allow = O_TOL[dtype] + half_ulp(o_ref, dtype)
    floor = np.abs(round_to(o_ref, dtype) - o_ref)
    lerr = np.abs(lse_gpu - lse_ref)
    res = {
        "max_abs_O": float(err.max()) if err.size else 0.0,
        "mean_abs_O": float(err.mean()) if err.size else 0.0,
        "max_rel_O": float((err / np.maximum(np.abs(o_ref), 1e-6)).max()) if err.size else 0.0,
        "floor_O": float(floor.max()) if floor.size else 0.0,
        "max_abs_lse": float(lerr.max()) if lerr.size else 0.0,
        "finite": bool(np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu))),
    }
    res["o_ok"] = bool(np.all(err <= allow)) and res["finite"]
    res["lse_ok"] = bool(np.all(lerr <= LSE_TOL)) and res["finite"]
    res["ok"] = res["o_ok"] and res["lse_ok"]
    return res


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the I/O format (round to nearest even)."""
    import torch
    t = torch.from_numpy(np.asarray(x, dtype=np.float64))
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return t.to(tdt).to(torch.float64).numpy()
