"""Exact IO-aware attention forward for MI355X (gfx950).

The compute lives in the C-ABI library ``libattn.so`` (hand-written HIP
kernels); :mod:`exact_io_aware_73_amd.attn` is the thin ctypes binding and
loads the library on import (failing loudly if it has not been built).
Importing the package itself loads nothing.
"""
