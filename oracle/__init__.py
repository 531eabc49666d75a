"""CPU oracle for exact attention forward and its gradients (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The GPU product path never
does, and this package never imports the GPU path.
"""
from .attention import (attention_head, attention_ref, attention_ref_rows,
                        attention_ref_sp, default_scale, head_scores, kv_head,
                        softmax_rows)
from .backward import attention_bwd_head, attention_bwd_ref
from .fp8 import (attention_fp8_ref, dequantize, e4m3_decode, fp8_bounds_rows, fp8_error_bound,
                  fp8_lse_bound, fp8_mean_square_bound, padded_keys)

__all__ = ["attention_head", "attention_ref", "attention_ref_rows",
           "attention_ref_sp", "default_scale", "head_scores", "kv_head",
           "softmax_rows", "attention_bwd_head", "attention_bwd_ref",
           "attention_fp8_ref", "dequantize", "e4m3_decode", "fp8_bounds_rows", "fp8_error_bound",
           "fp8_lse_bound", "fp8_mean_square_bound", "padded_keys"]
