"""CPU oracle for exact attention forward (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.  The GPU product path never
does, and this package never imports the GPU path.
"""
from .attention import (attention_head, attention_ref, attention_ref_rows,
                        attention_ref_sp, default_scale, head_scores, kv_head,
                        softmax_rows)

__all__ = ["attention_head", "attention_ref", "attention_ref_rows",
           "attention_ref_sp", "default_scale", "head_scores", "kv_head",
           "softmax_rows"]
