"""CPU fp64 attention oracle.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The GPU library never calls it.
"""
from .exact import (attention, attention_backward, attention_backward_magnitudes, attention_fp8, attention_kvcache, attention_kvcache_append, attention_varlen,
                    attend_head, decode_e4m3, default_scale, kvcache_append, merge_partials, paged_to_contiguous)

__all__ = ["attention", "attention_backward", "attention_backward_magnitudes", "attention_fp8", "attention_kvcache", "attention_kvcache_append", "attention_varlen",
           "attend_head", "decode_e4m3", "default_scale", "kvcache_append", "merge_partials", "paged_to_contiguous"]
