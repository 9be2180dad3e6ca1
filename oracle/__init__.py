"""CPU FP64 oracle for paged decode and prefill attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path never does.
"""

from .paged_attention import (PAGE_SIZE, attend_one_head, bf16_bits_to_f64,
                              decode_attention, gather_sequence, kv_append, kv_write,
                              prefill_attention)

__all__ = ["PAGE_SIZE", "attend_one_head", "bf16_bits_to_f64",
           "decode_attention", "gather_sequence", "kv_append", "kv_write",
           "prefill_attention"]
