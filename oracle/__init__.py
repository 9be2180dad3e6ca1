"""CPU FP64 oracle for paged decode and prefill attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. The product path never does.
"""

from .paged_attention import (K_SLAB, PAGE_SIZE, attend_one_head, bf16_bits_to_f64,
                              decode_attention, gather_sequence, k_slot_row, kv_append,
                              kv_write, prefill_attention, set_k_slot_row)

__all__ = ["K_SLAB", "PAGE_SIZE", "attend_one_head", "bf16_bits_to_f64",
           "decode_attention", "gather_sequence", "k_slot_row", "kv_append", "kv_write",
           "prefill_attention", "set_k_slot_row"]
