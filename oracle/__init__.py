"""CPU oracle (fp64, numpy) for paged-KV attention.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package.  The HIP library and its
Python binding never do.
"""
from .paged_attention import (append, attend, bf16_bits_to_f64, block_and_offset, decode,
                              decode_multi, gather_sequence, kv_head_of, prefill)

__all__ = ["append", "attend", "bf16_bits_to_f64", "block_and_offset", "decode", "decode_multi",
           "gather_sequence", "kv_head_of", "prefill"]
