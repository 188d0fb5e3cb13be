"""CPU oracle for paged decode attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  The GPU library does not use it in any way.
"""
from .oracle import (  # noqa: F401
    F32, F16, BF16,
    decode, decode_partitioned, prefill, write_kv, copy_blocks, swap_blocks,
    kv_cache_bytes, blocks_for_tokens, slot_of,
    f16_bits_to_float64, bf16_bits_to_float64,
    OracleError, num_threads, set_num_threads,
)
