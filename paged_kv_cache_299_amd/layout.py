"""Storage format of the KV pools and the other operands of the library.

The pools are the library's own format (the pages only show one head with K
and V interleaved per slot, [論文解説: PagedAttention, 技術的詳細 ›
アルゴリズムの擬似コード]).  K and V live in two separate tensors, one
physical block after another; inside a block each kv head holds one
contiguous tile:

  K pool  [NB, Hkv, D // x, B, x]   x = 16 bytes / element size
          (8 for bf16 / fp16, 4 for fp32): each run of x dims of one token is
          16 contiguous bytes, and the 16-byte runs of the B tokens of a block
          are adjacent, so one 64-lane load instruction reads 1 KiB in order.
  V pool  [NB, Hkv, D, B]           the B tokens of one dim are contiguous,
          which is the operand order the P.V contraction consumes.

  q, out        [S, Hq, D]
  block_tables  int32 [S, MB]      entries past ceil(ctx / B) are never read
  context_lens  int32 [S]
  slot_mapping  int64 [T]          slot = physical block * B + offset, < 0 = skip
  block_mapping int64 [n, 2]       (src, dst) physical block pairs
"""
from __future__ import annotations

from typing import Tuple

import torch

DTYPE_CODES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
ELEM_BYTES = {torch.float32: 4, torch.float16: 2, torch.bfloat16: 2}


def k_chunk(dtype: torch.dtype) -> int:
    """Elements per 16-byte K run (the x of the K pool shape)."""
    return 16 // ELEM_BYTES[dtype]


def kv_cache_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                    dtype: torch.dtype) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    x = k_chunk(dtype)
    if head_dim % x:
        raise ValueError(f"head_dim {head_dim} is not a multiple of {x}")
    k_shape = (num_blocks, num_kv_heads, head_dim // x, block_size, x)
    v_shape = (num_blocks, num_kv_heads, head_dim, block_size)
    return k_shape, v_shape


def block_bytes(num_kv_heads: int, head_dim: int, block_size: int, dtype: torch.dtype) -> int:
    """Bytes of one physical block of one pool (all kv heads)."""
    return num_kv_heads * head_dim * block_size * ELEM_BYTES[dtype]
