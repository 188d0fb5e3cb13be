"""Host-side KV block manager: free list, block tables, refcounts, copy-on-write.

This is the bookkeeping that sits beside the kernels, not on the GPU:

* a sequence of T tokens owns ceil(T / B) fixed-size physical blocks that may
  sit anywhere in the pool, and a block table maps its logical block i to a
  physical block [論文解説: PagedAttention, 技術的詳細 › PagedAttentionアルゴリズム,
  block definition and block table];
* position p of a sequence lives in slot  table[p // B] * B + p % B;
* forking a sequence (parallel sampling) shares its blocks and raises their
  reference count; a write into a block whose count is above one first copies
  the block to a fresh one [論文解説: PagedAttention, 技術的詳細 ›
  Copy-on-Write KVキャッシュ共有, steps 1-3];
* internal waste is at most B - 1 slots per sequence and there is no external
  fragmentation [same page, メモリ断片化の定量的分析].

The (src, dst) pairs it emits are what the copy kernel consumes, and the slots
are what the write kernel consumes.  Running out of free blocks raises
BlockPoolExhausted: in the pages' system that is the point where the scheduler
preempts a request (swap or recompute).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple


class BlockPoolExhausted(RuntimeError):
    """No free physical block is left."""


@dataclass
class _Seq:
    blocks: List[int] = field(default_factory=list)
    num_tokens: int = 0


class BlockManager:
    """Allocator for one pool of `num_blocks` blocks of `block_size` tokens.

    `free_order` fixes the order in which free blocks are handed out (the
    first element is allocated first); by default blocks go out as 0, 1, 2...
    A random permutation gives the shuffled placement the workloads use.
    """

    def __init__(self, num_blocks: int, block_size: int,
                 free_order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("num_blocks must be >= 0 and block_size > 0")
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of range(num_blocks)")
        self.num_blocks = num_blocks
        self.block_size = block_size
        # pop() takes from the end, so keep the list reversed
        self._free: List[int] = order[::-1]
        self.refcount: List[int] = [0] * num_blocks
        self._seqs: Dict[int, _Seq] = {}

    # ---- queries -------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def seq_ids(self) -> List[int]:
        return list(self._seqs)

    def block_table(self, seq_id: int) -> List[int]:
        return list(self._seqs[seq_id].blocks)

    def context_len(self, seq_id: int) -> int:
        return self._seqs[seq_id].num_tokens

    def slot(self, seq_id: int, position: int) -> int:
        """Flat slot (physical block * B + offset) of a logical position."""
        seq = self._seqs[seq_id]
        if not 0 <= position < len(seq.blocks) * self.block_size:
            raise ValueError(f"position {position} has no block in sequence {seq_id}")
        B = self.block_size
        return seq.blocks[position // B] * B + position % B

    def slots(self, seq_id: int) -> List[int]:
        return [self.slot(seq_id, p) for p in range(self._seqs[seq_id].num_tokens)]

    def wasted_slots(self, seq_id: int) -> int:
        seq = self._seqs[seq_id]
        return len(seq.blocks) * self.block_size - seq.num_tokens

    # ---- allocation ----------------------------------------------------
    def _take(self) -> int:
        if not self._free:
            raise BlockPoolExhausted(f"all {self.num_blocks} blocks are in use")
        b = self._free.pop()
        self.refcount[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self._free.append(b)

    def allocate(self, seq_id: int, num_tokens: int) -> List[int]:
        """New sequence holding `num_tokens` tokens: ceil(T / B) blocks."""
        if seq_id in self._seqs:
            raise ValueError(f"sequence {seq_id} exists")
        if num_tokens < 0:
            raise ValueError("num_tokens must be >= 0")
        need = -(-num_tokens // self.block_size)
        if need > len(self._free):
            raise BlockPoolExhausted(f"need {need} blocks, {len(self._free)} free")
        seq = _Seq([self._take() for _ in range(need)], num_tokens)
        self._seqs[seq_id] = seq
        return list(seq.blocks)

    def fork(self, parent_id: int, child_id: int) -> None:
        """Child shares every block of the parent; each shared count goes up."""
        if child_id in self._seqs:
            raise ValueError(f"sequence {child_id} exists")
        parent = self._seqs[parent_id]
        for b in parent.blocks:
            self.refcount[b] += 1
        self._seqs[child_id] = _Seq(list(parent.blocks), parent.num_tokens)

    def append_slot(self, seq_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Reserve the slot of the next token of a sequence.

        Returns (slot, copy) where copy is a (src, dst) block pair when the
        last block was shared and had to be copied first (copy-on-write), or
        None.  A full last block (or an empty sequence) gets a fresh block.
        """
        seq = self._seqs[seq_id]
        B = self.block_size
        pos = seq.num_tokens
        copy = None
        if pos == len(seq.blocks) * B:
            seq.blocks.append(self._take())
        else:
            last = seq.blocks[-1]
            if self.refcount[last] > 1:
                fresh = self._take()
                self.refcount[last] -= 1
                seq.blocks[-1] = fresh
                copy = (last, fresh)
        seq.num_tokens = pos + 1
        return seq.blocks[pos // B] * B + pos % B, copy

    def free(self, seq_id: int) -> None:
        seq = self._seqs.pop(seq_id)
        for b in seq.blocks:
            self._release(b)

    # ---- batch views ---------------------------------------------------
    def tables(self, seq_ids: Iterable[int], max_blocks: Optional[int] = None,
               pad: int = -1) -> List[List[int]]:
        """Block-table rows, padded with `pad` to `max_blocks` entries."""
        rows = [self.block_table(s) for s in seq_ids]
        width = max((len(r) for r in rows), default=0) if max_blocks is None else max_blocks
        for r in rows:
            if len(r) > width:
                raise ValueError("a table row is longer than max_blocks")
            r.extend([pad] * (width - len(r)))
        return rows
