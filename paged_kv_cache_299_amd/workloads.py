"""Seeded synthetic workloads for paged decode attention.

Inputs only: random values, length draws, block placement.  Nothing here
computes attention or touches the kernels; both the GPU path and the CPU
oracle are fed from these cases.

Recipe (every case):
  * numpy.random.default_rng(seed); draws in a fixed order: context lengths,
    block placement, pool contents, queries, new tokens;
  * values ~ N(0, 1) drawn as float32 and rounded to the case dtype
    (round-to-nearest-even through torch);
  * physical placement: a random permutation of the pool is the free-block
    order, and sequences take blocks from it in sequence order;
  * every slot that holds no token is NaN (unused blocks and the tail of each
    sequence's last block), so a kernel that reads one shows it;
  * a decode step appends one token per sequence: the pools hold ctx - 1
    tokens, the write step stores token ctx - 1, and decode attends over ctx.

Named cases (sizes of the five decode workloads of the method's benchmark
table, see `CASES`):
  tiny      1 seq, 1 head, D 64, B 16, ctx 100 (7 blocks, last 4/16 full),
            16 blocks, fp32; one new token at position 100, then ctx 101
  llama3_8b 32 seqs, 32 q heads / 8 kv heads, D 128, B 16, ctx ~ U{128..4096},
            pool 12,000 blocks, bf16
  opt_13b   64 seqs, 40 heads, D 128, B 16, ctx = clip(round(512 e^Z), 16, 2048),
            Z ~ N(0, 1), pool 10,000 blocks, fp16
  parallel_sampling
            16 prompts x 8 samples, 32 heads, D 128, B 16, bf16; a 1,024-token
            prompt whose 64 blocks all 8 samples share, then U{0..256} private
            tokens per sample.  The "cow" variant uses a 1,016-token prompt so
            the last prompt block is 8/16 full and the first divergent write
            copies it (7 copies per prompt, 112 pairs)
  long_ctx  4 seqs, 32 q heads / 8 kv heads, D 128, B 16, ctx 32,768 / 65,536 /
            98,304 / 131,072, pool 24,576 blocks, bf16, 512-token partitions
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from .block_manager import BlockManager
from .layout import kv_cache_shapes


@dataclass
class WriteStep:
    k_new: torch.Tensor          # [T, Hkv, D]
    v_new: torch.Tensor          # [T, Hkv, D]
    slot_mapping: torch.Tensor   # int64 [T]


@dataclass
class CopyStep:
    block_mapping: torch.Tensor  # int64 [n, 2]


@dataclass
class DecodeCase:
    name: str
    dtype: torch.dtype
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks: int
    q: torch.Tensor              # [S, Hq, D]
    k_cache: torch.Tensor        # K pool before the steps
    v_cache: torch.Tensor        # V pool before the steps
    block_tables: torch.Tensor   # int32 [S, MB]
    context_lens: torch.Tensor   # int32 [S], after the steps
    scale: float
    steps: List[object] = field(default_factory=list)   # CopyStep / WriteStep, in order
    partition_tokens: Optional[int] = None
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads


def _randn(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(a).to(dtype)


def _fill_pools(rng, bm: BlockManager, seq_ids: Sequence[int], Hkv: int, D: int, B: int,
                NB: int, dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    """Pools with N(0,1) in every slot that holds a token, NaN elsewhere."""
    k_shape, v_shape = kv_cache_shapes(NB, Hkv, D, B, dtype)
    k = torch.full(k_shape, float("nan"), dtype=dtype)
    v = torch.full(v_shape, float("nan"), dtype=dtype)
    used = sorted({b for s in seq_ids for b in bm.block_table(s)})
    if used:
        idx = torch.tensor(used, dtype=torch.long)
        k[idx] = _randn(rng, (len(used),) + k_shape[1:], dtype)
        v[idx] = _randn(rng, (len(used),) + v_shape[1:], dtype)
    # empty tail of each last block back to NaN (token offset is axis 3 of both pools)
    for s in seq_ids:
        n = bm.context_len(s)
        table = bm.block_table(s)
        if table and n % B:
            last = table[-1]
            k[last, :, :, n % B:, :] = float("nan")
            v[last, :, :, n % B:] = float("nan")
    return k, v


def _tables(bm: BlockManager, seq_ids, MB: int) -> torch.Tensor:
    return torch.tensor(bm.tables(seq_ids, MB), dtype=torch.int32).reshape(len(seq_ids), MB)


def random_pools(seed: int, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int,
                 dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    """A K and a V pool (CPU) with N(0,1) in every slot: source or
    destination pools of block moves, where every byte is compared."""
    rng = np.random.default_rng(seed)
    k_shape, v_shape = kv_cache_shapes(num_blocks, num_kv_heads, head_dim, block_size, dtype)
    return _randn(rng, k_shape, dtype), _randn(rng, v_shape, dtype)


def make_decode_case(name: str, *, seed: int, context_lens: Sequence[int], num_heads: int,
                     num_kv_heads: int, head_dim: int, block_size: int, num_blocks: int,
                     max_blocks: int, dtype: torch.dtype, partition_tokens: Optional[int] = None,
                     rng: Optional[np.random.Generator] = None, fill: bool = True) -> DecodeCase:
    """One decode step for independent sequences: write token ctx-1, attend over ctx.

    A sequence with ctx 0 holds nothing and gets no new token (slot -1)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    S = len(context_lens)
    B = block_size
    ctx = [int(c) for c in context_lens]
    if any(c < 0 for c in ctx):
        raise ValueError("context lengths must be >= 0")
    if any(-(-c // B) > max_blocks for c in ctx):
        raise ValueError("a context does not fit max_blocks")
    bm = BlockManager(num_blocks, B, free_order=rng.permutation(num_blocks))
    for s in range(S):
        bm.allocate(s, max(ctx[s] - 1, 0))
    k, v = (_fill_pools(rng, bm, range(S), num_kv_heads, head_dim, B, num_blocks, dtype)
            if fill else (None, None))
    q = _randn(rng, (S, num_heads, head_dim), dtype)
    # an empty sequence (ctx 0) gets no new token: slot -1 is skipped by the write
    slots = [bm.append_slot(s)[0] if ctx[s] > 0 else -1 for s in range(S)]
    step = WriteStep(_randn(rng, (S, num_kv_heads, head_dim), dtype),
                     _randn(rng, (S, num_kv_heads, head_dim), dtype),
                     torch.tensor(slots, dtype=torch.int64))
    case = DecodeCase(name, dtype, S, num_heads, num_kv_heads, head_dim, B, num_blocks,
                      max_blocks, q, k, v, _tables(bm, range(S), max_blocks),
                      torch.tensor(ctx, dtype=torch.int32), 1.0 / math.sqrt(head_dim),
                      [step], partition_tokens, seed)
    case.block_manager = bm
    return case


def tiny(seed: int = 1, fill: bool = True) -> DecodeCase:
    """1 seq, 1 head, D 64, ctx 100 -> write token 100 -> ctx 101, fp32, 16 blocks."""
    return make_decode_case("tiny", seed=seed, context_lens=[101], num_heads=1, num_kv_heads=1,
                            head_dim=64, block_size=16, num_blocks=16, max_blocks=7,
                            dtype=torch.float32, fill=fill)


def llama3_8b(seed: int = 2, num_seqs: int = 32, fill: bool = True,
              block_size: int = 16, max_tokens: int = 4096) -> DecodeCase:
    """Block sizes other than 16 keep the pool's token capacity (12,000 x 16);
    max_tokens is the block tables' capacity (the lengths stay U{128..4096})."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 4096, size=num_seqs, endpoint=True)
    return make_decode_case("llama3_8b", seed=seed, context_lens=ctx, num_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=block_size,
                            num_blocks=12000 * 16 // block_size,
                            max_blocks=max_tokens // block_size, dtype=torch.bfloat16, rng=rng,
                            fill=fill)


def many_seqs(seed: int = 6, num_seqs: int = 512, fill: bool = True) -> DecodeCase:
    """512 sequences of U{128..600} tokens, Llama-3-8B heads (32 q / 8 kv, D 128,
    bf16), tables of 40 blocks: the unit search walks 8 rounds of 64 sequences."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(128, 600, size=num_seqs, endpoint=True)
    need = int(sum(-(-int(c) // 16) for c in ctx))
    return make_decode_case("many_seqs", seed=seed, context_lens=ctx, num_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16,
                            num_blocks=need + 512, max_blocks=40, dtype=torch.bfloat16, rng=rng,
                            fill=fill)


def opt_13b(seed: int = 3, num_seqs: int = 64, fill: bool = True) -> DecodeCase:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal(num_seqs)
    ctx = np.clip(np.rint(512.0 * np.exp(z)), 16, 2048).astype(np.int64)
    return make_decode_case("opt_13b", seed=seed, context_lens=ctx, num_heads=40,
                            num_kv_heads=40, head_dim=128, block_size=16, num_blocks=10000,
                            max_blocks=128, dtype=torch.float16, rng=rng, fill=fill)


def long_ctx(seed: int = 5, fill: bool = True) -> DecodeCase:
    ctx = [32768, 65536, 98304, 131072]
    return make_decode_case("long_ctx", seed=seed, context_lens=ctx, num_heads=32,
                            num_kv_heads=8, head_dim=128, block_size=16, num_blocks=24576,
                            max_blocks=8192, dtype=torch.bfloat16, partition_tokens=512,
                            fill=fill)


def parallel_sampling(seed: int = 4, cow: bool = False, num_prompts: int = 16,
                      samples: int = 8, prompt_tokens: Optional[int] = None,
                      max_private: int = 256, num_heads: int = 32, head_dim: int = 128,
                      num_blocks: int = 4096, fill: bool = True,
                      num_kv_heads: Optional[int] = None) -> DecodeCase:
    """Parallel sampling over shared prompt blocks.

    Sequence id = prompt * samples + sample.  Sample 0 holds the prompt, the
    other samples fork from it (refcount = samples on every prompt block).
    Steps, in order:
      cow=False: prompt 1,024 tokens = 64 full blocks, so no write lands in a
        shared block; one write step stores all private tokens.
      cow=True:  prompt 1,016 tokens (last prompt block 8/16 full).  The first
        generated token of every sample hits the shared last block: samples
        0..6 copy it (CopyStep of 7 pairs per prompt), sample 7 finds
        refcount 1 and writes in place; then a write step for those first
        tokens and one for the remaining private tokens.
    Each sample has U{0..max_private} private tokens (cow: at least 1);
    decode attends over prompt + private tokens.
    """
    rng = np.random.default_rng(seed)
    B = 16
    P = (1016 if cow else 1024) if prompt_tokens is None else prompt_tokens
    S = num_prompts * samples
    n_priv = rng.integers(1 if cow else 0, max_private, size=S, endpoint=True)
    Hkv = num_heads if num_kv_heads is None else num_kv_heads
    max_blocks = -(-(P + max_private) // B)
    bm = BlockManager(num_blocks, B, free_order=rng.permutation(num_blocks))
    for p in range(num_prompts):
        bm.allocate(p * samples, P)
        for j in range(1, samples):
            bm.fork(p * samples, p * samples + j)
    k, v = (_fill_pools(rng, bm, range(S), Hkv, head_dim, B, num_blocks, torch.bfloat16)
            if fill else (None, None))
    q = _randn(rng, (S, num_heads, head_dim), torch.bfloat16)
    steps: List[object] = []
    first_slots: List[int] = []
    if cow:
        pairs = []
        for s in range(S):
            slot, copy = bm.append_slot(s)
            first_slots.append(slot)
            if copy is not None:
                pairs.append(copy)
        steps.append(CopyStep(torch.tensor(pairs, dtype=torch.int64).reshape(-1, 2)))
        steps.append(WriteStep(_randn(rng, (S, Hkv, head_dim), torch.bfloat16),
                               _randn(rng, (S, Hkv, head_dim), torch.bfloat16),
                               torch.tensor(first_slots, dtype=torch.int64)))
        rest = [int(n) - 1 for n in n_priv]
    else:
        rest = [int(n) for n in n_priv]
    slots = []
    for s in range(S):
        for _ in range(rest[s]):
            slots.append(bm.append_slot(s)[0])
    T = len(slots)
    steps.append(WriteStep(_randn(rng, (T, Hkv, head_dim), torch.bfloat16),
                           _randn(rng, (T, Hkv, head_dim), torch.bfloat16),
                           torch.tensor(slots, dtype=torch.int64)))
    ctx = torch.tensor([bm.context_len(s) for s in range(S)], dtype=torch.int32)
    case = DecodeCase("parallel_sampling_cow" if cow else "parallel_sampling", torch.bfloat16,
                      S, num_heads, Hkv, head_dim, B, num_blocks, max_blocks, q, k, v,
                      _tables(bm, range(S), max_blocks), ctx, 1.0 / math.sqrt(head_dim), steps,
                      None, seed)
    case.block_manager = bm  # kept for the copy-on-write bookkeeping checks
    return case


def shares_blocks(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int) -> bool:
    """True when a physical block appears in the used part of more than one
    table row (a block with reference count > 1): the hint pa_decode_ex takes
    as PA_DECODE_SHARED_BLOCKS."""
    bt = block_tables.numpy()
    used = [bt[s, :-(-int(c) // block_size)] for s, c in enumerate(context_lens.tolist())]
    ids = np.concatenate(used) if used else np.zeros(0, dtype=bt.dtype)
    return bool(ids.size) and np.unique(ids).size < ids.size


@dataclass
class PrefillCase:
    """Prefill of a chunk of new tokens per sequence: the chunk's K/V are
    written into their slots (write_step), then every new query attends
    causally over its sequence's tokens."""
    name: str
    dtype: torch.dtype
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks: int
    q: torch.Tensor              # [T, Hq, D], the chunks packed in sequence order
    k_cache: torch.Tensor        # K pool holding the cached prefixes
    v_cache: torch.Tensor        # V pool holding the cached prefixes
    block_tables: torch.Tensor   # int32 [S, MB]
    context_lens: torch.Tensor   # int32 [S], prefix + chunk
    query_start: torch.Tensor    # int32 [S + 1]
    scale: float
    write_step: Optional[WriteStep]
    seed: int = 0

    @property
    def group(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def query_lens(self) -> List[int]:
        qs = self.query_start.tolist()
        return [qs[i + 1] - qs[i] for i in range(self.num_seqs)]

    @property
    def max_query_len(self) -> int:
        return max(self.query_lens, default=0)


def make_prefill_case(name: str, *, seed: int, context_lens: Sequence[int],
                      query_lens: Sequence[int], num_heads: int, num_kv_heads: int,
                      head_dim: int, block_size: int, num_blocks: int, max_blocks: int,
                      dtype: torch.dtype, rng: Optional[np.random.Generator] = None,
                      fill: bool = True) -> PrefillCase:
    """Sequence s holds context_lens[s] - query_lens[s] cached tokens; its
    query_lens[s] new tokens get slots appended by the block manager, their
    K/V go in with one write step, and their queries are packed into q."""
    rng = np.random.default_rng(seed) if rng is None else rng
    S, B = len(context_lens), block_size
    ctx = [int(c) for c in context_lens]
    ql = [int(n) for n in query_lens]
    if len(ql) != S or any(n < 0 or n > c for n, c in zip(ql, ctx)):
        raise ValueError("need 0 <= query_lens[s] <= context_lens[s]")
    if any(-(-c // B) > max_blocks for c in ctx):
        raise ValueError("a context does not fit max_blocks")
    bm = BlockManager(num_blocks, B, free_order=rng.permutation(num_blocks))
    for s in range(S):
        bm.allocate(s, ctx[s] - ql[s])
    k, v = (_fill_pools(rng, bm, range(S), num_kv_heads, head_dim, B, num_blocks, dtype)
            if fill else (None, None))
    slots = []
    for s in range(S):
        for _ in range(ql[s]):
            slots.append(bm.append_slot(s)[0])
    T = len(slots)
    q = _randn(rng, (T, num_heads, head_dim), dtype)
    step = WriteStep(_randn(rng, (T, num_kv_heads, head_dim), dtype),
                     _randn(rng, (T, num_kv_heads, head_dim), dtype),
                     torch.tensor(slots, dtype=torch.int64)) if T else None
    qs = torch.tensor(np.concatenate([[0], np.cumsum(ql)]), dtype=torch.int32)
    return PrefillCase(name, dtype, S, num_heads, num_kv_heads, head_dim, B, num_blocks,
                       max_blocks, q, k, v, _tables(bm, range(S), max_blocks),
                       torch.tensor(ctx, dtype=torch.int32), qs, 1.0 / math.sqrt(head_dim),
                       step, seed)


def prefill_llama3_8b(seed: int = 6, fill: bool = True) -> PrefillCase:
    """Whole prompts, Llama-3-8B-shaped attention: 8 prompts of U{1024..4096}
    tokens, 32 query / 8 kv heads, D 128, bf16."""
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1024, 4096, size=8, endpoint=True)
    return make_prefill_case("prefill_llama3_8b", seed=seed, context_lens=ctx, query_lens=ctx,
                             num_heads=32, num_kv_heads=8, head_dim=128, block_size=16,
                             num_blocks=4096, max_blocks=256, dtype=torch.bfloat16, rng=rng,
                             fill=fill)


def prefill_chunked_llama3_8b(seed: int = 7, fill: bool = True) -> PrefillCase:
    """Chunked prefill: 8 sequences with cached prefixes of U{0..15360} tokens
    each take a 1,024-token chunk, Llama-3-8B-shaped, bf16."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 15360, size=8, endpoint=True)
    ctx = prefix + 1024
    return make_prefill_case("prefill_chunked_llama3_8b", seed=seed, context_lens=ctx,
                             query_lens=[1024] * 8, num_heads=32, num_kv_heads=8, head_dim=128,
                             block_size=16, num_blocks=9000, max_blocks=1024,
                             dtype=torch.bfloat16, rng=rng, fill=fill)


def prefill_flops(case: PrefillCase) -> int:
    """Useful flops: query i of n at position p = ctx - n + i scores p + 1
    keys (2 D flops each) and sums as many values (2 D flops each), per query
    head."""
    total = 0
    for c, n in zip(case.context_lens.tolist(), case.query_lens):
        keys = n * (c - n) + n * (n + 1) // 2  # sum over the chunk of (p + 1)
        total += 4 * case.head_dim * case.num_heads * keys
    return total


@dataclass
class SwapPlan:
    """Preemption by swapping for one decode batch: the preempted sequences'
    blocks go to a CPU pool (swap-out) and, on resume, come back into free
    device blocks (swap-in)."""
    seq_ids: List[int]
    out_map: torch.Tensor        # int64 [n, 2] (device block, host block)
    in_map: torch.Tensor         # int64 [n, 2] (host block, new device block)
    num_host_blocks: int


def swap_plan(case: DecodeCase, num_preempted: int, seed: int = 7) -> SwapPlan:
    """Preempt the num_preempted sequences holding the most blocks; host
    blocks are handed out in order from an empty CPU pool, and the swap-in
    targets are blocks no sequence of the case uses, in seeded order."""
    rng = np.random.default_rng(seed)
    B = case.block_size
    nblk = [-(-int(c) // B) for c in case.context_lens.tolist()]
    order = sorted(range(case.num_seqs), key=lambda s: (-nblk[s], s))[:num_preempted]
    dev_blocks = [int(b) for s in order for b in case.block_tables[s, :nblk[s]].tolist()]
    used = {int(b) for s in range(case.num_seqs) for b in case.block_tables[s, :nblk[s]].tolist()}
    free = np.array(sorted(set(range(case.num_blocks)) - used), dtype=np.int64)
    n = len(dev_blocks)
    if n > free.size:
        raise ValueError("not enough free device blocks to swap the sequences back in")
    host = np.arange(n, dtype=np.int64)
    back = rng.permutation(free)[:n]
    out_map = torch.from_numpy(np.stack([np.array(dev_blocks, dtype=np.int64), host], 1))
    in_map = torch.from_numpy(np.stack([host, back], 1))
    return SwapPlan(order, out_map.contiguous(), in_map.contiguous(), n)


def shared_prefix_groups(block_tables: torch.Tensor, context_lens: torch.Tensor,
                         block_size: int) -> Tuple[torch.Tensor, torch.Tensor, int]:
    """Groups of consecutive sequences whose tables start with the same
    physical block, and per group the number of leading table entries that
    are the same block in every member and lie wholly inside every member's
    context.  Returns (group_start int32 [NG+1], prefix_blocks int32 [NG],
    largest group size); a sequence that shares nothing is a group of one."""
    bt = block_tables.numpy()
    ctx = [int(c) for c in context_lens.tolist()]
    S = len(ctx)
    starts, prefix = [0], []
    s = 0
    while s < S:
        e = s + 1
        while e < S and ctx[s] > 0 and ctx[e] > 0 and bt[e, 0] == bt[s, 0]:
            e += 1
        full = min(ctx[s:e]) // block_size
        n = 0
        while n < full and all(bt[t, n] == bt[s, n] for t in range(s + 1, e)):
            n += 1
        prefix.append(n if e - s > 1 else 0)
        starts.append(e)
        s = e
    sizes = [starts[i + 1] - starts[i] for i in range(len(prefix))]
    return (torch.tensor(starts, dtype=torch.int32), torch.tensor(prefix, dtype=torch.int32),
            max(sizes, default=0))


CASES = {
    "tiny": tiny,
    "llama3_8b": llama3_8b,
    "llama3_8b_table128k": lambda **kw: llama3_8b(max_tokens=131072, **kw),
    "many_seqs": many_seqs,
    "opt_13b": opt_13b,
    "parallel_sampling": lambda **kw: parallel_sampling(cow=False, **kw),
    "parallel_sampling_cow": lambda **kw: parallel_sampling(cow=True, **kw),
    "long_ctx": long_ctx,
    "prefill_llama3_8b": prefill_llama3_8b,
    "prefill_chunked_llama3_8b": prefill_chunked_llama3_8b,
}
