"""Host-side logic: block manager (block table, refcounts, copy-on-write) and workloads."""
import json
import os

import numpy as np
import pytest
import torch

from paged_kv_cache_299_amd.block_manager import BlockManager, BlockPoolExhausted
from paged_kv_cache_299_amd import workloads
from paged_kv_cache_299_amd.layout import kv_cache_shapes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_block_manager_reproduces_the_worked_example():
    with open(os.path.join(GOLD, "worked_example.json"), encoding="utf-8") as f:
        g = json.load(f)
    B = g["block_size"]
    bm = BlockManager(8, B, free_order=[7, 1, 3, 5, 0, 2, 4, 6])
    for sid, name in enumerate(("A", "B")):
        req = g["requests"][name]
        bm.allocate(sid, req["tokens"])
        assert bm.block_table(sid) == [b for b, _ in req["blocks"]]
        # each token sits in the slot the picture shows
        for i in range(req["tokens"]):
            phys, picture = req["blocks"][i // B]
            assert bm.slot(sid, i) == phys * B + picture.index(f"t{i + 1}")
        assert bm.wasted_slots(sid) == sum(t == "_" for t in req["blocks"][-1][1])


def test_waste_is_below_one_block_and_no_block_is_shared_without_fork():
    rng = np.random.default_rng(0)
    B = 16
    bm = BlockManager(400, B, free_order=rng.permutation(400))
    lens = rng.integers(0, 300, size=20)
    for s, n in enumerate(lens):
        bm.allocate(s, int(n))
        assert 0 <= bm.wasted_slots(s) <= B - 1
    owned = [b for s in range(20) for b in bm.block_table(s)]
    assert len(owned) == len(set(owned))
    assert all(bm.refcount[b] == 1 for b in owned)


def test_fork_shares_blocks_with_refcount_equal_to_samples():
    bm = BlockManager(64, 16)
    bm.allocate(0, 40)
    for j in range(1, 8):
        bm.fork(0, j)
    for b in bm.block_table(0):
        assert bm.refcount[b] == 8
    assert all(bm.block_table(j) == bm.block_table(0) for j in range(8))


def test_copy_on_write_happens_iff_the_block_is_shared():
    bm = BlockManager(64, 4)
    bm.allocate(0, 6)               # blocks [a, b], b holds 2 of 4
    bm.fork(0, 1)
    last = bm.block_table(0)[-1]
    slot, copy = bm.append_slot(0)  # shared (refcount 2) -> copy
    assert copy is not None and copy[0] == last and copy[1] != last
    assert slot == copy[1] * 4 + 2
    assert bm.refcount[last] == 1 and bm.refcount[copy[1]] == 1
    slot, copy = bm.append_slot(1)  # now sole owner -> in place
    assert copy is None and slot == last * 4 + 2
    # a full last block gets a fresh block, never a copy
    bm.allocate(2, 8)
    bm.fork(2, 3)
    slot, copy = bm.append_slot(2)
    assert copy is None and bm.context_len(2) == 9 and len(bm.block_table(2)) == 3


def test_free_returns_blocks_and_exhaustion_raises():
    bm = BlockManager(4, 4)
    bm.allocate(0, 16)
    with pytest.raises(BlockPoolExhausted):
        bm.allocate(1, 1)
    bm.fork(0, 1)
    bm.free(0)
    assert bm.num_free == 0          # still held by the fork
    bm.free(1)
    assert bm.num_free == 4


def test_tiny_workload_matches_its_description():
    c = workloads.tiny()
    assert c.dtype == torch.float32 and c.q.shape == (1, 1, 64)
    assert int(c.context_lens[0]) == 101
    (step,) = c.steps
    table = c.block_tables[0].tolist()
    assert len(table) == 7 and len(set(table)) == 7
    assert int(step.slot_mapping[0]) == table[6] * 16 + 4
    k_shape, v_shape = kv_cache_shapes(16, 1, 64, 16, torch.float32)
    assert tuple(c.k_cache.shape) == k_shape and tuple(c.v_cache.shape) == v_shape
    # before the write: tokens 0..99 finite, slot of token 100 and after NaN
    last = table[6]
    assert torch.isfinite(c.k_cache[last, :, :, :4]).all()
    assert torch.isnan(c.k_cache[last, :, :, 4:]).all()
    assert torch.isnan(c.v_cache[last, :, :, 4:]).all()
    unused = sorted(set(range(16)) - set(table))
    assert torch.isnan(c.k_cache[unused]).all()


def test_parallel_sampling_copy_on_write_counts():
    plain = workloads.parallel_sampling(cow=False, num_prompts=2, max_private=40, num_heads=2,
                                        head_dim=16, num_blocks=256)
    assert all(not isinstance(s, workloads.CopyStep) for s in plain.steps)
    # all 8 samples of a prompt read the same 64 prompt blocks
    t = plain.block_tables
    for p in range(2):
        rows = t[p * 8:(p + 1) * 8, :64]
        assert (rows == rows[0]).all()
    cow = workloads.parallel_sampling(cow=True, num_prompts=2, max_private=40, num_heads=2,
                                      head_dim=16, num_blocks=256)
    copies = [s for s in cow.steps if isinstance(s, workloads.CopyStep)]
    assert len(copies) == 1 and copies[0].block_mapping.shape == (14, 2)  # 7 per prompt
    bm = cow.block_manager
    for p in range(2):
        rows = cow.block_tables[p * 8:(p + 1) * 8]
        assert (rows[:, :63] == rows[0, :63]).all()          # 63 full blocks still shared
        assert len(set(rows[:, 63].tolist())) == 8           # the partial block diverged
    pairs = copies[0].block_mapping
    assert len(set(pairs[:, 1].tolist())) == pairs.shape[0]  # destinations distinct
    assert not set(pairs[:, 1].tolist()) & set(pairs[:, 0].tolist())
    assert all(bm.refcount[b] >= 1 for b in cow.block_tables[cow.block_tables >= 0].tolist())


def test_workload_draws_are_seeded_and_in_range():
    rng = np.random.default_rng(2)
    ctx = rng.integers(128, 4096, size=32, endpoint=True)
    assert ctx.min() >= 128 and ctx.max() <= 4096
    z = np.random.default_rng(3).standard_normal(64)
    lens = np.clip(np.rint(512.0 * np.exp(z)), 16, 2048)
    assert lens.min() >= 16 and lens.max() <= 2048
    c1 = workloads.make_decode_case("x", seed=5, context_lens=[3, 40], num_heads=4,
                                    num_kv_heads=2, head_dim=64, block_size=16, num_blocks=12,
                                    max_blocks=3, dtype=torch.bfloat16)
    c2 = workloads.make_decode_case("x", seed=5, context_lens=[3, 40], num_heads=4,
                                    num_kv_heads=2, head_dim=64, block_size=16, num_blocks=12,
                                    max_blocks=3, dtype=torch.bfloat16)
    assert torch.equal(c1.q, c2.q) and torch.equal(c1.block_tables, c2.block_tables)
    assert torch.equal(c1.k_cache.isnan(), c2.k_cache.isnan())
    assert c1.block_tables[0, 1:].tolist() == [-1, -1]


def test_bench_traffic_record_is_used_only_for_the_recorded_kernel(tmp_path):
    """bench.py reports the committed HBM-traffic figure only for the workload,
    partitioning and kernel sources the counters were taken with."""
    import hashlib
    import json
    import bench
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "llama3_8b", "partition_tokens": "auto", "bytes_per_launch": 1234,
           "sources_sha256": {"k.hip": hashlib.sha256(b"kernel v1").hexdigest()}}
    (tmp_path / "profiles" / "decode_llama3_8b_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("llama3_8b", 0, root=str(tmp_path))[0] == 1234
    assert bench.measured_traffic("llama3_8b", 512, root=str(tmp_path))[0] is None
    assert bench.measured_traffic("opt_13b", 0, root=str(tmp_path)) == (None, None)
    src.write_text("kernel v2")
    assert bench.measured_traffic("llama3_8b", 0, root=str(tmp_path))[0] is None


def test_shares_blocks_reads_only_the_used_part_of_the_tables():
    from paged_kv_cache_299_amd.workloads import shares_blocks
    bt = torch.tensor([[3, 4, -1], [5, 4, 9]], dtype=torch.int32)
    assert shares_blocks(bt, torch.tensor([32, 17], dtype=torch.int32), 16)      # block 4 twice
    assert not shares_blocks(bt, torch.tensor([16, 17], dtype=torch.int32), 16)  # 4 unused in row 0
    assert not shares_blocks(bt, torch.tensor([0, 0], dtype=torch.int32), 16)
    ps = workloads.CASES["parallel_sampling"](fill=False, num_prompts=2, samples=3, num_blocks=512)
    assert shares_blocks(ps.block_tables, ps.context_lens, 16)
    ll = workloads.CASES["llama3_8b"](fill=False)
    assert not shares_blocks(ll.block_tables, ll.context_lens, 16)


def test_bench_refuses_more_than_one_gpu():
    """The build measures one GPU: --gpus N > 1 stops with a message, before
    anything touches a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_bench_decode_bytes_follow_the_per_token_closed_form():
    """Algorithmic bytes of one decode: 2 * Hkv * D * e per token (K and V),
    plus q in, out, the used table entries and the lengths.  At the
    Llama-3-8B shape a token costs 2 * 8 * 128 * 2 = 4,096 bytes."""
    import bench
    ctx = [1, 16, 17, 4096]
    S, Hq, Hkv, D, B, e = len(ctx), 32, 8, 128, 16, 2
    got = bench.decode_bytes(ctx, S, Hq, Hkv, D, B, e)
    tokens = sum(ctx)
    blocks = 1 + 1 + 2 + 256
    assert got == 4096 * tokens + 2 * S * Hq * D * e + 4 * blocks + 4 * S
    # no block shared: the unique-block count equals the logical one
    tables = np.arange(S * 256, dtype=np.int32).reshape(S, 256)
    assert bench.unique_decode_bytes(tables, ctx, S, Hq, Hkv, D, B, e) == got


# --------------------------------------------------------------------------
# block manager under random operation sequences (hypothesis): the pages'
# invariants after every step -- internal waste below one block, reference
# count = sequences holding the block, copy-on-write exactly when the block
# written to is shared -- and, through a model of the pool's contents, that
# no sequence ever sees a token another sequence wrote.
# [論文解説: PagedAttention, 技術的詳細 › メモリ断片化の定量的分析 and
#  › Copy-on-Write KVキャッシュ共有]
# --------------------------------------------------------------------------
from hypothesis import given, settings, strategies as st  # noqa: E402

_OPS = st.lists(st.tuples(st.sampled_from(["alloc", "fork", "append", "free"]),
                          st.integers(0, 1000), st.integers(0, 40)),
                min_size=1, max_size=120)


@settings(max_examples=150, deadline=None)
@given(ops=_OPS, B=st.sampled_from([1, 2, 4, 16]), nblocks=st.integers(1, 48))
def test_block_manager_invariants_under_random_operations(ops, B, nblocks):
    from paged_kv_cache_299_amd.block_manager import BlockPoolExhausted as Exhausted
    bm = BlockManager(nblocks, B)
    storage = {}   # slot -> token id: what the pool holds
    seen = {}      # sequence -> the token ids it must read, in order
    next_tok = [0]
    next_seq = [0]

    def new_tok():
        next_tok[0] += 1
        return next_tok[0]

    def new_seq():
        next_seq[0] += 1
        return next_seq[0]

    for op, pick, n in ops:
        live = sorted(seen)
        if op == "alloc":
            sid = new_seq()
            try:
                bm.allocate(sid, n)
            except Exhausted:
                continue
            seen[sid] = [new_tok() for _ in range(n)]
            for p, t in enumerate(seen[sid]):
                storage[bm.slot(sid, p)] = t
        elif not live:
            continue
        elif op == "fork":
            parent = live[pick % len(live)]
            child = new_seq()
            bm.fork(parent, child)
            seen[child] = list(seen[parent])
        elif op == "append":
            sid = live[pick % len(live)]
            table = bm.block_table(sid)
            ctx = bm.context_len(sid)
            last_shared = (ctx % B != 0) and bm.refcount[table[-1]] > 1
            try:
                slot, copy = bm.append_slot(sid)
            except Exhausted:
                assert bm.block_table(sid) == table and bm.context_len(sid) == ctx
                continue
            # copy-on-write exactly when the partly filled last block is shared
            assert (copy is not None) == last_shared
            if copy is not None:
                src, dst = copy
                for off in range(B):
                    if src * B + off in storage:
                        storage[dst * B + off] = storage[src * B + off]
            assert bm.refcount[slot // B] == 1      # the slot written is private
            t = new_tok()
            storage[slot] = t
            seen[sid].append(t)
        else:  # free
            sid = live[pick % len(live)]
            bm.free(sid)
            del seen[sid]

        # invariants after every operation
        holders = {}
        for sid in seen:
            table = bm.block_table(sid)
            ctx = bm.context_len(sid)
            assert ctx == len(seen[sid])
            assert len(table) == -(-ctx // B)
            assert 0 <= bm.wasted_slots(sid) <= B - 1
            assert len(set(table)) == len(table)
            for b in table:
                holders[b] = holders.get(b, 0) + 1
            # every sequence reads back exactly its own tokens
            assert [storage.get(bm.slot(sid, p)) for p in range(ctx)] == seen[sid]
        for b in range(nblocks):
            assert bm.refcount[b] == holders.get(b, 0)
        assert bm.num_free == nblocks - len(holders)
