"""Automatic partitions planned on the device.

Where the plain pa_decode splits contexts automatically on the matrix-core
kernel at B = 16 (fewer than 2,048 rows, at most 256 sequences, tables longer
than 512 tokens), every workgroup picks the partition length from the context
lengths it reads, by the rule pa_decode_plan applies to host lengths.  The
same length and the same fold order give the same bits, so pa_decode with
automatic partitions must equal pa_decode_ex at the host-planned length bit
for bit, whichever merge each takes; and both stay within the bound of the
oracle.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_299_amd as pa
from paged_kv_cache_299_amd import workloads

from parity import GpuCase, check_decode, log, oracle_apply_steps, oracle_decode, same_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = torch.device("cuda:0")
    pa.load_library()
    return d


def _case(ctxs, Hq, Hkv, D, dtype, seed, MB=None):
    need = sum(-(-c // 16) for c in ctxs)
    MB = MB or max(1, max(-(-c // 16) for c in ctxs))
    return workloads.make_decode_case("plan", seed=seed, context_lens=ctxs, num_heads=Hq,
                                      num_kv_heads=Hkv, head_dim=D, block_size=16,
                                      num_blocks=need + 7, max_blocks=MB, dtype=dtype)


def _plan(case):
    return pa.pa_decode_plan(case.context_lens, case.num_heads, case.num_kv_heads,
                             case.block_size, case.max_blocks, case.dtype)


def _run(g, P, **kw):
    pa.pa_decode(g.q, g.k, g.v, g.bt, g.cl, g.case.scale, g.out, partition_tokens=P, **kw)
    torch.cuda.synchronize()
    return g.out.cpu().clone()


def _draw(rng, S, cap, zeros=True):
    c = rng.integers(1, cap + 1, size=S)
    if zeros and S > 3:
        c[rng.integers(0, S)] = 0
        c[rng.integers(0, S)] = 1
        c[rng.integers(0, S)] = cap
    return [int(x) for x in c]


# (S, Hq, Hkv, D, dtype, table capacity in tokens)
SHAPES = [
    (32, 32, 8, 128, torch.bfloat16, 4096),     # the Llama-3-8B shape
    (7, 32, 8, 128, torch.float16, 2048),
    (64, 32, 8, 128, torch.bfloat16, 3000),     # one full round of the lane loop
    (65, 16, 4, 128, torch.bfloat16, 1500),     # a second round, 260 rows
    (200, 8, 8, 64, torch.float16, 1100),       # G = 1, 1,600 rows
    (256, 16, 4, 128, torch.bfloat16, 700),     # the most sequences the device plan takes
    (3, 64, 8, 128, torch.bfloat16, 20000),     # rows of more than 8 partitions: merge kernel
    (12, 32, 4, 128, torch.float16, 5000),      # kv heads not a multiple of 8: merge kernel
]


@pytest.mark.parametrize("idx", range(len(SHAPES)))
def test_device_plan_equals_host_plan(dev, idx):
    S, Hq, Hkv, D, dtype, cap = SHAPES[idx]
    rng = np.random.default_rng(500 + idx)
    ctxs = _draw(rng, S, cap)
    case = _case(ctxs, Hq, Hkv, D, dtype, seed=510 + idx, MB=-(-cap // 16))
    P = _plan(case)
    assert P in (512, 640, 768, 896, 1024), P
    g = GpuCase(case, dev)
    g.apply_steps()
    auto = _run(g, 0)
    planned = _run(g, P)
    mode = pa.pa_decode_merge_mode(S, Hq, Hkv, D, 16, case.max_blocks, dtype, 0)
    log(f"shape {idx}: S={S} Hq={Hq} Hkv={Hkv} cap={cap}: host plan P={P}, merge mode {mode}")
    assert same_bits(auto, planned), f"shape {idx}: automatic partitions differ from P={P}"
    # the separate merge kernel at the same device-planned length: same bits
    assert same_bits(_run(g, 0, merge_kernel=True), planned)
    if S * Hq <= 2048:
        kc, vc = oracle_apply_steps(case)
        check_decode(auto, oracle_decode(case, kc, vc), dtype, f"shape {idx} automatic")


def test_device_plan_follows_the_lengths_not_the_table(dev):
    """The same lengths in tables of 4,096 and of 131,072 tokens: one plan, one result."""
    rng = np.random.default_rng(77)
    ctxs = [int(c) for c in rng.integers(128, 4097, size=32)]
    small = _case(ctxs, 32, 8, 128, torch.bfloat16, seed=78, MB=256)
    P = _plan(small)
    g = GpuCase(small, dev)
    g.apply_steps()
    ref = _run(g, 0)
    assert same_bits(ref, _run(g, P))
    big_bt = torch.zeros((32, 8192), dtype=torch.int32)
    big_bt[:, :256] = small.block_tables
    cl = g.cl
    bt = big_bt.to(dev)
    out = torch.empty_like(g.q)
    pa.pa_decode(g.q, g.k, g.v, bt, cl, small.scale, out)
    torch.cuda.synchronize()
    assert same_bits(out.cpu(), ref)


def test_device_plan_full_size_llama(dev):
    case = workloads.llama3_8b()
    P = _plan(case)
    g = GpuCase(case, dev)
    g.apply_steps()
    kc, vc = oracle_apply_steps(case)
    ref = oracle_decode(case, kc, vc)
    auto = _run(g, 0)
    check_decode(auto, ref, case.dtype, f"llama automatic (host plan P={P})", strict=True)
    assert same_bits(auto, _run(g, P))


def test_device_plan_append_and_allocation_free(dev):
    ctxs = [3000, 1, 700, 0, 2048, 2049, 4096, 90]
    case = _case(ctxs, 32, 8, 128, torch.bfloat16, seed=81, MB=256)
    P = _plan(case)
    g = GpuCase(case, dev)
    g.apply_steps()
    ref = _run(g, P)
    out = torch.full_like(g.q, float("nan"))
    pa.pa_decode_noalloc(g.q, g.k, g.v, g.bt, g.cl, case.scale, out)
    torch.cuda.synchronize()
    assert same_bits(out.cpu(), ref)
    # one call that stores the new tokens and decodes, automatic partitions
    g2 = GpuCase(case, dev)
    st = case.steps[-1]
    pa.pa_decode_append(g2.q, st.k_new.to(dev), st.v_new.to(dev), g2.k, g2.v, g2.bt, g2.cl,
                        case.scale, g2.out)
    torch.cuda.synchronize()
    assert same_bits(g2.out.cpu(), ref)
    assert same_bits(g2.k.cpu(), g.k.cpu()) and same_bits(g2.v.cpu(), g.v.cpu())


def test_no_device_plan_outside_its_shapes(dev):
    """More than 256 sequences, 2,048 rows or more, fp32, B = 32: the automatic
    length as before (the result equals pa_decode_ex with partition_tokens 0)."""
    rng = np.random.default_rng(90)
    for S, Hq, Hkv, dtype in [(300, 8, 2, torch.bfloat16), (260, 32, 8, torch.bfloat16),
                              (20, 8, 8, torch.float32)]:
        ctxs = [int(c) for c in rng.integers(0, 1500, size=S)]
        case = _case(ctxs, Hq, Hkv, 64, dtype, seed=91, MB=100)
        g = GpuCase(case, dev)
        g.apply_steps()
        a = _run(g, 0)
        if dtype != torch.float32 and S <= 256:
            assert same_bits(a, _run(g, _plan(case)))
        kc, vc = oracle_apply_steps(case)
        check_decode(a, oracle_decode(case, kc, vc), dtype, f"S={S} Hkv={Hkv} {dtype}")
