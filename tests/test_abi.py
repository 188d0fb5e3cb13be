"""The C ABI without a GPU: the library loads, exports what include/pa.h
declares, and rejects bad host-visible arguments before enqueuing anything."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_299_amd as pa
from paged_kv_cache_299_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
BF16, F16, F32 = 2, 1, 0
ALIGNED = ctypes.c_void_p(1 << 20)   # never dereferenced: checks fail before any launch


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # pragma: no cover
        return False


# The argument-check tests pass a fake device address (ALIGNED) and rely on
# every host check rejecting the call before a launch.  Where a GPU is
# visible a weakened check would launch kernels on that address, so they run
# only without one; the GPU suite covers real calls there.
fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only test")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pa.load_library()
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = pa.load_library()
    assert pa.pa_status_str(OK) == "PA_OK"
    assert pa.pa_status_str(INVALID) == "PA_ERR_INVALID_ARG"
    assert pa.pa_status_str(99) == "PA_ERR_UNKNOWN"
    assert lib.pa_version() >= 100


def _decode(lib, **kw):
    args = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, bt=ALIGNED, ctx=ALIGNED, scale=0.1, out=ALIGNED,
                S=4, Hq=32, Hkv=8, D=128, B=16, MB=16, NB=100, dtype=BF16, P=0, flags=0,
                stream=None)
    args.update(kw)
    return lib.pa_decode_ex(args["q"], args["k"], args["v"], args["bt"], args["ctx"],
                            args["scale"], args["out"], args["S"], args["Hq"], args["Hkv"],
                            args["D"], args["B"], args["MB"], args["NB"], args["dtype"], args["P"],
                            args["flags"], args["stream"])


@fake_pointers
@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30, Hkv=8), INVALID),
    (dict(dtype=7), INVALID),
    (dict(Hkv=0), INVALID),
    (dict(NB=0), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(P=20), INVALID),
    (dict(P=2048), INVALID),
    (dict(flags=8), INVALID),
    (dict(flags=2, B=32), UNSUPPORTED),          # the VALU kernel takes 16-token blocks
    (dict(B=24), UNSUPPORTED),
    (dict(B=32, dtype=F32), UNSUPPORTED),        # block sizes 8 / 32: matrix-core kernel only
    (dict(B=32, Hq=136, Hkv=4), UNSUPPORTED),    # more than 16 query heads per kv head
    (dict(B=8, P=1024), UNSUPPORTED),            # block size 8: partitions up to 512 tokens
    (dict(B=32, P=48), UNSUPPORTED),             # block size 32: partitions of whole blocks
    (dict(B=8, NB=300000), UNSUPPORTED),         # block size 8: pools under 2 GiB
    (dict(D=96), UNSUPPORTED),
    (dict(q=None), INVALID),
    (dict(out=ctypes.c_void_p((1 << 20) + 2)), INVALID),
    (dict(S=0), OK),
])
def test_decode_argument_checks(kw, status):
    lib = pa.load_library()
    assert _decode(lib, **kw) == status
    if status != OK:
        assert lib.pa_last_error().decode()


@fake_pointers
def test_read_tiles_argument_checks():
    lib = pa.load_library()
    A = ALIGNED

    def call(**kw):
        a = dict(sink=A, S=4, Hq=32, Hkv=8, D=128, B=16, MB=16, dtype=BF16, P=0)
        a.update(kw)
        return lib.pa_read_tiles(A, A, A, A, a["sink"], a["S"], a["Hq"], a["Hkv"], a["D"],
                                 a["B"], a["MB"], 100, a["dtype"], a["P"], None)
    assert call(dtype=F32) == UNSUPPORTED
    assert call(B=32) == UNSUPPORTED
    assert call(Hq=136, Hkv=4) == UNSUPPORTED
    assert call(sink=None) == INVALID
    assert call(sink=ctypes.c_void_p((1 << 20) + 2)) == INVALID
    assert call(Hq=30) == INVALID
    assert call(P=20) == INVALID
    assert call(S=0) == OK


def test_decode_plan_checks_and_choices():
    """pa_decode_plan: argument checks, 0 where the plan does not apply, and
    the partition length that minimises ceil(units / CUs) * longest unit
    (256 compute units where no GPU is visible), ties to the longer length."""
    lib = pa.load_library()
    out = ctypes.c_int(-1)

    def plan(ctx, Hq=32, Hkv=8, B=16, MB=256, dtype=BF16, ptr=True):
        arr = (ctypes.c_int32 * max(1, len(ctx)))(*ctx)
        rc = lib.pa_decode_plan(arr if len(ctx) else None, len(ctx), Hq, Hkv, B, MB, dtype,
                                ctypes.byref(out) if ptr else None)
        return rc, out.value
    assert plan([100], ptr=False)[0] == INVALID
    assert plan([100], dtype=7)[0] == INVALID
    assert plan([100], Hq=30)[0] == INVALID
    assert plan([]) == (OK, 0)
    assert plan([100], dtype=F32) == (OK, 0)                # VALU kernel: automatic
    assert plan([100], Hq=136, Hkv=4) == (OK, 0)
    assert plan([100], B=8) == (OK, 0)
    # block size 32: units are counted in 32-token blocks (100 tokens: 4 blocks)
    assert plan([100] * 32, B=32, MB=128) == (OK, 1024)
    # 1,100 tokens = 35 blocks of 32: 3 units of 12 at 512 (3 * 12 = 36),
    # 2 of 18 at 640..1024 (2 * 18 = 36): the tie goes to 1024
    assert plan([1100] * 32, B=32, MB=128) == (OK, 1024)
    assert plan([100] * 256) == (OK, 0)                      # 2048 rows: automatic
    # 32 sequences of 4096 tokens: n partitions cost n * ceil(256 / n) blocks,
    # 256 at P = 512 and 1024 (the longer wins the tie), more in between
    assert plan([4096] * 32) == (OK, 1024)
    # short contexts: one unit each at every length
    assert plan([100] * 32) == (OK, 1024)
    # 1,100 tokens (69 blocks): 3 units of 23 blocks at P = 512, cost 3 * 23 = 69;
    # 2 units of 35 blocks at 640..1024, cost 2 * 35 = 70
    assert plan([1100] * 32) == (OK, 512)
    # context lengths beyond the table are clamped (64 blocks = 1024 tokens)
    assert plan([100000] * 32, MB=64) == plan([1024] * 32, MB=64)


@fake_pointers
def test_write_and_copy_argument_checks():
    lib = pa.load_library()
    A = ALIGNED
    assert lib.pa_write_kv(A, A, A, A, A, 0, 8, 128, 16, 10, BF16, None) == OK
    assert lib.pa_write_kv(A, A, A, A, A, 5, 8, 12, 16, 10, BF16, None) == INVALID  # 12 % 8
    assert lib.pa_write_kv(A, A, A, A, A, 5, 8, 128, 16, 10, 9, None) == INVALID
    assert lib.pa_write_kv(None, A, A, A, A, 5, 8, 128, 16, 10, BF16, None) == INVALID
    assert lib.pa_copy_blocks(A, A, A, 0, 8, 128, 16, 10, BF16, None) == OK
    assert lib.pa_copy_blocks(A, A, None, 3, 8, 128, 16, 10, BF16, None) == INVALID
    assert lib.pa_copy_blocks(A, A, A, -1, 8, 128, 16, 10, BF16, None) == INVALID


@fake_pointers
def test_swap_argument_checks():
    """Every check that needs no HIP call comes before the pointer queries."""
    lib = pa.load_library()
    A = ALIGNED
    assert lib.pa_swap_blocks(A, A, A, A, A, 0, 8, 128, 16, 10, 20, BF16, None) == OK
    assert lib.pa_swap_blocks(A, A, A, A, A, 3, 8, 128, 16, 10, 0, BF16, None) == INVALID
    assert lib.pa_swap_blocks(A, A, A, A, A, 3, 8, 128, 16, 0, 20, BF16, None) == INVALID
    assert lib.pa_swap_blocks(A, A, A, A, A, -1, 8, 128, 16, 10, 20, BF16, None) == INVALID
    assert lib.pa_swap_blocks(A, A, A, A, A, 3, 8, 128, 16, 10, 20, 5, None) == INVALID
    assert lib.pa_swap_blocks(A, A, A, A, A, 3, 1, 1, 1, 10, 20, BF16, None) == INVALID  # 2 bytes
    assert lib.pa_swap_blocks(A, A, None, A, A, 3, 8, 128, 16, 10, 20, BF16, None) == INVALID
    odd = ctypes.c_void_p((1 << 20) + 8)
    assert lib.pa_swap_blocks(A, odd, A, A, A, 3, 8, 128, 16, 10, 20, BF16, None) == INVALID
    assert lib.pa_swap_blocks(A, A, A, A, ctypes.c_void_p((1 << 20) + 4), 3, 8, 128, 16, 10, 20,
                              BF16, None) == INVALID
    assert "pa_swap_blocks" in lib.pa_last_error().decode()


def test_python_swap_rejects_pageable_and_mismatched_pools():
    import torch
    from paged_kv_cache_299_amd.layout import kv_cache_shapes
    ks, vs = kv_cache_shapes(4, 2, 64, 16, torch.bfloat16)
    k, v = torch.zeros(ks, dtype=torch.bfloat16), torch.zeros(vs, dtype=torch.bfloat16)
    m = torch.zeros(1, 2, dtype=torch.int64)
    with pytest.raises(ValueError, match="pinned"):
        pa.pa_swap_blocks(k, v, k.clone(), v.clone(), m)
    ks2, vs2 = kv_cache_shapes(4, 2, 64, 8, torch.bfloat16)
    with pytest.raises(ValueError, match="block format"):
        pa.pa_swap_blocks(k, v, torch.zeros(ks2, dtype=torch.bfloat16),
                          torch.zeros(vs2, dtype=torch.bfloat16), m)
    with pytest.raises(ValueError, match="int64"):
        pa.pa_swap_blocks(k, v, k.clone(), v.clone(), m.int())


def test_append_argument_checks():
    lib = pa.load_library()
    A = ALIGNED
    args = [A, A, A, A, A, A, A, 0.1, A, 4, 32, 8, 128, 16, 16, 100, BF16, 0, None]
    assert lib.pa_decode_append(*args[:1], None, *args[2:]) == INVALID            # no k_new
    a = list(args); a[16] = F32
    assert lib.pa_decode_append(*a) == UNSUPPORTED                                  # fp32
    a = list(args); a[13] = 32
    assert lib.pa_decode_append(*a) == UNSUPPORTED                                  # block 32
    a = list(args); a[10] = 136; a[11] = 4
    assert lib.pa_decode_append(*a) == UNSUPPORTED                                  # G = 34
    a = list(args); a[1] = ctypes.c_void_p((1 << 20) + 4)
    assert lib.pa_decode_append(*a) == INVALID                                      # misaligned
    a = list(args); a[9] = 0
    assert lib.pa_decode_append(*a) == OK                                           # no sequence


def _prefill(lib, **kw):
    args = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, bt=ALIGNED, ctx=ALIGNED, qs=ALIGNED, scale=0.1,
                out=ALIGNED, S=4, T=100, MQ=50, Hq=32, Hkv=8, D=128, B=16, MB=16, NB=100,
                dtype=BF16, stream=None)
    args.update(kw)
    return lib.pa_prefill(args["q"], args["k"], args["v"], args["bt"], args["ctx"], args["qs"],
                          args["scale"], args["out"], args["S"], args["T"], args["MQ"],
                          args["Hq"], args["Hkv"], args["D"], args["B"], args["MB"], args["NB"],
                          args["dtype"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30, Hkv=8), INVALID),
    (dict(dtype=7), INVALID),
    (dict(T=-1), INVALID),
    (dict(MQ=101), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(qs=None), INVALID),
    (dict(qs=ctypes.c_void_p((1 << 20) + 2)), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(B=32), UNSUPPORTED),
    (dict(D=96), UNSUPPORTED),
    (dict(S=70000), UNSUPPORTED),
    (dict(T=10_000_000, MQ=10_000_000), UNSUPPORTED),
    (dict(S=65535, T=2_000_000, MQ=2_000_000), UNSUPPORTED),  # workgroup ids overflow int32
    (dict(S=0), OK),
    (dict(T=0, MQ=0), OK),
])
def test_prefill_argument_checks(kw, status):
    lib = pa.load_library()
    assert _prefill(lib, **kw) == status
    if status != OK:
        assert "pa_prefill" in lib.pa_last_error().decode()


def _cascade(lib, **kw):
    args = dict(q=ALIGNED, k=ALIGNED, v=ALIGNED, bt=ALIGNED, ctx=ALIGNED, gs=ALIGNED, pb=ALIGNED,
                NG=2, MG=4, scale=0.1, out=ALIGNED, S=8, Hq=32, Hkv=8, D=128, B=16, MB=16,
                NB=100, dtype=BF16, P=0, stream=None)
    args.update(kw)
    return lib.pa_decode_cascade(args["q"], args["k"], args["v"], args["bt"], args["ctx"],
                                 args["gs"], args["pb"], args["NG"], args["MG"], args["scale"],
                                 args["out"], args["S"], args["Hq"], args["Hkv"], args["D"],
                                 args["B"], args["MB"], args["NB"], args["dtype"], args["P"],
                                 args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=30, Hkv=8), INVALID),
    (dict(dtype=7), INVALID),
    (dict(NG=9), INVALID),
    (dict(NG=0), INVALID),
    (dict(MG=0), INVALID),
    (dict(MG=9), INVALID),
    (dict(P=24), INVALID),
    (dict(scale=float("inf")), INVALID),
    (dict(gs=None), INVALID),
    (dict(pb=ctypes.c_void_p((1 << 20) + 2)), INVALID),
    (dict(dtype=F32), UNSUPPORTED),
    (dict(B=8), UNSUPPORTED),
    (dict(D=80), UNSUPPORTED),
    (dict(S=0, NG=0, MG=0), OK),
])
def test_cascade_argument_checks(kw, status):
    lib = pa.load_library()
    assert _cascade(lib, **kw) == status
    if status != OK:
        assert "pa_decode_cascade" in lib.pa_last_error().decode()


def test_vkv_argument_checks():
    """The virtual-memory KV calls check their host arguments before any HIP
    call, and every call rejects a null handle."""
    lib = pa.load_library()
    h = ctypes.c_void_p(123)
    for args in [(0, 4, 1024, 8, 128, BF16, 0), (2, 0, 1024, 8, 128, BF16, 0),
                 (2, 4, 1000, 8, 128, BF16, 0), (2, 4, 1024, 8, 128, 9, 0),
                 (2, 4, 1024, 8, 12, BF16, 0), (2, 4, 1024, 8, 128, BF16, -1)]:
        assert lib.pa_vkv_create(*args, ctypes.byref(h)) == INVALID, args
        assert h.value is None
    assert lib.pa_vkv_create(2, 4, 1024, 8, 128, BF16, 0, None) == INVALID
    null = None
    r = ctypes.c_int()
    assert lib.pa_vkv_alloc_reqid(null, ctypes.byref(r)) == INVALID
    assert lib.pa_vkv_free_reqid(null, 0) == INVALID
    assert lib.pa_vkv_step(null, None) == INVALID
    assert lib.pa_vkv_reclaim(null) == INVALID
    assert lib.pa_vkv_info(null, None, None, None, None, None) == INVALID
    assert lib.pa_vkv_destroy(null) == OK
    assert lib.pa_vkv_write_kv(null, 0, A_, A_, A_, 1, None) == INVALID
    assert lib.pa_vkv_decode(null, 0, A_, A_, A_, 0.1, A_, 1, 8, 0, None) == INVALID


A_ = ALIGNED


def test_workspace_size_query():
    lib = pa.load_library()
    # 32 seqs x 32 heads x ceil(4096/256) partitions x (128 + 2) floats
    assert lib.pa_decode_workspace_bytes(32, 32, 128, 16, 256, 256) == 32 * 32 * 16 * 130 * 4
    assert lib.pa_decode_workspace_bytes(32, 32, 128, 16, 8, 256) == 0   # one partition
    assert lib.pa_decode_workspace_bytes(0, 32, 128, 16, 8, 256) == 0


def test_python_binding_maps_invalid_arguments_to_value_error():
    import torch
    k = torch.zeros(4, 2, 16, 16, 8, dtype=torch.bfloat16)
    v = torch.zeros(4, 2, 128, 16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        pa.pa_decode(torch.zeros(1, 3, 128, dtype=torch.bfloat16), k, v,
                     torch.zeros(1, 4, dtype=torch.int32), torch.zeros(1, dtype=torch.int32),
                     0.1, torch.zeros(1, 3, 128, dtype=torch.bfloat16))


def test_pa_debug_environment_variable():
    """PA_DEBUG=1 in the environment switches the checks on when the library
    first needs the setting; pa_set_debug returns the previous setting."""
    import subprocess
    import sys
    code = ("import ctypes, sys; lib = ctypes.CDLL(sys.argv[1]); "
            "print(lib.pa_set_debug(0), lib.pa_set_debug(1), lib.pa_set_debug(0))")
    for env_value, first in (("1", 1), ("0", 0), (None, 0)):
        env = {k: v for k, v in os.environ.items() if k != "PA_DEBUG"}
        if env_value is not None:
            env["PA_DEBUG"] = env_value
        r = subprocess.run([sys.executable, "-c", code, binding.library_path()], env=env,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        assert r.stdout.split() == [str(first), "0", "1"], (env_value, r.stdout)


@fake_pointers
def test_noalloc_rejects_a_workspace_past_its_static_array():
    """pa_decode_noalloc refuses, before anything else, partials that would
    not fit its 32 MiB static array; sizes that fit pass the same check."""
    lib = pa.load_library()
    A = ALIGNED
    # 4 sequences x 32 heads x 2^16 partitions of 16 tokens: ~4.4 GB of partials
    rc = lib.pa_decode_noalloc(A, A, A, A, A, 0.1, A, 4, 32, 8, 128, 16, 65536, 100, BF16, 16,
                               0, None)
    assert rc == UNSUPPORTED and "static workspace" in lib.pa_last_error().decode()
    # the same arguments are fine for pa_decode_ex's size checks: it would
    # allocate (not called here past its checks: num_seqs = 0 returns first)
    assert lib.pa_decode_noalloc(A, A, A, A, A, 0.1, A, 0, 32, 8, 128, 16, 65536, 100, BF16, 16,
                                 0, None) == OK


def test_merge_mode_query():
    """pa_decode_merge_mode: argument checks, and the cases that need no device."""
    import torch
    lib = pa.load_library()
    # bad arguments: -(status)
    assert lib.pa_decode_merge_mode(4, 32, 8, 128, 16, 10, 9, 0, 0) == -INVALID   # dtype
    assert lib.pa_decode_merge_mode(4, 30, 8, 128, 16, 10, BF16, 0, 0) == -INVALID  # Hq % Hkv
    assert lib.pa_decode_merge_mode(4, 32, 8, 128, 16, 10, BF16, 24, 0) == -INVALID  # P
    assert lib.pa_decode_merge_mode(4, 32, 8, 128, 16, 10, BF16, 0, 8) == -INVALID  # flags
    with pytest.raises(ValueError):
        pa.pa_decode_merge_mode(4, 32, 8, 128, 16, 10, torch.bfloat16, partition_tokens=24)
    # tables of 160 tokens fit one partition; no sequences; the merge kernel asked for
    assert pa.pa_decode_merge_mode(4, 32, 8, 128, 16, 10, torch.bfloat16) == pa.PA_MERGE_NONE
    assert pa.pa_decode_merge_mode(0, 32, 8, 128, 16, 256, torch.bfloat16, 256) == \
        pa.PA_MERGE_NONE
    assert pa.pa_decode_merge_mode(32, 32, 8, 128, 16, 256, torch.bfloat16, 640,
                                   merge_kernel=True) == pa.PA_MERGE_KERNEL
    # no in-kernel merge for: more than 8 partitions; kv heads not a multiple of 8;
    # fp32 (VALU kernel); block size 32; more than 2,048 units
    for args in [(32, 32, 8, 128, 16, 256, torch.bfloat16, 256),
                 (32, 32, 4, 128, 16, 256, torch.bfloat16, 640),
                 (32, 32, 8, 128, 16, 256, torch.float32, 640),
                 (32, 32, 8, 128, 32, 128, torch.bfloat16, 640),
                 (64, 32, 8, 128, 16, 256, torch.bfloat16, 640)]:
        assert pa.pa_decode_merge_mode(*args) == pa.PA_MERGE_KERNEL, args
