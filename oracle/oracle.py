"""ctypes front end of the C oracle (oracle/pa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the GPU library.

Arrays are numpy arrays.  16-bit element types are passed as raw bits:
float16 data as numpy.float16 (or uint16 bits), bfloat16 data as numpy.uint16
bit patterns.  Outputs of decode are float64.

Storage format (same definition the library documents):
  K pool  [NB][Hkv][D/x][B][x], x = k_x elements
  V pool  [NB][Hkv][D][B]
"""
import ctypes
import os

import numpy as np

F32, F16, BF16 = 0, 1, 2
_ELEM = {F32: 4, F16: 2, BF16: 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIBRARY names another build of the same source (the sanitizer run uses it)
_LIB_PATH = os.environ.get("ORACLE_LIBRARY") or os.path.join(_HERE, "liboracle.so")
_lib = None

_ERRORS = {
    -1: "bad dimensions",
    -2: "bad dtype",
    -3: "context length out of range",
    -4: "block id out of range",
    -5: "slot out of range",
    -6: "duplicate slot",
    -7: "bad copy pair (range, duplicate dst, or dst that is also a src)",
    -8: "out of memory",
}


class OracleError(ValueError):
    """A broken precondition reported by the oracle."""


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_decode.argtypes = [P, P, P, P, P, D, P, I64, I64, I64, I64, I64, I64, I64, I64, I32]
    lib.oracle_decode.restype = I32
    lib.oracle_decode_partitioned.argtypes = [P, P, P, P, P, D, P, I64, I64, I64, I64, I64, I64,
                                              I64, I64, I32, I64, P, P, P]
    lib.oracle_decode_partitioned.restype = I32
    lib.oracle_prefill.argtypes = [P, P, P, P, P, P, D, P, I64, I64, I64, I64, I64, I64, I64,
                                   I64, I64, I32]
    lib.oracle_prefill.restype = I32
    lib.oracle_write_kv.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, I32]
    lib.oracle_write_kv.restype = I32
    lib.oracle_copy_blocks.argtypes = [P, P, P, I64, I64, I64, I64, I64, I32]
    lib.oracle_copy_blocks.restype = I32
    lib.oracle_swap_blocks.argtypes = [P, P, P, P, P, I64, I64, I64, I64, I64, I64, I32]
    lib.oracle_swap_blocks.restype = I32
    lib.oracle_kv_cache_bytes.argtypes = [I64, I64, I64, I64, I64]
    lib.oracle_kv_cache_bytes.restype = I64
    lib.oracle_blocks_for_tokens.argtypes = [I64, I64]
    lib.oracle_blocks_for_tokens.restype = I64
    lib.oracle_slot_of.argtypes = [P, I64, I64]
    lib.oracle_slot_of.restype = I64
    lib.oracle_f16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_double.restype = D
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = D
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = I32
    lib.oracle_set_num_threads.argtypes = [I32]
    lib.oracle_set_num_threads.restype = I32
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc):
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"oracle error {rc}"))


def _raw(a, dtype):
    """Contiguous numpy view of the element bits with the right item size."""
    a = np.ascontiguousarray(a)
    if a.dtype.itemsize != _ELEM[dtype]:
        raise OracleError(f"array itemsize {a.dtype.itemsize} does not match dtype {dtype}")
    return a


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Thread count for later oracle calls from this thread; returns the previous one."""
    if n < 1:
        raise OracleError("thread count must be >= 1")
    return int(_load().oracle_set_num_threads(int(n)))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, *, num_kv_heads, head_dim,
           block_size, k_x, dtype):
    """fp64 paged decode attention; returns float64 [S, Hq, D]."""
    lib = _load()
    q = _raw(q, dtype)
    k_cache = _raw(k_cache, dtype)
    v_cache = _raw(v_cache, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = cl.shape[0]
    D = head_dim
    Hq = q.size // max(1, S * D) if S else 1
    MB = bt.shape[1] if bt.ndim == 2 else 0
    NB = k_cache.size // (num_kv_heads * block_size * D)
    out = np.zeros((S, Hq, D), dtype=np.float64)
    rc = lib.oracle_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                           float(scale), _ptr(out), S, Hq, num_kv_heads, D, block_size, MB, NB,
                           k_x, dtype)
    _check(rc)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, *,
            num_kv_heads, head_dim, block_size, k_x, dtype):
    """fp64 paged prefill: q [T, Hq, D] packed per sequence (query_start [S+1]);
    the i-th of a sequence's n queries attends over positions 0..ctx-n+i.
    Returns float64 [T, Hq, D]."""
    lib = _load()
    q = _raw(q, dtype)
    k_cache = _raw(k_cache, dtype)
    v_cache = _raw(v_cache, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    qs = np.ascontiguousarray(query_start, dtype=np.int32)
    S = cl.shape[0]
    if qs.shape != (S + 1,):
        raise ValueError("query_start must have num_seqs + 1 entries")
    T = int(qs[-1]) if S else 0
    D = head_dim
    Hq = q.size // max(1, T * D) if T else 1
    MB = bt.shape[1] if bt.ndim == 2 else 0
    NB = k_cache.size // (num_kv_heads * block_size * D)
    out = np.zeros((T, Hq, D), dtype=np.float64)
    rc = lib.oracle_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl), _ptr(qs),
                            float(scale), _ptr(out), S, T, Hq, num_kv_heads, D, block_size, MB,
                            NB, k_x, dtype)
    _check(rc)
    return out


def decode_partitioned(q, k_cache, v_cache, block_tables, context_lens, scale, *, num_kv_heads,
                       head_dim, block_size, k_x, dtype, partition_tokens, return_parts=False):
    """fp64 attention per run of `partition_tokens` tokens merged by log-sum-exp.

    With return_parts=True also returns (m, l, o) per run, shaped
    [S, Hq, NP], [S, Hq, NP], [S, Hq, NP, D].
    """
    lib = _load()
    q = _raw(q, dtype)
    k_cache = _raw(k_cache, dtype)
    v_cache = _raw(v_cache, dtype)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S = cl.shape[0]
    D = head_dim
    Hq = q.size // max(1, S * D) if S else 1
    MB = bt.shape[1] if bt.ndim == 2 else 0
    NB = k_cache.size // (num_kv_heads * block_size * D)
    P = int(partition_tokens)
    NP = max(1, -(-MB * block_size // P)) if P > 0 else 1
    out = np.zeros((S, Hq, D), dtype=np.float64)
    pm = np.zeros((S, Hq, NP), dtype=np.float64)
    pl = np.zeros((S, Hq, NP), dtype=np.float64)
    po = np.zeros((S, Hq, NP, D), dtype=np.float64)
    rc = lib.oracle_decode_partitioned(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl),
                                       float(scale), _ptr(out), S, Hq, num_kv_heads, D,
                                       block_size, MB, NB, k_x, dtype, P, _ptr(pm), _ptr(pl),
                                       _ptr(po))
    _check(rc)
    if return_parts:
        return out, (pm, pl, po)
    return out


def write_kv(k_new, v_new, k_cache, v_cache, slot_mapping, *, num_kv_heads, head_dim,
             block_size, k_x, dtype):
    """Scatter new K/V into copies of the pools; returns (k_cache', v_cache')."""
    lib = _load()
    k_new = _raw(k_new, dtype)
    v_new = _raw(v_new, dtype)
    kc = _raw(k_cache, dtype).copy()
    vc = _raw(v_cache, dtype).copy()
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    T = sm.shape[0]
    NB = kc.size // (num_kv_heads * block_size * head_dim)
    rc = lib.oracle_write_kv(_ptr(k_new), _ptr(v_new), _ptr(kc), _ptr(vc), _ptr(sm), T,
                             num_kv_heads, head_dim, block_size, NB, k_x, dtype)
    _check(rc)
    return kc, vc


def copy_blocks(k_cache, v_cache, block_mapping, *, num_kv_heads, head_dim, block_size, dtype):
    """Copy whole blocks (src -> dst) in copies of the pools; returns (k', v')."""
    lib = _load()
    kc = _raw(k_cache, dtype).copy()
    vc = _raw(v_cache, dtype).copy()
    bm = np.ascontiguousarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    NB = kc.size // (num_kv_heads * block_size * head_dim)
    rc = lib.oracle_copy_blocks(_ptr(kc), _ptr(vc), _ptr(bm), bm.shape[0], num_kv_heads,
                                head_dim, block_size, NB, dtype)
    _check(rc)
    return kc, vc


def swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping, *, num_kv_heads, head_dim,
                block_size, dtype):
    """Copy whole blocks from the source pools into copies of the destination
    pools (src block -> dst block per pair); returns (dst_k', dst_v')."""
    lib = _load()
    sk = np.ascontiguousarray(_raw(src_k, dtype))
    sv = np.ascontiguousarray(_raw(src_v, dtype))
    dk = _raw(dst_k, dtype).copy()
    dv = _raw(dst_v, dtype).copy()
    bm = np.ascontiguousarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    per = num_kv_heads * block_size * head_dim
    rc = lib.oracle_swap_blocks(_ptr(sk), _ptr(sv), _ptr(dk), _ptr(dv), _ptr(bm), bm.shape[0],
                                num_kv_heads, head_dim, block_size, sk.size // per, dk.size // per,
                                dtype)
    _check(rc)
    return dk, dv


def kv_cache_bytes(t, L, H, D_h, elem_bytes=2):
    return int(_load().oracle_kv_cache_bytes(t, L, H, D_h, elem_bytes))


def blocks_for_tokens(T, B):
    return int(_load().oracle_blocks_for_tokens(T, B))


def slot_of(block_table_row, B, i):
    row = np.ascontiguousarray(block_table_row, dtype=np.int32)
    return int(_load().oracle_slot_of(_ptr(row), B, i))


def f16_bits_to_float64(bits):
    lib = _load()
    return np.array([lib.oracle_f16_to_double(int(b)) for b in np.asarray(bits).ravel()],
                    dtype=np.float64)


def bf16_bits_to_float64(bits):
    lib = _load()
    return np.array([lib.oracle_bf16_to_double(int(b)) for b in np.asarray(bits).ravel()],
                    dtype=np.float64)
