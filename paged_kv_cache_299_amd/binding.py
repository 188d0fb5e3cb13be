"""Python binding of libpa: argument marshalling only.

Each function takes torch tensors, checks what the C ABI needs (device,
dtype, contiguity, shapes), and calls the entry point of the same name in
libpa.so through ctypes.  All computation happens in the HIP kernels; there is
no fallback.  If libpa.so is missing, loading raises.

Shapes (see layout.py for the pool format):
  pa_write_kv(k_new [T,Hkv,D], v_new [T,Hkv,D], k_cache, v_cache, slot_mapping int64 [T])
  pa_decode(q [S,Hq,D], k_cache, v_cache, block_tables int32 [S,MB], context_lens int32 [S],
            scale, out [S,Hq,D], stream=None, partition_tokens=0, shared_blocks=False)
    (calls pa_decode, or pa_decode_ex when a partition length, the
    PA_DECODE_SHARED_BLOCKS hint (shared_blocks) or PA_DECODE_FORCE_VALU
    (force_valu: the VALU kernel on 16-bit data, for measurement) or
    PA_DECODE_MERGE_KERNEL (merge_kernel: the separate merge kernel) is given)
  pa_decode_cascade(q, k_cache, v_cache, block_tables, context_lens, group_start int32 [NG+1],
                    prefix_blocks int32 [NG], scale, out, max_group_size=None)
  pa_prefill(q [T,Hq,D], k_cache, v_cache, block_tables int32 [S,MB], context_lens int32 [S],
             query_start int32 [S+1], scale, out [T,Hq,D], max_query_len=None)
  pa_copy_blocks(k_cache, v_cache, block_mapping int64 [n,2])
  pa_swap_blocks(src_k, src_v, dst_k, dst_v, block_mapping int64 [n,2])
    (each tensor on the GPU or in pinned host memory)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .layout import DTYPE_CODES, k_chunk

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY names another build of the same sources (the host-sanitizer run uses it)
_LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")
_lib = None

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP, PA_ERR_NO_MEMORY = range(5)
PA_DECODE_SHARED_BLOCKS = 1
PA_DECODE_FORCE_VALU = 2
PA_DECODE_MERGE_KERNEL = 4
PA_MERGE_NONE, PA_MERGE_KERNEL, PA_MERGE_IN_KERNEL = 0, 1, 2

# every symbol include/pa.h declares
EXPORTS = (
    "pa_write_kv", "pa_decode", "pa_decode_ex", "pa_decode_noalloc", "pa_read_tiles",
    "pa_decode_append",
    "pa_decode_cascade",
    "pa_prefill",
    "pa_copy_blocks", "pa_swap_blocks",
    "pa_vkv_create", "pa_vkv_info", "pa_vkv_layer", "pa_vkv_alloc_reqid", "pa_vkv_step",
    "pa_vkv_free_reqid", "pa_vkv_reclaim", "pa_vkv_destroy", "pa_vkv_write_kv", "pa_vkv_decode",
    "pa_status_str",
    "pa_last_error", "pa_decode_plan", "pa_decode_merge_mode", "pa_decode_workspace_bytes",
    "pa_release_workspaces",
    "pa_version", "pa_set_debug",
)


class PAError(RuntimeError):
    """A non-OK status from libpa."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libpa.so (built by `python -m paged_kv_cache_299_amd.build`)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_299_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    lib.pa_write_kv.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I64, I32, P]
    lib.pa_write_kv.restype = I32
    lib.pa_decode.argtypes = [P, P, P, P, P, F32, P, I32, I32, I32, I32, I32, I32, I64, I32, P]
    lib.pa_decode.restype = I32
    lib.pa_decode_ex.argtypes = [P, P, P, P, P, F32, P, I32, I32, I32, I32, I32, I32, I64, I32,
                                 I32, I32, P]
    lib.pa_decode_ex.restype = I32
    lib.pa_decode_noalloc.argtypes = lib.pa_decode_ex.argtypes
    lib.pa_decode_noalloc.restype = I32
    lib.pa_read_tiles.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, I32, I64, I32, I32, P]
    lib.pa_read_tiles.restype = I32
    lib.pa_copy_blocks.argtypes = [P, P, P, I64, I32, I32, I32, I64, I32, P]
    lib.pa_copy_blocks.restype = I32
    PP, PI64, PD = ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(I64), ctypes.POINTER(ctypes.c_double)
    lib.pa_vkv_create.argtypes = [I32, I32, I32, I32, I32, I32, I64, PP]
    lib.pa_vkv_info.argtypes = [P, PI64, PI64, PI64, PD, PD]
    lib.pa_vkv_layer.argtypes = [P, I32, PP, PP]
    lib.pa_vkv_alloc_reqid.argtypes = [P, ctypes.POINTER(I32)]
    lib.pa_vkv_step.argtypes = [P, P]
    lib.pa_vkv_free_reqid.argtypes = [P, I32]
    lib.pa_vkv_reclaim.argtypes = [P]
    lib.pa_vkv_destroy.argtypes = [P]
    lib.pa_vkv_write_kv.argtypes = [P, I32, P, P, P, I64, P]
    lib.pa_vkv_decode.argtypes = [P, I32, P, P, P, F32, P, I32, I32, I32, P]
    for name in ("pa_vkv_create", "pa_vkv_info", "pa_vkv_layer", "pa_vkv_alloc_reqid",
                 "pa_vkv_step", "pa_vkv_free_reqid", "pa_vkv_reclaim", "pa_vkv_destroy",
                 "pa_vkv_write_kv", "pa_vkv_decode"):
        getattr(lib, name).restype = I32
    lib.pa_decode_append.argtypes = [P, P, P, P, P, P, P, F32, P, I32, I32, I32, I32, I32, I32,
                                     I64, I32, I32, P]
    lib.pa_decode_append.restype = I32
    lib.pa_decode_cascade.argtypes = [P, P, P, P, P, P, P, I32, I32, F32, P, I32, I32, I32, I32,
                                      I32, I32, I64, I32, I32, P]
    lib.pa_decode_cascade.restype = I32
    lib.pa_prefill.argtypes = [P, P, P, P, P, P, F32, P, I32, I32, I32, I32, I32, I32, I32, I32,
                               I64, I32, P]
    lib.pa_prefill.restype = I32
    lib.pa_swap_blocks.argtypes = [P, P, P, P, P, I64, I32, I32, I32, I64, I64, I32, P]
    lib.pa_swap_blocks.restype = I32
    lib.pa_status_str.argtypes = [I32]
    lib.pa_status_str.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_decode_plan.argtypes = [P, I32, I32, I32, I32, I32, I32, ctypes.POINTER(I32)]
    lib.pa_decode_plan.restype = I32
    lib.pa_decode_merge_mode.argtypes = [I32] * 9
    lib.pa_decode_merge_mode.restype = I32
    lib.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pa_decode_workspace_bytes.restype = I64
    lib.pa_release_workspaces.argtypes = []
    lib.pa_release_workspaces.restype = I32
    lib.pa_version.argtypes = []
    lib.pa_version.restype = I32
    lib.pa_set_debug.argtypes = [I32]
    lib.pa_set_debug.restype = I32
    _lib = lib
    return lib


def pa_status_str(status: int) -> str:
    return load_library().pa_status_str(status).decode()


def pa_set_debug(on: bool) -> bool:
    """PA_DEBUG on or off (device-side precondition checks before every call,
    ValueError on a violation); returns the previous setting."""
    return bool(load_library().pa_set_debug(1 if on else 0))


def _check(rc: int, what: str) -> None:
    if rc == PA_OK:
        return
    lib = load_library()
    msg = f"{what}: {lib.pa_status_str(rc).decode()}: {lib.pa_last_error().decode()}"
    if rc == PA_ERR_INVALID_ARG:
        raise ValueError(msg)
    raise PAError(rc, msg)


def _stream_handle(stream, device) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _cache_dims(k_cache: torch.Tensor, v_cache: torch.Tensor, on_gpu: bool = True):
    _need(k_cache.dim() == 5 and v_cache.dim() == 4,
          "k_cache must be [NB, Hkv, D/x, B, x] and v_cache [NB, Hkv, D, B]")
    NB, Hkv, DX, B, X = k_cache.shape
    _need(X == k_chunk(k_cache.dtype), f"k_cache last dim must be {k_chunk(k_cache.dtype)}")
    D = DX * X
    _need(tuple(v_cache.shape) == (NB, Hkv, D, B), "v_cache shape does not match k_cache")
    _need(k_cache.dtype == v_cache.dtype, "k_cache and v_cache dtypes differ")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    if on_gpu:
        _need(k_cache.is_cuda and v_cache.device == k_cache.device, "caches must be on one GPU")
    return NB, Hkv, D, B


def _reachable(t: torch.Tensor, name: str) -> None:
    _need(t.is_cuda or (t.device.type == "cpu" and t.is_pinned()),
          f"{name} must be on the GPU or in pinned host memory")


def pa_write_kv(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, slot_mapping: torch.Tensor, stream=None) -> None:
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    _need(k_new.shape == v_new.shape and k_new.dim() == 3 and tuple(k_new.shape[1:]) == (Hkv, D),
          "k_new / v_new must be [T, Hkv, D]")
    _need(k_new.dtype == k_cache.dtype == v_new.dtype, "new tokens and caches differ in dtype")
    _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
          and slot_mapping.shape[0] == k_new.shape[0], "slot_mapping must be int64 [T]")
    for t in (k_new, v_new, slot_mapping):
        _need(t.is_contiguous() and t.device == k_cache.device, "inputs must be contiguous, same GPU")
    rc = load_library().pa_write_kv(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(slot_mapping), k_new.shape[0], Hkv, D, B, NB,
                                    DTYPE_CODES[k_cache.dtype],
                                    _stream_handle(stream, k_cache.device))
    _check(rc, "pa_write_kv")


def pa_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
              out: torch.Tensor, stream=None, partition_tokens: Optional[int] = 0,
              shared_blocks: bool = False, force_valu: bool = False,
              merge_kernel: bool = False) -> None:
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == D, "q must be [S, Hq, D]")
    _need(out.shape == q.shape and out.dtype == q.dtype == k_cache.dtype,
          "out must match q, and q must match the caches' dtype")
    S, Hq = q.shape[0], q.shape[1]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    for t in (q, out, block_tables, context_lens):
        _need(t.is_contiguous() and t.device == k_cache.device, "inputs must be contiguous, same GPU")
    lib = load_library()
    if not (partition_tokens or shared_blocks or force_valu or merge_kernel):  # the plain entry
        rc = lib.pa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                           _ptr(context_lens), float(scale), _ptr(out), S, Hq, Hkv, D, B,
                           block_tables.shape[1], NB, DTYPE_CODES[q.dtype],
                           _stream_handle(stream, q.device))
    else:
        rc = lib.pa_decode_ex(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                              _ptr(context_lens), float(scale), _ptr(out), S, Hq, Hkv, D, B,
                              block_tables.shape[1], NB, DTYPE_CODES[q.dtype],
                              int(partition_tokens or 0),
                              (PA_DECODE_SHARED_BLOCKS if shared_blocks else 0)
                              | (PA_DECODE_FORCE_VALU if force_valu else 0)
                              | (PA_DECODE_MERGE_KERNEL if merge_kernel else 0),
                              _stream_handle(stream, q.device))
    _check(rc, "pa_decode")


def pa_decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor, scale: float,
                      out: torch.Tensor, stream=None, partition_tokens: int = 0,
                      shared_blocks: bool = False) -> None:
    """pa_decode_ex that allocates nothing: partials in the library's static
    per-GPU array (calls on one GPU must not overlap in time)."""
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == D, "q must be [S, Hq, D]")
    _need(out.shape == q.shape and out.dtype == q.dtype == k_cache.dtype,
          "out must match q, and q must match the caches' dtype")
    S, Hq = q.shape[0], q.shape[1]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,),
          "context_lens must be int32 [S]")
    for t in (q, out, block_tables, context_lens):
        _need(t.is_contiguous() and t.device == k_cache.device, "inputs must be contiguous, same GPU")
    rc = load_library().pa_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        float(scale), _ptr(out), S, Hq, Hkv, D, B, block_tables.shape[1], NB,
        DTYPE_CODES[q.dtype], int(partition_tokens or 0),
        PA_DECODE_SHARED_BLOCKS if shared_blocks else 0, _stream_handle(stream, q.device))
    _check(rc, "pa_decode_noalloc")


def pa_decode_plan(context_lens, num_heads: int, num_kv_heads: int, block_size: int,
                   max_blocks_per_seq: int, dtype: torch.dtype) -> int:
    """Partition length for pa_decode from host-side context lengths (0: the
    library's automatic choice)."""
    cl = torch.as_tensor(context_lens, dtype=torch.int32).cpu().contiguous()
    _need(cl.dim() == 1, "context_lens must be one-dimensional")
    out = ctypes.c_int(0)
    rc = load_library().pa_decode_plan(ctypes.c_void_p(cl.data_ptr()), cl.shape[0],
                                       int(num_heads), int(num_kv_heads), int(block_size),
                                       int(max_blocks_per_seq), DTYPE_CODES[dtype],
                                       ctypes.byref(out))
    _check(rc, "pa_decode_plan")
    return int(out.value)


def pa_decode_merge_mode(num_seqs: int, num_heads: int, num_kv_heads: int, head_dim: int,
                         block_size: int, max_blocks_per_seq: int, dtype: torch.dtype,
                         partition_tokens: int = 0, shared_blocks: bool = False,
                         force_valu: bool = False, merge_kernel: bool = False) -> int:
    """How pa_decode merges split contexts for these sizes on the current device:
    PA_MERGE_NONE, PA_MERGE_KERNEL or PA_MERGE_IN_KERNEL."""
    flags = ((PA_DECODE_SHARED_BLOCKS if shared_blocks else 0)
             | (PA_DECODE_FORCE_VALU if force_valu else 0)
             | (PA_DECODE_MERGE_KERNEL if merge_kernel else 0))
    r = load_library().pa_decode_merge_mode(int(num_seqs), int(num_heads), int(num_kv_heads),
                                            int(head_dim), int(block_size),
                                            int(max_blocks_per_seq), DTYPE_CODES[dtype],
                                            int(partition_tokens or 0), flags)
    if r < 0:
        _check(-r, "pa_decode_merge_mode")
    return int(r)


def pa_read_tiles(k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                  context_lens: torch.Tensor, sink: torch.Tensor, num_heads: int, stream=None,
                  partition_tokens: Optional[int] = 0) -> None:
    """Measurement aid: the K/V reads of pa_decode for these arguments, nothing else."""
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    S = context_lens.shape[0] if context_lens.dim() == 1 else -1
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S, "block_tables must be int32 [S, MB]")
    _need(context_lens.dtype == torch.int32, "context_lens must be int32 [S]")
    _need(sink.dtype == torch.int32 and sink.numel() >= 1, "sink must be an int32 tensor")
    for t in (block_tables, context_lens, sink):
        _need(t.is_contiguous() and t.device == k_cache.device, "inputs must be contiguous, same GPU")
    rc = load_library().pa_read_tiles(_ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                      _ptr(context_lens), _ptr(sink), S, int(num_heads), Hkv, D,
                                      B, block_tables.shape[1], NB, DTYPE_CODES[k_cache.dtype],
                                      int(partition_tokens or 0),
                                      _stream_handle(stream, k_cache.device))
    _check(rc, "pa_read_tiles")


def pa_decode_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     k_cache: torch.Tensor, v_cache: torch.Tensor, block_tables: torch.Tensor,
                     context_lens: torch.Tensor, scale: float, out: torch.Tensor,
                     partition_tokens: int = 0, stream=None) -> None:
    """Store each sequence's newest token (position context_lens[s] - 1; k_new /
    v_new [S, Hkv, D]) into its slot and decode, in one call."""
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    S = q.shape[0]
    _need(q.dim() == 3 and q.shape[2] == D and q.shape == out.shape,
          "q and out must be [S, Hq, D] with the caches' D")
    _need(tuple(k_new.shape) == (S, Hkv, D) and k_new.shape == v_new.shape,
          "k_new / v_new must be [S, Hkv, D]")
    _need(q.dtype == k_new.dtype == v_new.dtype == k_cache.dtype == out.dtype,
          "q, new tokens, caches and out differ in dtype")
    for t in (q, out, k_new, v_new):
        _need(t.is_contiguous() and t.device == k_cache.device,
              "q, out and new tokens must be contiguous on the caches' GPU")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S and block_tables.is_contiguous()
          and block_tables.device == k_cache.device, "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,)
          and context_lens.is_contiguous() and context_lens.device == k_cache.device,
          "context_lens must be contiguous int32 [S]")
    rc = load_library().pa_decode_append(
        _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), _ptr(out), S, q.shape[1], Hkv, D, B,
        block_tables.shape[1], NB, DTYPE_CODES[q.dtype], int(partition_tokens),
        _stream_handle(stream, k_cache.device))
    _check(rc, "pa_decode_append")


def pa_decode_cascade(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      block_tables: torch.Tensor, context_lens: torch.Tensor,
                      group_start: torch.Tensor, prefix_blocks: torch.Tensor, scale: float,
                      out: torch.Tensor, max_group_size: Optional[int] = None,
                      partition_tokens: int = 0, stream=None) -> None:
    """pa_decode with the first prefix_blocks[i] blocks of the sequences of
    group i (group_start[i] .. group_start[i+1]-1) read once for the group.
    max_group_size: a bound on the members of a group; None reads it from
    group_start (a device-to-host copy)."""
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    S, Hq = q.shape[0], q.shape[1]
    _need(q.dim() == 3 and q.shape[2] == D and q.shape == out.shape,
          "q and out must be [S, Hq, D] with the caches' D")
    _need(q.dtype == k_cache.dtype == out.dtype, "q, caches and out differ in dtype")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and tuple(context_lens.shape) == (S,)
          and context_lens.is_contiguous(), "context_lens must be contiguous int32 [S]")
    NG = prefix_blocks.shape[0]
    _need(group_start.dtype == torch.int32 and tuple(group_start.shape) == (NG + 1,)
          and group_start.is_contiguous(), "group_start must be contiguous int32 [NG + 1]")
    _need(prefix_blocks.dtype == torch.int32 and prefix_blocks.dim() == 1
          and prefix_blocks.is_contiguous(), "prefix_blocks must be contiguous int32 [NG]")
    for t in (q, out, block_tables, context_lens, group_start, prefix_blocks):
        _need(t.device == k_cache.device, "all tensors must be on the caches' GPU")
    if max_group_size is None:
        max_group_size = int((group_start[1:] - group_start[:-1]).max().item()) if NG else 0
    rc = load_library().pa_decode_cascade(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        _ptr(group_start), _ptr(prefix_blocks), NG, int(max_group_size), float(scale), _ptr(out),
        S, Hq, Hkv, D, B, block_tables.shape[1], NB, DTYPE_CODES[q.dtype], int(partition_tokens),
        _stream_handle(stream, k_cache.device))
    _check(rc, "pa_decode_cascade")


def pa_prefill(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               block_tables: torch.Tensor, context_lens: torch.Tensor, query_start: torch.Tensor,
               scale: float, out: torch.Tensor, max_query_len: Optional[int] = None,
               stream=None) -> None:
    """Causal attention of each sequence's new queries (rows query_start[s] ..
    query_start[s+1]-1 of q) over its context_lens[s] tokens in the pool.
    max_query_len: a bound on the queries per sequence; None reads it from
    query_start (a device-to-host copy)."""
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == D and q.shape == out.shape,
          "q and out must be [T, Hq, D] with the caches' D")
    _need(q.dtype == k_cache.dtype == out.dtype, "q, caches and out differ in dtype")
    _need(q.is_contiguous() and out.is_contiguous(), "q and out must be contiguous")
    S = context_lens.shape[0]
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == S and block_tables.is_contiguous(),
          "block_tables must be contiguous int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.is_contiguous(),
          "context_lens must be contiguous int32 [S]")
    _need(query_start.dtype == torch.int32 and tuple(query_start.shape) == (S + 1,)
          and query_start.is_contiguous(), "query_start must be contiguous int32 [S + 1]")
    for t in (q, out, block_tables, context_lens, query_start):
        _need(t.device == k_cache.device, "all tensors must be on the caches' GPU")
    if max_query_len is None:
        max_query_len = int((query_start[1:] - query_start[:-1]).max().item()) if S else 0
    rc = load_library().pa_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                                   _ptr(context_lens), _ptr(query_start), float(scale), _ptr(out),
                                   S, q.shape[0], int(max_query_len), q.shape[1], Hkv, D, B,
                                   block_tables.shape[1], NB, DTYPE_CODES[q.dtype],
                                   _stream_handle(stream, k_cache.device))
    _check(rc, "pa_prefill")


def pa_copy_blocks(k_cache: torch.Tensor, v_cache: torch.Tensor, block_mapping: torch.Tensor,
                   stream=None) -> None:
    NB, Hkv, D, B = _cache_dims(k_cache, v_cache)
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2, "block_mapping must be int64 [n, 2]")
    _need(block_mapping.is_contiguous() and block_mapping.device == k_cache.device,
          "block_mapping must be contiguous on the caches' GPU")
    rc = load_library().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                                       block_mapping.shape[0], Hkv, D, B, NB,
                                       DTYPE_CODES[k_cache.dtype],
                                       _stream_handle(stream, k_cache.device))
    _check(rc, "pa_copy_blocks")


def pa_swap_blocks(src_k: torch.Tensor, src_v: torch.Tensor, dst_k: torch.Tensor,
                   dst_v: torch.Tensor, block_mapping: torch.Tensor, stream=None) -> None:
    """Block src of (src_k, src_v) -> block dst of (dst_k, dst_v) for each
    (src, dst) row of block_mapping; pools on the GPU or in pinned host memory."""
    NS, Hkv, D, B = _cache_dims(src_k, src_v, on_gpu=False)
    ND, Hkv2, D2, B2 = _cache_dims(dst_k, dst_v, on_gpu=False)
    _need((Hkv, D, B) == (Hkv2, D2, B2) and src_k.dtype == dst_k.dtype,
          "source and destination pools differ in block format")
    _need(block_mapping.dtype == torch.int64 and block_mapping.dim() == 2
          and block_mapping.shape[1] == 2 and block_mapping.is_contiguous(),
          "block_mapping must be contiguous int64 [n, 2]")
    tensors = dict(src_k=src_k, src_v=src_v, dst_k=dst_k, dst_v=dst_v,
                   block_mapping=block_mapping)
    gpus = {t.device for t in tensors.values() if t.is_cuda}
    _need(len(gpus) <= 1, "GPU tensors must be on one device")
    for name, t in tensors.items():
        _reachable(t, name)
    device = gpus.pop() if gpus else torch.device("cuda", torch.cuda.current_device())
    with torch.cuda.device(device):
        rc = load_library().pa_swap_blocks(_ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v),
                                           _ptr(block_mapping), block_mapping.shape[0], Hkv, D,
                                           B, NS, ND, DTYPE_CODES[src_k.dtype],
                                           _stream_handle(stream, device))
    _check(rc, "pa_swap_blocks")


class VirtualKV:
    """KV storage on HIP virtual memory (pa_vkv_*): one contiguous virtual
    range per request slot, physical pages mapped as sequences grow."""

    def __init__(self, num_layers: int, max_batch: int, max_context_len: int, num_kv_heads: int,
                 head_dim: int, dtype: torch.dtype, page_bytes: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.pa_vkv_create(num_layers, max_batch, max_context_len, num_kv_heads, head_dim,
                                 DTYPE_CODES[dtype], int(page_bytes), ctypes.byref(h)),
               "pa_vkv_create")
        self._h = h
        self.num_layers, self.max_batch, self.max_context_len = num_layers, max_batch, \
            max_context_len
        self.num_kv_heads, self.head_dim, self.dtype = num_kv_heads, head_dim, dtype
        info = self.info()
        self.page_bytes = info["page_bytes"]
        self.request_stride_blocks = info["request_stride_blocks"]

    def _handle(self):
        if self._h is None:
            raise ValueError("VirtualKV is closed")
        return self._h

    def info(self) -> dict:
        pb, rs, mb = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        cu, mu = ctypes.c_double(), ctypes.c_double()
        _check(load_library().pa_vkv_info(self._handle(), ctypes.byref(pb), ctypes.byref(rs),
                                          ctypes.byref(mb), ctypes.byref(cu), ctypes.byref(mu)),
               "pa_vkv_info")
        return {"page_bytes": pb.value, "request_stride_blocks": rs.value,
                "mapped_bytes": mb.value, "create_us_per_page": cu.value,
                "map_us_per_page": mu.value}

    def layer(self, layer: int):
        k, v = ctypes.c_void_p(), ctypes.c_void_p()
        _check(load_library().pa_vkv_layer(self._handle(), layer, ctypes.byref(k),
                                           ctypes.byref(v)), "pa_vkv_layer")
        return k.value, v.value

    def alloc_reqid(self) -> int:
        r = ctypes.c_int()
        _check(load_library().pa_vkv_alloc_reqid(self._handle(), ctypes.byref(r)),
               "pa_vkv_alloc_reqid")
        return r.value

    def step(self, seq_lens) -> None:
        lens = (ctypes.c_int32 * self.max_batch)(*[int(x) for x in seq_lens])
        _need(len(seq_lens) == self.max_batch, "seq_lens needs one entry per request slot")
        _check(load_library().pa_vkv_step(self._handle(), lens), "pa_vkv_step")

    def free_reqid(self, req_id: int) -> None:
        _check(load_library().pa_vkv_free_reqid(self._handle(), req_id), "pa_vkv_free_reqid")

    def reclaim(self) -> None:
        _check(load_library().pa_vkv_reclaim(self._handle()), "pa_vkv_reclaim")

    def close(self) -> None:
        if self._h is not None:
            _check(load_library().pa_vkv_destroy(self._h), "pa_vkv_destroy")
            self._h = None

    def slot(self, req_id: int, position: int) -> int:
        """The slot of position `position` of request slot `req_id`."""
        return req_id * self.request_stride_blocks * 16 + position

    def write_kv(self, layer: int, k_new: torch.Tensor, v_new: torch.Tensor,
                 slot_mapping: torch.Tensor, stream=None) -> None:
        _need(k_new.shape == v_new.shape and k_new.dim() == 3
              and tuple(k_new.shape[1:]) == (self.num_kv_heads, self.head_dim),
              "k_new / v_new must be [T, Hkv, D]")
        _need(k_new.dtype == v_new.dtype == self.dtype, "new tokens differ in dtype")
        _need(k_new.is_cuda and k_new.is_contiguous() and v_new.is_contiguous(),
              "new tokens must be contiguous on the GPU")
        _need(slot_mapping.dtype == torch.int64 and slot_mapping.dim() == 1
              and slot_mapping.shape[0] == k_new.shape[0] and slot_mapping.is_contiguous(),
              "slot_mapping must be contiguous int64 [T]")
        _check(load_library().pa_vkv_write_kv(self._handle(), layer, _ptr(k_new), _ptr(v_new),
                                              _ptr(slot_mapping), k_new.shape[0],
                                              _stream_handle(stream, k_new.device)),
               "pa_vkv_write_kv")

    def decode(self, layer: int, q: torch.Tensor, req_ids: torch.Tensor,
               context_lens: torch.Tensor, scale: float, out: torch.Tensor,
               partition_tokens: int = 0, stream=None) -> None:
        _need(q.dim() == 3 and q.shape[2] == self.head_dim and q.shape == out.shape,
              "q and out must be [S, Hq, D]")
        _need(q.dtype == out.dtype == self.dtype, "q and out differ in dtype")
        _need(q.is_cuda and q.is_contiguous() and out.is_contiguous(), "q and out: contiguous GPU")
        S = q.shape[0]
        for t, name in ((req_ids, "req_ids"), (context_lens, "context_lens")):
            _need(t.dtype == torch.int32 and tuple(t.shape) == (S,) and t.is_contiguous()
                  and t.device == q.device, f"{name} must be contiguous int32 [S] on q's GPU")
        _check(load_library().pa_vkv_decode(self._handle(), layer, _ptr(q), _ptr(req_ids),
                                            _ptr(context_lens), float(scale), _ptr(out), S,
                                            q.shape[1], int(partition_tokens),
                                            _stream_handle(stream, q.device)),
               "pa_vkv_decode")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
