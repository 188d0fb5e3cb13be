"""Paged decode attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library libpa.so (hand-written HIP kernels);
this package is the argument-marshalling layer above it plus host-side
helpers (storage format, block manager, seeded workloads).
"""
from .layout import kv_cache_shapes, k_chunk, DTYPE_CODES  # noqa: F401
from .binding import (  # noqa: F401
    pa_write_kv, pa_decode, pa_decode_noalloc, pa_decode_plan, pa_decode_merge_mode,
    pa_read_tiles, pa_decode_append,
    pa_decode_cascade,
    pa_prefill, pa_copy_blocks, pa_swap_blocks, pa_status_str, pa_set_debug, library_path,
    load_library,
    VirtualKV, PAError, PA_MERGE_NONE, PA_MERGE_KERNEL, PA_MERGE_IN_KERNEL,
)
