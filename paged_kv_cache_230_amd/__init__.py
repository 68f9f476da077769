"""MI355X-native paged KV-cache decode attention.

Python binding of ``libpagedkv.so`` (C ABI: ``include/pagedkv.h``).  The
functions below only marshal torch tensors into the library's entry points
of the same names; the HIP kernels and the C++ block manager do the work.
Importing fails if the library has not been built (no CPU fallback).
"""
from ._native import EXPORTED, LIB_PATH, PKVError, last_error  # noqa: F401
from .api import (  # noqa: F401
    BlockManager,
    RadixIndex,
    block_digest,
    device_status,
    stream_read,
    mfma_rate,
    tile_read,
    host_pools,
    new_pools,
    paged_attention_decode,
    paged_attention_decode_append,
    paged_attention_decode_append_noalloc,
    paged_attention_prefill,
    paged_attention_segment_cost,
    paged_attention_workgroups_per_head,
    paged_attention_workspace_bytes,
    paged_kv_append,
    paged_kv_copy_blocks,
    paged_kv_swap_blocks,
    pool_shapes,
)
from .cache import PagedKVCache  # noqa: F401
