"""Python binding: the C-ABI entry points with torch tensors as arguments.

Each function checks shapes/dtypes/devices of the tensors, takes their data
pointers and the current HIP stream, and calls the library function of the
same name.  No computation of the method happens here.  Pool shapes follow
the storage format of include/pagedkv.h:

    K pool: [num_blocks][num_kv_heads][head_dim // x][block_size][x]
    V pool: [num_blocks][num_kv_heads][head_dim][block_size]
    x = 16 // element size (4 for float32, 8 for bfloat16)
"""
from __future__ import annotations

import ctypes as C
import math

import numpy as np
import torch

from . import _native as N

__all__ = [
    "pool_shapes",
    "new_pools",
    "paged_kv_append",
    "paged_kv_copy_blocks",
    "paged_attention_decode",
    "paged_attention_decode_append",
    "paged_attention_decode_append_noalloc",
    "paged_attention_workspace_bytes",
    "paged_attention_workgroups_per_head",
    "paged_attention_segment_cost",
    "BlockManager",
    "device_status",
    "stream_read",
]

_DT = {torch.float32: N.PKV_F32, torch.bfloat16: N.PKV_BF16}


def _dt(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t} (float32 or bfloat16)")
    return _DT[t]


def _stream(device: torch.device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return C.c_void_p(t.data_ptr() if t is not None else 0)


def _need(t: torch.Tensor, name: str, dtype=None, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def device_status(device=None, clear: bool = True) -> int:
    """OR of the PKV_DEV_* flags kernels set on ``device`` since the last
    clear (0: every device-side index was in range); waits for the current
    stream first, and clears the word unless ``clear`` is false."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    flags = C.c_int32(0)
    with torch.cuda.device(dev):
        N.check(N.lib.pkv_device_status(_stream(dev), 1 if clear else 0, C.byref(flags)))
    return int(flags.value)


def stream_read(buf: torch.Tensor, sink: torch.Tensor):
    """Read the whole of ``buf`` (a contiguous device tensor, 16-byte aligned,
    a multiple of 16 bytes) once with the library's streaming probe on the
    current stream; ``sink`` (device int32) receives one word per
    workgroup."""
    dev = buf.device
    _need(sink, "sink", torch.int32, dev, 1)
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    N.check(N.lib.pkv_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                  _stream(dev)))


def tile_read(pool: torch.Tensor, tile_bytes: int, ids: torch.Tensor, sink: torch.Tensor):
    """Read the tiles ``pool`` + ids[i] * tile_bytes (``pool`` a contiguous
    device tensor; ``ids`` device int32, clamped to the pool's tiles) once
    with the library's tile probe on the current stream; ``sink`` (device
    int32) receives one word per workgroup."""
    dev = pool.device
    _need(ids, "ids", torch.int32, dev, 1)
    _need(sink, "sink", torch.int32, dev, 1)
    if not pool.is_contiguous():
        raise ValueError("pool must be contiguous")
    nbytes = pool.numel() * pool.element_size()
    if tile_bytes <= 0 or nbytes < tile_bytes:
        raise ValueError(f"tile_bytes {tile_bytes} does not fit a pool of {nbytes} bytes")
    N.check(N.lib.pkv_tile_read(_ptr(pool), tile_bytes, nbytes // tile_bytes, _ptr(ids), ids.numel(), _ptr(sink),
                                sink.numel(), _stream(dev)))


def mfma_rate(sink: torch.Tensor, workgroups: int, iters: int) -> int:
    """Run the library's matrix-core probe on the current stream:
    ``workgroups`` workgroups of 8 waves, each wave issuing ``iters`` x 16
    bf16 32x32x16 products; ``sink`` (device float32, at least
    ``workgroups * 512`` elements) receives one value per thread.  Returns
    the flops issued."""
    dev = sink.device
    _need(sink, "sink", torch.float32, dev, 1)
    if sink.numel() < workgroups * 512:
        raise ValueError(f"sink holds {sink.numel()} floats, needs {workgroups * 512}")
    N.check(N.lib.pkv_mfma_rate(_ptr(sink), workgroups, iters, _stream(dev)))
    return workgroups * 8 * iters * 16 * 32768


def pool_shapes(num_blocks, num_kv_heads, head_dim, block_size, dtype):
    x = 16 // torch.empty((), dtype=dtype).element_size()
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x), (num_blocks, num_kv_heads, head_dim, block_size))


def new_pools(num_blocks, num_kv_heads, head_dim, block_size, dtype, device="cuda"):
    ks, vs = pool_shapes(num_blocks, num_kv_heads, head_dim, block_size, dtype)
    return torch.zeros(ks, dtype=dtype, device=device), torch.zeros(vs, dtype=dtype, device=device)


def host_pools(num_blocks, num_kv_heads, head_dim, block_size, dtype):
    """A host swap pool (K, V) in the device pool's format, in pinned memory."""
    ks, vs = pool_shapes(num_blocks, num_kv_heads, head_dim, block_size, dtype)
    return torch.zeros(ks, dtype=dtype, pin_memory=True), torch.zeros(vs, dtype=dtype, pin_memory=True)


def _pool_dims(k_cache, v_cache):
    _need(k_cache, "k_cache", ndim=5)
    _need(v_cache, "v_cache", dtype=k_cache.dtype, device=k_cache.device, ndim=4)
    nb, H, nch, bs, x = k_cache.shape
    d = nch * x
    if tuple(v_cache.shape) != (nb, H, d, bs):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} does not match k_cache {tuple(k_cache.shape)}")
    if x * k_cache.element_size() != 16:
        raise ValueError("k_cache last dim must span 16 bytes")
    if not k_cache.is_cuda:
        raise ValueError(f"k_cache must be a GPU tensor, got {k_cache.device}")
    return nb, H, d, bs


def paged_kv_append(k_new, v_new, k_cache, v_cache, slot_mapping):
    """Write each new token's K/V into its slot (slot < 0 skips)."""
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(k_new, "k_new", k_cache.dtype, dev, 3)
    _need(v_new, "v_new", k_cache.dtype, dev, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, dev, 1)
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, H, d) or tuple(v_new.shape) != (T, H, d) or slot_mapping.shape[0] != T:
        raise ValueError("k_new/v_new must be [T][num_kv_heads][head_dim] with T slots")
    N.check(
        N.lib.paged_kv_append(
            _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), T, H, d, bs, nb,
            _dt(k_cache.dtype), _stream(dev),
        )
    )


def paged_kv_copy_blocks(k_cache, v_cache, src_dst):
    """Copy whole blocks ``pool[dst] = pool[src]`` for each row of ``src_dst`` ([n][2] int32)."""
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(src_dst, "src_dst", torch.int32, dev, 2)
    if src_dst.shape[1] != 2:
        raise ValueError("src_dst must be [num_pairs][2]")
    N.check(
        N.lib.paged_kv_copy_blocks(
            _ptr(k_cache), _ptr(v_cache), _ptr(src_dst), src_dst.shape[0], H, d, bs, nb, _dt(k_cache.dtype),
            _stream(dev),
        )
    )


def paged_attention_workgroups_per_head(num_seqs, num_kv_heads, head_dim, block_size, max_context_len,
                                        partition_size=0, dtype=torch.bfloat16):
    return N.check(N.lib.paged_attention_workgroups_per_head(num_seqs, num_kv_heads, head_dim, block_size,
                                                             max_context_len, partition_size, _dt(dtype)))


def paged_attention_segment_cost(block_size):
    """Blocks each non-empty sequence is charged for its fixed work in the
    decode kernel's balanced split of a kv head's block list."""
    return N.check(N.lib.paged_attention_segment_cost(block_size))


def paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
                                    partition_size=0):
    n = N.lib.paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                              max_context_len, partition_size)
    if n == 0 and N.last_error():
        raise N.PKVError(N.PKV_ERR_INVALID_ARG, N.last_error())
    return n


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, max_context_len, scale=None,
                           partition_size=0, workspace=None, shared_blocks=False):
    """Decode attention; writes ``out`` ([S][H_q][d], dtype of q) and returns it.

    ``workspace`` is a uint8 device tensor of at least
    ``paged_attention_workspace_bytes(...)`` bytes; allocated with torch
    when omitted.  ``shared_blocks``: several sequences read the same blocks
    (shared prefixes, forks), so K/V are read through the caches instead of
    streamed (``PKV_DECODE_SHARED_BLOCKS``); the result is the same either
    way.
    """
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", k_cache.dtype, dev, 3)
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    S, Hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, Hq, d):
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have num_seqs rows")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        # the library checks a caller's workspace against the size it needs
        need = paged_attention_workspace_bytes(S, Hq, H, d, bs, int(max_context_len), partition_size)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev, 1)
    N.check(
        N.lib.paged_attention_decode(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens), S, Hq, H, d,
            bs, nb, block_tables.shape[1], int(max_context_len), float(scale), int(partition_size), _ptr(workspace),
            workspace.numel() if workspace is not None else 0, _dt(k_cache.dtype), _flags(shared_blocks),
            _stream(dev),
        )
    )
    return out


def _flags(shared_blocks):
    return N.PKV_DECODE_SHARED_BLOCKS if shared_blocks else 0


def paged_attention_decode_append(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, scale=None, partition_size=0, workspace=None, shared_blocks=False):
    """Append each sequence's new token (position ``context_lens[s] - 1``)
    from ``k_new``/``v_new`` ([S][H_kv][d]) into its slot, then decode
    attention as :func:`paged_attention_decode`; one call, one launch fewer."""
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", k_cache.dtype, dev, 3)
    _need(k_new, "k_new", k_cache.dtype, dev, 3)
    _need(v_new, "v_new", k_cache.dtype, dev, 3)
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    S, Hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, Hq, d):
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
    if tuple(k_new.shape) != (S, H, d) or tuple(v_new.shape) != (S, H, d):
        raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have num_seqs rows")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        # the library checks a caller's workspace against the size it needs
        need = paged_attention_workspace_bytes(S, Hq, H, d, bs, int(max_context_len), partition_size)
        if need:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, dev, 1)
    N.check(
        N.lib.paged_attention_decode_append(
            _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, Hq, H, d, bs, nb, block_tables.shape[1], int(max_context_len), float(scale),
            int(partition_size), _ptr(workspace), workspace.numel() if workspace is not None else 0,
            _dt(k_cache.dtype), _flags(shared_blocks), _stream(dev),
        )
    )
    return out


def paged_attention_decode_append_noalloc(out, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                          max_context_len, scale=None, partition_size=0, shared_blocks=False):
    """:func:`paged_attention_decode_append` with the library's built-in
    scratch instead of a workspace: the call allocates no device memory."""
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", k_cache.dtype, dev, 3)
    _need(k_new, "k_new", k_cache.dtype, dev, 3)
    _need(v_new, "v_new", k_cache.dtype, dev, 3)
    _need(block_tables, "block_tables", torch.int32, dev, 2)
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    S, Hq, dq = q.shape
    if dq != d or tuple(out.shape) != (S, Hq, d):
        raise ValueError("q/out must be [num_seqs][num_q_heads][head_dim]")
    if tuple(k_new.shape) != (S, H, d) or tuple(v_new.shape) != (S, H, d):
        raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("block_tables/context_lens must have num_seqs rows")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    N.check(
        N.lib.paged_attention_decode_append_noalloc(
            _ptr(out), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            _ptr(context_lens), S, Hq, H, d, bs, nb, block_tables.shape[1], int(max_context_len), float(scale),
            int(partition_size), _dt(k_cache.dtype), _flags(shared_blocks), _stream(dev),
        )
    )
    return out


def paged_kv_swap_blocks(src_k, src_v, dst_k, dst_v, pairs):
    """Whole-block copies ``dst[d] = src[s]`` between a device pool and a
    host swap pool (either direction; host pools must be pinned).

    ``pairs``: int32 ``[n][2]`` (source block, destination block), on the
    device or in pinned host memory.  Runs on the current stream of the
    device pool's GPU."""
    dev = src_k.device if src_k.is_cuda else dst_k.device
    nb_s, H, _, bs, _ = src_k.shape
    nb_d = dst_k.shape[0]
    d = src_v.shape[2]
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be on the GPU or in pinned host memory")
    if src_k.shape[1:] != dst_k.shape[1:] or src_v.shape[1:] != dst_v.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools must have the same block format")
    if pairs.dtype != torch.int32 or pairs.dim() != 2 or pairs.shape[1] != 2 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int32 [n][2] tensor")
    if not (pairs.is_cuda or pairs.is_pinned()):
        raise ValueError("pairs must be on the GPU or in pinned host memory")
    N.check(
        N.lib.paged_kv_swap_blocks(
            _ptr(src_k), _ptr(src_v), _ptr(dst_k), _ptr(dst_v), _ptr(pairs), pairs.shape[0], H, d, bs, nb_s, nb_d,
            _dt(src_k.dtype), _stream(dev),
        )
    )


def paged_attention_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                            scale=None):
    """Causal chunked-prefill attention over the paged cache (bf16).

    ``q``/``out``: ``[T][H_q][d]`` with sequence s owning rows
    ``query_start[s] .. query_start[s+1]-1`` (its newest tokens, already
    appended); ``query_start``: int32 ``[S+1]`` on the device;
    ``max_query_len``: host bound on the chunk lengths."""
    nb, H, d, bs = _pool_dims(k_cache, v_cache)
    dev = k_cache.device
    _need(q, "q", k_cache.dtype, dev, 3)
    _need(out, "out", k_cache.dtype, dev, 3)
    T, Hq, dq = q.shape
    if dq != d:
        raise ValueError(f"q head_dim {dq} does not match the pools' {d}")
    _need(context_lens, "context_lens", torch.int32, dev, 1)
    S = context_lens.shape[0]
    for t, name in ((block_tables, "block_tables"), (context_lens, "context_lens"), (query_start, "query_start")):
        _need(t, name, torch.int32, dev)
    if tuple(out.shape) != (T, Hq, d):
        raise ValueError("out must have the shape of q")
    if block_tables.dim() != 2 or block_tables.shape[0] != S or tuple(query_start.shape) != (S + 1,):
        raise ValueError("block_tables must be [S][max_blocks] and query_start [S+1]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    N.check(
        N.lib.paged_attention_prefill(
            _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
            _ptr(query_start), S, T, Hq, H, d, bs, nb, block_tables.shape[1], int(max_query_len), float(scale),
            _dt(k_cache.dtype), _stream(dev),
        )
    )
    return out


def _i64p(a: np.ndarray):
    return a.ctypes.data_as(C.POINTER(C.c_int64))


def _i32p(a: np.ndarray | None):
    return a.ctypes.data_as(C.POINTER(C.c_int32)) if a is not None else None


def _ids32(token_ids, count: int):
    if token_ids is None:
        return None
    if isinstance(token_ids, np.ndarray) and token_ids.dtype == np.int32 and token_ids.flags.c_contiguous:
        if token_ids.shape != (count,):
            raise ValueError(f"token_ids must hold {count} ids")
        return token_ids
    a = np.ascontiguousarray(token_ids, dtype=np.int64)
    if a.shape != (count,):
        raise ValueError(f"token_ids must hold {count} ids")
    if a.size and (a.min() < -(2 ** 31) or a.max() >= 2 ** 31):
        raise ValueError("token ids must fit in int32")
    return a.astype(np.int32)


def _u8p(a: np.ndarray | None):
    return a.ctypes.data_as(C.POINTER(C.c_uint8)) if a is not None else None


def block_digest(parent: bytes | None, salt: int, tokens) -> bytes:
    """Prefix-cache digest of one block (pkv_block_digest)."""
    toks = _ids32(tokens, len(tokens))
    par = None
    if parent is not None:
        if len(parent) != 32:
            raise ValueError("parent digest must be 32 bytes")
        par = np.frombuffer(bytes(parent), np.uint8).copy()
    out = np.zeros(32, np.uint8)
    N.check(N.lib.pkv_block_digest(_u8p(par), _salt(salt), _i32p(toks), toks.shape[0], _u8p(out)))
    return out.tobytes()


def _salt(salt: int) -> int:
    salt = int(salt)
    if not 0 <= salt < 2 ** 64:
        raise ValueError("salt must fit in 64 unsigned bits")
    return salt


class BlockManager:
    """Host block manager (pkv_bm_*): free pool, refcounts, fork, copy-on-write,
    and prefix caching by chained block digests."""

    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        order = None
        if initial_free_order is not None:
            order = np.ascontiguousarray(initial_free_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise ValueError("initial_free_order must have num_blocks entries")
        h = C.c_void_p()
        N.check(N.lib.pkv_bm_create(self.num_blocks, self.block_size, _i32p(order), C.byref(h)))
        self._h = h
        self._destroy = N.lib.pkv_bm_destroy  # kept so __del__ works during interpreter shutdown
        self._slots = np.empty(0, np.int32)
        self._pairs = np.empty(0, np.int32)

    def close(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add_seq(self, seq_id: int):
        N.check(N.lib.pkv_bm_add_seq(self._h, int(seq_id)))

    def add_seq_cached(self, seq_id: int, tokens, salt: int = 0) -> int:
        """Register a sequence for a prompt, sharing its cached leading blocks;
        returns the number of prompt tokens already cached."""
        toks = _ids32(tokens, len(tokens))
        n = C.c_int32(0)
        N.check(N.lib.pkv_bm_add_seq_cached(self._h, int(seq_id), _i32p(toks), toks.shape[0], _salt(salt),
                                            C.byref(n)))
        return n.value

    def add_host_pool(self, num_host_blocks: int):
        N.check(N.lib.pkv_bm_add_host_pool(self._h, int(num_host_blocks)))
        self.num_host_blocks = int(num_host_blocks)

    def _swap(self, fn, seq_id):
        cap = max(self.num_blocks, getattr(self, "num_host_blocks", 0), 1)
        pairs = np.empty((cap, 2), np.int32)
        n = C.c_int32(0)
        N.check(fn(self._h, int(seq_id), _i32p(pairs), cap, C.byref(n)))
        return pairs[: n.value].copy()

    def swap_out(self, seq_id: int):
        """Move a sequence to the host pool; returns (GPU block, host block) pairs to copy."""
        return self._swap(N.lib.pkv_bm_swap_out, seq_id)

    def swap_in(self, seq_id: int):
        """Bring a sequence back; returns (host block, GPU block) pairs to copy."""
        return self._swap(N.lib.pkv_bm_swap_in, seq_id)

    def num_free_host(self) -> int:
        return N.check(N.lib.pkv_bm_num_free_host(self._h))

    def is_swapped(self, seq_id: int) -> bool:
        return bool(N.check(N.lib.pkv_bm_is_swapped(self._h, int(seq_id))))

    def match_prefix(self, tokens, salt: int = 0) -> int:
        toks = _ids32(tokens, len(tokens))
        return N.check(N.lib.pkv_bm_match_prefix(self._h, _i32p(toks), toks.shape[0], _salt(salt)))

    def num_cached(self) -> int:
        return N.check(N.lib.pkv_bm_num_cached(self._h))

    def evictable(self) -> list[int]:
        buf = np.empty(max(self.num_blocks, 1), np.int32)
        n = N.check(N.lib.pkv_bm_evictable(self._h, _i32p(buf), buf.shape[0]))
        return buf[:n].tolist()

    def cached_digest(self, block: int) -> bytes | None:
        out = np.zeros(32, np.uint8)
        return out.tobytes() if N.check(N.lib.pkv_bm_cached_digest(self._h, int(block), _u8p(out))) else None

    def fork(self, parent: int, child: int, num_tokens: int):
        N.check(N.lib.pkv_bm_fork(self._h, int(parent), int(child), int(num_tokens)))

    def free_seq(self, seq_id: int):
        N.check(N.lib.pkv_bm_free_seq(self._h, int(seq_id)))

    def append_slots(self, seq_ids, num_tokens=None, token_ids=None):
        """Returns ``(slots int32[T], cow_pairs int32[n][2])`` (NumPy views valid until the next call).

        ``token_ids`` (T ids in slot order, or None) feed the prefix cache."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        nt = None if num_tokens is None else np.ascontiguousarray(num_tokens, dtype=np.int32)
        total = n if nt is None else int(nt.sum())
        tid = _ids32(token_ids, total)
        if self._slots.shape[0] < max(total, 1):
            self._slots = np.empty(max(total, 1), np.int32)
        cow_cap = n
        if self._pairs.shape[0] < 2 * max(cow_cap, 1):
            self._pairs = np.empty(2 * max(cow_cap, 1), np.int32)
        ns, nc = C.c_int32(0), C.c_int32(0)
        N.check(
            N.lib.pkv_bm_append_slots(
                self._h, _i64p(ids), n, _i32p(nt), _i32p(tid), _i32p(self._slots), self._slots.shape[0], C.byref(ns),
                _i32p(self._pairs), self._pairs.shape[0] // 2, C.byref(nc),
            )
        )
        return self._slots[: ns.value], self._pairs[: 2 * nc.value].reshape(-1, 2)

    def block_tables(self, seq_ids, max_blocks_per_seq: int, tables_out=None, lens_out=None):
        """Fill (or allocate) int32 ``[n][max_blocks]`` tables padded with -1 and ``[n]`` lengths."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        if tables_out is None:
            tables_out = np.empty((n, max_blocks_per_seq), np.int32)
        if lens_out is None:
            lens_out = np.empty(n, np.int32)
        assert tables_out.dtype == np.int32 and tables_out.flags.c_contiguous and tables_out.shape == (n, max_blocks_per_seq)
        assert lens_out.dtype == np.int32 and lens_out.flags.c_contiguous and lens_out.shape == (n,)
        N.check(N.lib.pkv_bm_block_tables(self._h, _i64p(ids), n, max_blocks_per_seq, _i32p(tables_out),
                                          _i32p(lens_out)))
        return tables_out, lens_out

    def stage_step(self, seq_ids, stage, block_tables, context_lens, slot_mapping, cow_pairs, full=False,
                   token_ids=None):
        """One decode step's bookkeeping, staged to the device without copies.

        ``stage``: pinned int32 CPU tensor of at least ``stage_capacity``
        entries (alternate two and wait for the GPU before reusing one);
        ``block_tables`` [n][max_blocks], ``context_lens`` [n],
        ``slot_mapping`` [n], ``cow_pairs`` [n][2]: int32 device tensors.
        ``token_ids``: the new tokens' ids ([n], host) for the prefix cache.
        Returns ``(n_cow, max_len)``; the work runs on the current stream.
        """
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = ids.shape[0]
        tid = _ids32(token_ids, n)
        if not (stage.dtype == torch.int32 and stage.is_pinned() and stage.is_contiguous()):
            raise ValueError("stage must be a contiguous pinned int32 CPU tensor")
        dev = block_tables.device
        for t, name, shape in ((block_tables, "block_tables", None), (context_lens, "context_lens", (n,)),
                               (slot_mapping, "slot_mapping", (n,)), (cow_pairs, "cow_pairs", None)):
            _need(t, name, torch.int32, dev)
            if shape is not None and tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}")
        if block_tables.dim() != 2 or block_tables.shape[0] != n:
            raise ValueError("block_tables must be [n_seqs][max_blocks_per_seq]")
        if cow_pairs.dim() != 2 or cow_pairs.shape[1] != 2:
            raise ValueError("cow_pairs must be [capacity][2]")
        n_cow, max_len = C.c_int32(0), C.c_int32(0)
        N.check(
            N.lib.pkv_bm_stage_step(
                self._h, _i64p(ids), n, _i32p(tid), C.c_void_p(stage.data_ptr()), stage.numel(), _ptr(block_tables),
                block_tables.shape[1], _ptr(context_lens), _ptr(slot_mapping), _ptr(cow_pairs), cow_pairs.shape[0],
                int(bool(full)), C.byref(n_cow), C.byref(max_len), _stream(dev),
            )
        )
        return n_cow.value, max_len.value

    @staticmethod
    def stage_capacity(n_seqs: int, max_blocks_per_seq: int) -> int:
        return N.check(N.lib.pkv_bm_stage_capacity(int(n_seqs), int(max_blocks_per_seq)))

    def num_free(self) -> int:
        return N.check(N.lib.pkv_bm_num_free(self._h))

    def refcount(self, block: int) -> int:
        return N.check(N.lib.pkv_bm_refcount(self._h, int(block)))

    def num_shared(self) -> int:
        """Device blocks held by more than one sequence (the hint for ``shared_blocks``)."""
        return N.check(N.lib.pkv_bm_num_shared(self._h))

    def seq_len(self, seq_id: int) -> int:
        return N.check(N.lib.pkv_bm_seq_len(self._h, int(seq_id)))

    def num_seqs(self) -> int:
        return N.check(N.lib.pkv_bm_num_seqs(self._h))

    def free_stack(self) -> list[int]:
        buf = np.empty(max(self.num_free(), 1), np.int32)
        n = N.check(N.lib.pkv_bm_free_stack(self._h, _i32p(buf), buf.shape[0]))
        return buf[:n].tolist()


class RadixIndex:
    """Radix-tree prefix index over a BlockManager (pkv_radix_*): token-level
    longest-prefix reuse, path insertion and LRU eviction of unlocked leaves."""

    def __init__(self, bm: BlockManager):
        h = C.c_void_p()
        N.check(N.lib.pkv_radix_create(bm._h, C.byref(h)))
        self._h = h
        self.bm = bm  # the block manager must outlive the index
        self._destroy = N.lib.pkv_radix_destroy

    def close(self):
        if getattr(self, "_h", None) and getattr(self.bm, "_h", None):
            self._destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def match(self, tokens) -> int:
        t = _ids32(tokens, len(tokens))
        return N.check(N.lib.pkv_radix_match(self._h, _i32p(t), t.shape[0]))

    def admit(self, seq_id: int, tokens) -> int:
        """New request sharing the longest cached prefix; returns its length."""
        t = _ids32(tokens, len(tokens))
        n = C.c_int32(0)
        N.check(N.lib.pkv_radix_admit(self._h, int(seq_id), _i32p(t), t.shape[0], C.byref(n)))
        return n.value

    def insert(self, seq_id: int, tokens) -> int:
        t = _ids32(tokens, len(tokens))
        n = C.c_int32(0)
        N.check(N.lib.pkv_radix_insert(self._h, int(seq_id), _i32p(t), t.shape[0], C.byref(n)))
        return n.value

    def release(self, seq_id: int):
        N.check(N.lib.pkv_radix_release(self._h, int(seq_id)))

    def evict(self, num_free_blocks: int) -> int:
        n = C.c_int32(0)
        N.check(N.lib.pkv_radix_evict(self._h, int(num_free_blocks), C.byref(n)))
        return n.value

    def nodes(self):
        """[(holder, depth, edge_len, locks, stamp)] depth-first, children by first token."""
        cap = max(N.check(N.lib.pkv_radix_num_nodes(self._h)), 1)
        h, st = np.empty(cap, np.int64), np.empty(cap, np.int64)
        d, e, lk = (np.empty(cap, np.int32) for _ in range(3))
        n = N.check(N.lib.pkv_radix_nodes(self._h, _i64p(h), _i32p(d), _i32p(e), _i32p(lk), _i64p(st), cap))
        return list(zip(h[:n].tolist(), d[:n].tolist(), e[:n].tolist(), lk[:n].tolist(), st[:n].tolist()))
