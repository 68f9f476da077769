"""Oracle: physical K/V block pools, cache append and block copy (CPU, NumPy).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Storage format.  The pages fix only that the cache is split into fixed-size
blocks of token slots, per layer, placed anywhere in GPU memory and reached
through a per-sequence block table ("PagedAttention" glossary, *Définition*;
robocikowo "PagedAttention", *Jak działa*).  The byte layout inside a block
is this library's interface and is defined here independently of the GPU
code.  With ``x = 16 // itemsize`` (4 for fp32, 8 for bf16):

* K pool, shape ``[num_blocks][H_kv][head_dim / x][block_size][x]``: token
  ``o`` of block ``b``, kv head ``h``, dimension ``i`` sits at
  ``[b][h][i // x][o][i % x]`` -- each 16-byte chunk holds ``x`` consecutive
  dimensions of one token, and the chunks of one dimension range are
  contiguous over the block's tokens.
* V pool, shape ``[num_blocks][H_kv][head_dim][block_size]``: element
  ``[b][h][i][o]`` (each dimension's values for the block's tokens are
  contiguous).

bf16 values are held as their raw uint16 bit patterns (NumPy has no bf16);
append and copy are pure bit moves, so the pools compare byte for byte.

Pins: append -> gather round trip returns the logical token rows exactly
(``test_oracle_pool``), a hand-written placement fixture
(``tests/golden/pool_layout_tiny.json``), and copy-on-write leaving the
source block untouched.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "chunk_width",
    "new_pools",
    "append",
    "copy_blocks",
    "gather",
    "to_f64",
    "swap_copy",
]


def chunk_width(itemsize: int) -> int:
    """Elements per 16-byte K chunk."""
    if 16 % itemsize:
        raise ValueError("itemsize must divide 16")
    return 16 // itemsize


def new_pools(num_blocks, num_kv_heads, head_dim, block_size, storage_dtype, fill=0):
    """Allocate zero- (or ``fill``-) initialised K and V pools in the storage format."""
    dt = np.dtype(storage_dtype)
    x = chunk_width(dt.itemsize)
    if head_dim % x:
        raise ValueError("head_dim must be a multiple of the chunk width")
    k = np.full((num_blocks, num_kv_heads, head_dim // x, block_size, x), fill, dtype=dt)
    v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=dt)
    return k, v


def append(k_pool, v_pool, k_new, v_new, slot_mapping):
    """Scatter each new token's K and V into its slot.

    ``slot = block * block_size + offset``; a negative slot means "skip".
    ``k_new``/``v_new``: ``[T][H_kv][head_dim]`` in the storage dtype.
    This is the write implied by on-demand growth: a token occupies exactly
    the next slot of its sequence (aitalk page, *PagedAttention* section,
    third step).
    """
    nb, H, nch, bs, x = k_pool.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    kn = np.asarray(k_new)[keep]
    vn = np.asarray(v_new)[keep]
    if len(slots) and slots.max() >= nb * bs:
        raise IndexError("slot outside the pool")
    b = slots // bs
    o = slots % bs
    # Advanced indices on the block and slot axes: element t of the result
    # is token t's [H][d/x][x] chunk grid (slots are distinct).
    k_pool[b, :, :, o, :] = kn.reshape(len(slots), H, nch, x)
    v_pool[b, :, :, o] = vn


def copy_blocks(k_pool, v_pool, pairs):
    """Copy-on-write block copy: ``pool[dst] = pool[src]`` for each pair, in order.

    The whole block (all slots, all kv heads) is duplicated; the source is
    only read (robocikowo "PagedAttention", *Komponenty*, reference counting
    with lazy duplication; aitalk page, fourth step).
    """
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2):
        k_pool[dst] = k_pool[src].copy()
        v_pool[dst] = v_pool[src].copy()


def swap_copy(src_k, src_v, dst_k, dst_v, pairs):
    """Whole-block copies between two pools of the same format (device pool
    and host swap pool): ``dst[d] = src[s]`` for every ``(s, d)``."""
    for s, d in pairs:
        dst_k[d] = src_k[s]
        dst_v[d] = src_v[s]


def gather(k_pool, v_pool, table_row, length):
    """A sequence's K and V, ``[length][H_kv][head_dim]``, in logical order.

    The engine reads the block table to collect the blocks, so the model
    sees one contiguous sequence (aitalk page, second step).
    """
    nb, H, nch, bs, x = k_pool.shape
    d = nch * x
    if length == 0:
        return (np.zeros((0, H, d), k_pool.dtype), np.zeros((0, H, d), v_pool.dtype))
    nblk = -(-length // bs)
    blocks = np.asarray(table_row[:nblk], dtype=np.int64)
    if len(blocks) < nblk or (blocks < 0).any() or (blocks >= nb).any():
        raise IndexError("block table does not cover the context")
    kb = k_pool[blocks]  # [n][H][d/x][bs][x]
    kb = kb.transpose(0, 3, 1, 2, 4).reshape(nblk * bs, H, d)
    vb = v_pool[blocks]  # [n][H][d][bs]
    vb = vb.transpose(0, 3, 1, 2).reshape(nblk * bs, H, d)
    return kb[:length], vb[:length]


def to_f64(a):
    """Exact upcast of stored values (fp32, or bf16 bit patterns) to fp64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if a.dtype == np.float32:
        return a.astype(np.float64)
    if a.dtype == np.float64:
        return a
    raise TypeError(f"unsupported storage dtype {a.dtype}")
