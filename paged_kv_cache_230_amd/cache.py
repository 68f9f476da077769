"""PagedKVCache: one layer's K/V pools plus a block manager, driven from Python.

A convenience layer over the binding: it owns the device pools (torch
tensors), a ``BlockManager``, and forwards each operation to the library
(block manager on the host, copy/append/decode kernels on the GPU).  All
arithmetic of the method runs in the library.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .api import BlockManager, new_pools, paged_attention_decode, paged_kv_append, paged_kv_copy_blocks


class PagedKVCache:
    def __init__(self, num_blocks, num_kv_heads, head_dim, block_size, dtype, device="cuda", free_order=None):
        self.num_blocks = int(num_blocks)
        self.num_kv_heads = int(num_kv_heads)
        self.head_dim = int(head_dim)
        self.block_size = int(block_size)
        self.dtype = dtype
        self.device = torch.device(device)
        self.k_cache, self.v_cache = new_pools(num_blocks, num_kv_heads, head_dim, block_size, dtype, self.device)
        self.bm = BlockManager(num_blocks, block_size, free_order)
        self.cow_log = []
        self.admitted = {}  # sid -> prompt tokens found in the prefix cache

    # ------------------------------------------------------------- sequences
    def add_seq(self, sid):
        self.bm.add_seq(sid)

    def fork(self, parent, child, n):
        self.bm.fork(parent, child, n)

    def free_seq(self, sid):
        self.bm.free_seq(sid)

    def admit(self, sid, tokens, k, v, salt=0):
        """Cached admission of a prompt: share its cached leading blocks, then
        append the rest (K/V rows ``k[i]``, ``v[i]`` for prompt position i).
        Returns the number of prompt tokens found in the cache."""
        n = self.bm.add_seq_cached(sid, tokens, salt)
        self.admitted[sid] = n
        rest = len(tokens) - n
        if rest:
            self.append([sid], [rest], k[n:], v[n:], token_ids=np.asarray(tokens)[n:])
        return n

    def append(self, sids, ntoks, k, v, token_ids=None):
        """Reserve slots, run copy-on-write copies, then write the tokens' K/V."""
        slots, pairs = self.bm.append_slots(sids, ntoks, token_ids=token_ids)
        self.cow_log.append(pairs.copy())
        if pairs.shape[0]:
            paged_kv_copy_blocks(self.k_cache, self.v_cache, torch.from_numpy(pairs.copy()).to(self.device))
        if slots.shape[0]:
            paged_kv_append(
                k.to(self.device).contiguous(),
                v.to(self.device).contiguous(),
                self.k_cache,
                self.v_cache,
                torch.from_numpy(slots.copy()).to(self.device),
            )
        return slots.copy(), pairs.copy()

    def apply(self, op, kv_fn):
        """Run one script operation; ``kv_fn(key)`` returns the (K, V) rows of an append."""
        kind = op[0]
        if kind == "add":
            self.add_seq(op[1])
        elif kind == "fork":
            self.fork(op[1], op[2], op[3])
        elif kind == "free":
            self.free_seq(op[1])
        elif kind == "append":
            _, sids, ntoks, key = op
            k, v = kv_fn(key)
            self.append(sids, ntoks, k, v)
        elif kind == "admit":
            _, sid, tokens, key, salt = op
            k, v = kv_fn(key)
            self.admit(sid, tokens, k, v, salt)
        else:
            raise ValueError(f"unknown operation {op!r}")

    # ---------------------------------------------------------------- decode
    def tables(self, sids, max_blocks=None):
        """Device int32 block tables and context lengths for ``sids``; also returns the host copies."""
        lens = np.array([self.bm.seq_len(s) for s in sids], np.int32)
        if max_blocks is None:
            max_blocks = max(1, int(math.ceil(int(lens.max(initial=0)) / self.block_size)))
        t, l = self.bm.block_tables(sids, max_blocks)
        return torch.from_numpy(t).to(self.device), torch.from_numpy(l).to(self.device), t, l

    def decode(self, q, sids, scale=None, partition_size=0, out=None):
        tables, lens, _, lh = self.tables(sids)
        if out is None:
            out = torch.empty_like(q)
        max_len = int(lh.max(initial=0))
        return paged_attention_decode(out, q, self.k_cache, self.v_cache, tables, lens, max_len, scale=scale,
                                      partition_size=partition_size, shared_blocks=self.bm.num_shared() > 0)
