"""Oracle: execute a workload script on the CPU model.

TEST INFRASTRUCTURE ONLY (see the package docstring).

``OracleRun`` plays a ``workloads.Workload`` script through
``BlockManagerModel`` and, when ``materialize`` is true, through NumPy pools
(``oracle.pool``).  Independently of any paging it also records, for every
sequence, where each of its logical tokens came from (value key and row),
so a sequence's contiguous K/V can be rebuilt without a pool: that is the
"sequence looks contiguous" view the pages describe ("PagedAttention et
RadixAttention : parlons de KV Cache", *PagedAttention : la mémoire comme
un système d'exploitation*, second step), used for sampled checks at sizes
where a full CPU pool is too slow.
"""
from __future__ import annotations

import numpy as np
import torch

from . import attention as _att
from . import pool as _pool
from .block_manager import BlockManagerModel


def _storage(t: torch.Tensor) -> np.ndarray:
    """Torch CPU tensor -> NumPy storage array (bf16 as uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.contiguous().numpy()
    raise TypeError(t.dtype)


class OracleRun:
    def __init__(self, workload, materialize=True):
        self.w = workload
        c = workload.config
        self.bm = BlockManagerModel(workload.num_blocks, c.block_size, workload.free_order)
        self.materialize = materialize
        if materialize:
            sd = np.float32 if c.dtype == "f32" else np.uint16
            self.k_pool, self.v_pool = _pool.new_pools(
                workload.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, sd
            )
        self.sources = {}  # sid -> list of (key, row)
        self.cow_log = []
        self.admitted = {}  # sid -> prompt tokens found in the prefix cache
        self._kv_cache = {}
        self.step_done = -1
        for op in workload.setup_ops:
            self._apply(op)

    # ------------------------------------------------------------ script
    def _kv(self, key):
        if key not in self._kv_cache:
            self._kv_cache[key] = self.w.kv(key)
        return self._kv_cache[key]

    def _apply(self, op):
        kind = op[0]
        if kind == "add":
            self.bm.add_seq(op[1])
            self.sources[op[1]] = []
        elif kind == "fork":
            _, parent, child, n = op
            self.bm.fork(parent, child, n)
            self.sources[child] = list(self.sources[parent][:n])
        elif kind == "free":
            self.bm.free_seq(op[1])
            del self.sources[op[1]]
        elif kind == "append":
            _, sids, ntoks, key = op
            self._append(sids, ntoks, key)
        elif kind == "admit":
            _, sid, tokens, key, salt = op
            tokens = [int(t) for t in tokens]
            n = self.bm.add_seq_cached(sid, tokens, salt)
            self.admitted[sid] = n
            # the cached positions hold the same values as the prompt's rows
            self.sources[sid] = [(key, i) for i in range(n)]
            self._append([sid], [len(tokens) - n], key, token_ids=tokens[n:], first_row=n)
        else:
            raise ValueError(op)

    def _append(self, sids, ntoks, key, token_ids=None, first_row=0):
        slots, pairs = self.bm.append_slots(sids, ntoks, token_ids=token_ids)
        self.cow_log.append(pairs)
        row = first_row
        for sid, n in zip(sids, ntoks):
            self.sources[sid].extend((key, row + i) for i in range(n))
            row += n
        if self.materialize:
            _pool.copy_blocks(self.k_pool, self.v_pool, pairs)
            k, v = self._kv(key)
            end = first_row + len(slots)
            _pool.append(self.k_pool, self.v_pool, _storage(k[first_row:end]), _storage(v[first_row:end]), slots)
            self._kv_cache.pop(key, None)
        return slots, pairs

    def step(self, k):
        """Decode step ``k``: append one token per decode sequence; returns (slots, pairs)."""
        sids = self.w.decode_seqs
        key = ("step", k)
        ids = self.w.step_tokens(k) if hasattr(self.w, "step_tokens") else None
        out = self._append(sids, [1] * len(sids), key, token_ids=None if ids is None else [int(t) for t in ids])
        self.step_done = k
        return out

    def prefill_step(self, k):
        """Prefill step ``k``: append each sequence's chunk; returns (slots, pairs)."""
        sids = self.w.decode_seqs
        out = self._append(sids, list(self.w.chunk_lens), ("chunk", k))
        self.step_done = k
        return out

    # ------------------------------------------------------------ views
    def tables(self, max_blocks=None):
        sids = self.w.decode_seqs
        if max_blocks is None:
            max_blocks = max(len(self.bm.tables[s]) for s in sids)
        rows, lens = self.bm.block_tables(sids, max_blocks)
        return np.asarray(rows, dtype=np.int32), np.asarray(lens, dtype=np.int32)

    def attention(self, q, scale=None):
        """Oracle decode over the materialised pools, fp64 ``[S][H_q][d]``."""
        tables, lens = self.tables()
        return _att.decode_attention(_storage(q), self.k_pool, self.v_pool, tables, lens, scale)

    def prefill_attention(self, q, scale=None):
        """Oracle chunked-prefill attention over the materialised pools, fp64 ``[T][H_q][d]``."""
        tables, lens = self.tables()
        return _att.prefill_attention(_storage(q), self.k_pool, self.v_pool, tables, lens, self.w.query_start(), scale)

    def logical_prefill_row(self, q, row, scale=None, abs_v=False):
        """Oracle attention of one chunk row from its sequence's logical tokens
        (positions 0..p); with ``abs_v`` the same weights applied to |V|."""
        qs = self.w.query_start()
        s = int(np.searchsorted(qs, row, side="right")) - 1
        sid = self.w.decode_seqs[s]
        L = len(self.sources[sid])
        p = L - int(qs[s + 1] - qs[s]) + (row - int(qs[s]))
        k, v = self.logical_kv(sid)
        qrow = _pool.to_f64(_storage(q[row]))
        if scale is None:
            scale = 1.0 / np.sqrt(qrow.shape[-1])
        if abs_v:
            v = np.abs(v)
        return _att.dense_attention(qrow, k[: p + 1], v[: p + 1], scale)

    def logical_kv(self, sid):
        """fp64 K, V ``[L][H_kv][d]`` of one sequence, rebuilt from its token sources."""
        srcs = self.sources[sid]
        keys = {}
        for key, _ in srcs:
            if key not in keys:
                k, v = self.w.kv(key)
                keys[key] = (_pool.to_f64(_storage(k)), _pool.to_f64(_storage(v)))
        kk = np.stack([keys[key][0][r] for key, r in srcs]) if srcs else None
        vv = np.stack([keys[key][1][r] for key, r in srcs]) if srcs else None
        return kk, vv

    def logical_attention(self, q, seq_index, scale=None):
        """Oracle attention of decode sequence ``seq_index`` from its logical tokens."""
        sid = self.w.decode_seqs[seq_index]
        qrow = _pool.to_f64(_storage(q[seq_index]))
        k, v = self.logical_kv(sid)
        if scale is None:
            scale = 1.0 / np.sqrt(qrow.shape[-1])
        if k is None:
            return np.zeros_like(qrow)
        return _att.dense_attention(qrow, k, v, scale)
