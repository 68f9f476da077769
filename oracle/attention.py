"""Oracle: single-query decode attention over a paged KV cache (CPU, fp64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition.  Paging changes only where K/V live, never what attention
computes ("PagedAttention et RadixAttention : parlons de KV Cache",
*PagedAttention : la mémoire comme un système d'exploitation*, closing
paragraph; the second step there: the engine consults the table to collect
the blocks and the sequence looks contiguous).  So for each sequence ``s``
with context length ``L`` (tokens read, including this step's appended
token) and query head ``h``:

    K, V = gather(blocks of s through its table)[:L]       # [L][H_kv][d]
    g    = h // (H_q / H_kv)                                # GQA group
    x_t  = scale * <q[s,h], K[t,g]>                         # t < L
    out[s,h] = sum_t softmax(x)_t * V[t,g]

with ``scale = 1/sqrt(head_dim)`` unless given.  ``L = 0`` gives a zero row.
Stored values are upcast exactly to fp64; all arithmetic is fp64.

Readings where the pages are silent: the pages never write the attention
formula or mention grouped-query attention; the head mapping
``g = h // (H_q/H_kv)`` (consecutive query heads share a kv head) and the
scale are taken from the benchmark spec of the problem.

Multi-token (chunked prefill) form: a prompt's K/V are computed during the
prefill phase and written into the cache ("PagedAttention et RadixAttention :
parlons de KV Cache", the part on the two independent problems: the engine
computes the prompt's keys and values during prefill; the closing part on
prefix caching: skipping the prefill of prefixes already seen).  Reading
where the pages are silent: a chunk of the C newest tokens of a sequence of
length L (their K/V already appended) is attended causally, the token at
position p = L - C + i reading cache positions 0..p; the rows of a batch
are packed, sequence s owning rows ``query_start[s] .. query_start[s+1]-1``.
Each row is therefore the decode result of the same cache at context
length p + 1.

Pins (``tests/test_oracle_attention.py``): scalar brute force with
``math.fsum`` on tiny inputs; closed forms (L = 1 returns V_0; q = 0 or all
keys equal returns the mean of V; constant V returns V; two tokens give a
logistic blend; a dominant needle key returns its value); GQA equals MHA
with replicated kv heads; the output is invariant under any physical
permutation of the blocks and under sharing versus private copies; and the
split-context log-sum-exp merge equals the unsplit result.
"""
from __future__ import annotations

import math

import numpy as np

from . import pool as _pool

__all__ = ["dense_attention", "decode_attention", "decode_attention_bruteforce", "lse_merge", "partition_partials",
           "prefill_attention"]


def dense_attention(q_row, k_seq, v_seq, scale):
    """Attention of one sequence on contiguous fp64 K/V.

    ``q_row``: ``[H_q][d]``; ``k_seq``/``v_seq``: ``[L][H_kv][d]`` (fp64).
    Returns ``[H_q][d]`` fp64.
    """
    Hq, d = q_row.shape
    L, Hkv, _ = k_seq.shape
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    out = np.zeros((Hq, d), dtype=np.float64)
    if L == 0:
        return out
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)  # query heads h with h // G == g
        x = (k_seq[:, g, :] @ q_row[heads].T) * scale  # [L][G] logits
        p = np.exp(x - x.max(axis=0))
        out[heads] = (p.T @ v_seq[:, g, :]) / p.sum(axis=0)[:, None]
    return out


def decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale=None):
    """Paged decode attention for a batch, fp64 ``[S][H_q][d]``.

    ``q``: ``[S][H_q][d]`` storage dtype; pools in the format of
    ``oracle.pool``; ``block_tables``: ``[S][max_blocks]`` int; ``context_lens``:
    ``[S]`` int.
    """
    q64 = _pool.to_f64(q)
    S, Hq, d = q64.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        k_seq, v_seq = _pool.gather(k_pool, v_pool, block_tables[s], L)
        out[s] = dense_attention(q64[s], _pool.to_f64(k_seq), _pool.to_f64(v_seq), scale)
    return out


def prefill_attention(q, k_pool, v_pool, block_tables, context_lens, query_start, scale=None):
    """Causal attention of each sequence's newest tokens over its paged cache,
    fp64 ``[T][H_q][d]``.

    ``q``: ``[T][H_q][d]`` storage dtype, rows packed by sequence;
    ``query_start``: ``[S+1]`` int, sequence s owning rows
    ``query_start[s] .. query_start[s+1]-1`` = its ``C`` newest tokens, at
    positions ``L-C .. L-1`` (``C <= L``).  Row of position p reads cache
    positions ``0..p``.
    """
    q64 = _pool.to_f64(q)
    T, Hq, d = q64.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qs = [int(x) for x in query_start]
    S = len(qs) - 1
    if qs[0] != 0 or qs[-1] != T or any(qs[s + 1] < qs[s] for s in range(S)):
        raise ValueError("query_start must rise from 0 to the number of rows")
    out = np.zeros((T, Hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        C = qs[s + 1] - qs[s]
        if C > L:
            raise ValueError("a sequence has more new tokens than context")
        if C == 0:
            continue
        k_seq, v_seq = _pool.gather(k_pool, v_pool, block_tables[s], L)
        k64, v64 = _pool.to_f64(k_seq), _pool.to_f64(v_seq)
        for i in range(C):
            p = L - C + i
            out[qs[s] + i] = dense_attention(q64[qs[s] + i], k64[: p + 1], v64[: p + 1], scale)
    return out


def decode_attention_bruteforce(q, k_pool, v_pool, block_tables, context_lens, scale=None):
    """Scalar re-statement of ``decode_attention`` for tiny inputs.

    Reads every element through explicit flat index arithmetic of the
    storage format (no reshapes), and sums with ``math.fsum``.
    """
    q64 = _pool.to_f64(q)
    S, Hq, d = q64.shape
    nb, Hkv, nch, bs, x = k_pool.shape
    kflat = _pool.to_f64(k_pool).reshape(-1)
    vflat = _pool.to_f64(v_pool).reshape(-1)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = Hq // Hkv

    def kval(b, h, o, i):
        return kflat[(((b * Hkv + h) * nch + i // x) * bs + o) * x + i % x]

    def vval(b, h, o, i):
        return vflat[((b * Hkv + h) * d + i) * bs + o]

    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        for h in range(Hq):
            g = h // G
            if L == 0:
                continue
            logits = []
            for t in range(L):
                b = int(block_tables[s][t // bs])
                o = t % bs
                logits.append(scale * math.fsum(q64[s, h, i] * kval(b, g, o, i) for i in range(d)))
            mx = max(logits)
            w = [math.exp(z - mx) for z in logits]
            den = math.fsum(w)
            for i in range(d):
                num = math.fsum(
                    w[t] * vval(int(block_tables[s][t // bs]), g, t % bs, i) for t in range(L)
                )
                out[s, h, i] = num / den
    return out


def partition_partials(q_row, k_seq, v_seq, scale, partition):
    """Per-partition ``(m, l, acc)`` for one sequence, fp64 (split-context form).

    For tokens ``[p*P, (p+1)*P)``: ``m`` = max logit, ``l = sum exp(x - m)``,
    ``acc = sum exp(x - m) V``.  Empty partitions give ``m = -inf, l = 0``.
    The split itself is not on the pages; it is the standard way to spread
    one long context over many workgroups.
    """
    Hq, d = q_row.shape
    L, Hkv, _ = k_seq.shape
    G = Hq // Hkv
    npart = max(1, -(-L // partition))
    m = np.full((npart, Hq), -np.inf)
    l = np.zeros((npart, Hq))
    acc = np.zeros((npart, Hq, d))
    for p in range(npart):
        lo, hi = p * partition, min(L, (p + 1) * partition)
        if lo >= hi:
            continue
        for h in range(Hq):
            g = h // G
            x = (k_seq[lo:hi, g, :] @ q_row[h]) * scale
            m[p, h] = x.max()
            e = np.exp(x - m[p, h])
            l[p, h] = e.sum()
            acc[p, h] = e @ v_seq[lo:hi, g, :]
    return m, l, acc


def lse_merge(m, l, acc):
    """Combine partition partials: weights ``exp(m_p - max_p m_p)``; empty parts weigh 0."""
    M = m.max(axis=0)
    w = np.where(np.isfinite(m), np.exp(m - M), 0.0)
    num = (w[:, :, None] * acc).sum(axis=0)
    den = (w * l).sum(axis=0)
    return num / den[:, None]
