"""Seeded random shapes against the oracle, beyond the fixed cases.

Decode: bf16 and fp32, every kernel instantiation (head_dim 64/128 x block
16/32), group sizes up to the kernel's limit, one to eight sequences of 1 to
700 tokens, several partition sizes, two consecutive steps.

Prefill (bf16): group sizes 1..256, histories and chunks drawn so that the
tiles' step counts cover every residue of the barrier period and the context
end falls on steps with and without a barrier.

Tolerances: decode as ``helpers.TOL``; prefill the bound of
``helpers.assert_within_prefill_bound``.  The case's parameters are printed
before it runs."""
import math

import numpy as np
import pytest
import torch

from helpers import (assert_close, assert_pools_equal, assert_within_prefill_bound, product_cache,
                     product_prefill_step, say)
import oracle.attention as oatt
from oracle.runner import OracleRun, _storage
from workloads import Workload

pytestmark = pytest.mark.gpu


def _decode_workload(i):
    r = np.random.default_rng(7000 + i)
    f32 = i % 3 == 0
    hkv = int(r.choice([1, 2, 4, 8]))
    g = int(r.choice([1, 2, 3, 4, 5, 8, 16] if f32 else [1, 2, 3, 4, 5, 8]))
    d = int(r.choice([64, 128]))
    bs = int(r.choice([16, 32]))
    lengths = [int(x) for x in r.integers(1, 701, size=int(r.integers(1, 9)))]
    nb = sum(math.ceil((L + 2) / bs) for L in lengths) + 16
    name = "c1_tiny_f32" if f32 else "c2_8b_bf16"
    return Workload(name, seed=7000 + i, overrides=dict(lengths=lengths, num_q_heads=hkv * g, num_kv_heads=hkv,
                                                         head_dim=d, block_size=bs, num_blocks=nb, steps=2))


@pytest.mark.parametrize("i", range(12))
def test_decode_random_shape(i):
    w = _decode_workload(i)
    c = w.config
    say(f"decode case {i}: {c.dtype} Hq={c.num_q_heads} Hkv={c.num_kv_heads} d={c.head_dim} bs={c.block_size} "
        f"lengths={list(w.lengths)}")
    cache = product_cache(w)
    run = OracleRun(w)
    for k in range(2):
        kn, vn = w.kv(("step", k))
        slots, pairs = cache.append(w.decode_seqs, [1] * w.num_seqs, kn, vn)
        rslots, rpairs = run.step(k)
        assert slots.tolist() == rslots and pairs.tolist() == [list(p) for p in rpairs]
        q = w.q(k)
        ref = run.attention(q)
        for P in (0, c.block_size, 4 * c.block_size):
            out = cache.decode(q.cuda(), w.decode_seqs, partition_size=P)
            torch.cuda.synchronize()
            assert_close(out, ref, c.dtype, f"case {i} step {k} P={P}")
    assert_pools_equal(cache, run)


def _prefill_workload(i):
    r = np.random.default_rng(8000 + i)
    g = int(r.choice([1, 2, 4, 5, 8, 16, 32, 64, 128, 256]))
    hkv = int(r.choice([1, 2])) if g >= 64 else int(r.choice([1, 2, 4, 8]))
    d = int(r.choice([64, 128]))
    bs = int(r.choice([16, 32]))
    S = int(r.integers(1, 5))
    # keep the oracle's work bounded: chunk rows x query heads
    max_chunk = max(1, min(200, 6000 // (hkv * g)))
    chunks = [int(x) for x in r.integers(1, max_chunk + 1, size=S)]
    hist = [int(x) for x in r.integers(0, 600, size=S)]
    nb = sum(math.ceil((h + c) / bs) for h, c in zip(hist, chunks)) + 16
    return Workload("c7_prefill_bf16", seed=8000 + i,
                    overrides=dict(histories=hist, chunks=chunks, num_q_heads=hkv * g, num_kv_heads=hkv,
                                   head_dim=d, block_size=bs, num_blocks=nb))


@pytest.mark.parametrize("i", range(10))
def test_prefill_random_shape(i):
    w = _prefill_workload(i)
    c = w.config
    say(f"prefill case {i}: Hq={c.num_q_heads} Hkv={c.num_kv_heads} d={c.head_dim} bs={c.block_size} "
        f"chunks={w.chunk_lens}")
    cache = product_cache(w)
    run = OracleRun(w)
    out, slots, _ = product_prefill_step(cache, w, 0)
    o_slots, _ = run.prefill_step(0)
    assert slots.tolist() == o_slots
    q = w.prefill_q(0)
    ref = run.prefill_attention(q)
    tables, lens = run.tables()
    absv = run.v_pool & np.uint16(0x7FFF)  # |V|: clear the bf16 sign bit
    A = oatt.prefill_attention(_storage(q), run.k_pool, absv, tables, lens, w.query_start())
    assert_within_prefill_bound(out, ref, A, f"prefill case {i}")
