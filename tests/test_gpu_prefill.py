"""Chunked-prefill attention on the GPU against the oracle: every kernel
instantiation (head_dim 64/128 x block 16/32) and group sizes 1..256, ragged
chunks (1 token, tile-sized, tile + tail) over histories from empty to
several hundred tokens, the stress value distributions, NaN in unused pool
slots, two consecutive chunks, and sampled rows of the full-size batch
against each sequence's logical (contiguous) K/V.

Tolerance: the elementwise bound of ``helpers.assert_within_prefill_bound``
(bf16 probabilities in the value product: u * mean_w|V| + u * |out|), plus
the decode bar's 2e-3 absolute error."""

import numpy as np
import pytest
import torch

from helpers import (assert_pools_equal, assert_within_prefill_bound, product_cache, product_prefill_step,
                     say)
import oracle.attention as oatt
from oracle.runner import OracleRun, _storage
from workloads import Workload

pytestmark = pytest.mark.gpu

SMALL = dict(histories=[0, 5, 33, 100, 250], chunks=[1, 17, 40, 64, 130], num_blocks=220)

SHAPES = [  # (q heads, kv heads, head_dim, block size)
    (32, 8, 128, 16),   # G 4 (8B-shaped)
    (64, 8, 128, 16),   # G 8 (70B-shaped)
    (8, 8, 128, 32),    # G 1
    (40, 8, 64, 16),    # G 5: a tile of 25 tokens, 3 idle rows
    (64, 8, 64, 32),    # G 8, head_dim 64, block 32
    (128, 1, 128, 16),  # G 128: two tokens per tile
    (256, 1, 64, 32),   # G 256: one token per tile
]


def _check(run, w, out, k, what):
    q = w.prefill_q(k)
    ref = run.prefill_attention(q)
    tables, lens = run.tables()
    absv = run.v_pool & np.uint16(0x7FFF)  # |V|: clear the bf16 sign bit
    A = oatt.prefill_attention(_storage(q), run.k_pool, absv, tables, lens, w.query_start())
    assert_within_prefill_bound(out, ref, A, what)


def _w(shape, variant="plain", **extra):
    hq, hkv, d, bs = shape
    return Workload("c7_prefill_bf16", variant=variant,
                    overrides=dict(SMALL, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, **extra))


@pytest.mark.parametrize("shape", SHAPES, ids=[f"hq{a}-hkv{b}-d{c}-bs{e}" for a, b, c, e in SHAPES])
def test_prefill_matches_oracle(shape):
    w = _w(shape)
    say(f"prefill {shape}: chunks {w.chunk_lens}")
    cache = product_cache(w)
    run = OracleRun(w)
    out, slots, _ = product_prefill_step(cache, w, 0)
    o_slots, _ = run.prefill_step(0)
    assert slots.tolist() == o_slots
    assert_pools_equal(cache, run)
    _check(run, w, out, 0, f"prefill {shape}")


@pytest.mark.parametrize("variant", ["q64", "q512", "large"])
def test_prefill_stress_values(variant):
    w = _w((64, 8, 128, 16), variant)
    say(f"prefill stress {variant}")
    cache = product_cache(w)
    run = OracleRun(w)
    out, _, _ = product_prefill_step(cache, w, 0)
    run.prefill_step(0)
    _check(run, w, out, 0, f"prefill {variant}")


def test_prefill_ignores_nan_in_unused_slots_and_chains_chunks():
    from paged_kv_cache_230_amd import PagedKVCache

    w = _w((32, 8, 128, 32), "q64")

    c = w.config
    cache = PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, "cuda", w.free_order)
    cache.k_cache.fill_(float("nan"))
    cache.v_cache.fill_(float("nan"))
    for op in w.setup_ops:
        cache.apply(op, w.kv)
    run = OracleRun(w)
    for k in range(2):  # the second chunk attends over the history and the first chunk
        out, _, _ = product_prefill_step(cache, w, k)
        run.prefill_step(k)
        _check(run, w, out, k, f"prefill NaN pool, chunk {k}")


def test_prefill_full_size_sampled_rows():
    w = Workload("c7_prefill_bf16")
    say(f"prefill full size: {w.num_seqs} sequences, chunks {min(w.chunk_lens)}..{max(w.chunk_lens)}")
    cache = product_cache(w)
    run = OracleRun(w, materialize=False)
    out, _, _ = product_prefill_step(cache, w, 0)
    run.prefill_step(0)
    q = w.prefill_q(0)
    qs = w.query_start()
    rng = np.random.default_rng(0)
    rows = set()
    for s in range(w.num_seqs):  # first, last and two random rows of every chunk
        rows |= {int(qs[s]), int(qs[s + 1]) - 1, *rng.integers(qs[s], qs[s + 1], 2).tolist()}
    rows = sorted(rows)
    ref = np.stack([run.logical_prefill_row(q, r) for r in rows])
    absv = np.stack([run.logical_prefill_row(q, r, abs_v=True) for r in rows])
    assert_within_prefill_bound(out[rows], ref, absv, "prefill full size, sampled rows")
    assert torch.isfinite(out.float()).all()


def test_prefill_rejects_unsupported():
    import paged_kv_cache_230_amd as pkv

    k, v = pkv.new_pools(4, 1, 64, 16, torch.float32, "cuda")
    q = torch.zeros(2, 1, 64, device="cuda")
    t = torch.zeros(1, 4, dtype=torch.int32, device="cuda")
    l = torch.full((1,), 2, dtype=torch.int32, device="cuda")
    qs = torch.tensor([0, 2], dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PKVError) as e:
        pkv.paged_attention_prefill(torch.empty_like(q), q, k, v, t, l, qs, 2)
    assert "bf16" in str(e.value)
