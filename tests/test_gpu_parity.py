"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Append, copy-on-write copy and bookkeeping must match bit for bit; decode
attention within the tolerances in ``helpers.TOL``.  Inputs are the seeded
workloads of ``workloads.py`` at their full sizes (the 70B-shaped 32k layer
on sampled sequences) and scaled-down variants that still span several
blocks, partitions and a ragged tail.
"""
import math

import numpy as np
import pytest
import torch

from helpers import (TOL, assert_close, assert_pools_equal, bits, errors, product_cache, product_step, say,
                     storage_np, to_f64)
from oracle.runner import OracleRun
from workloads import Workload

pytestmark = pytest.mark.gpu


def _tables_match(cache, run, w):
    _, _, t, l = cache.tables(w.decode_seqs)
    rt, rl = run.tables(t.shape[1])
    assert np.array_equal(t, rt) and np.array_equal(l, rl), "block tables differ from the oracle's"


def _full_parity(w, partition_sizes, steps=None, check_steps=None):
    c = w.config
    say(f"case {w.name} variant={w.variant} seqs={w.num_seqs} P={partition_sizes}")
    cache = product_cache(w)
    run = OracleRun(w)
    assert_pools_equal(cache, run)
    steps = c.steps if steps is None else steps
    check_steps = range(steps) if check_steps is None else check_steps
    for k in range(steps):
        kn, vn = w.kv(("step", k))
        slots, pairs = cache.append(w.decode_seqs, [1] * w.num_seqs, kn, vn)
        rslots, rpairs = run.step(k)
        assert slots.tolist() == rslots and pairs.tolist() == [list(p) for p in rpairs]
        if k not in check_steps:
            continue
        _tables_match(cache, run, w)
        q = w.q(k)
        ref = run.attention(q)
        for P in partition_sizes:
            out = cache.decode(q.cuda(), w.decode_seqs, partition_size=P)
            torch.cuda.synchronize()
            assert_close(out, ref, c.dtype, f"{w.name}/{w.variant} step {k} P={P}")
    torch.cuda.synchronize()
    assert_pools_equal(cache, run)
    return cache, run


def test_c1_tiny_fp32_full():
    _full_parity(Workload("c1_tiny_f32"), [0, 16, 32, 48])


def test_c1_shape_edge_lengths_fp32():
    # lengths around block boundaries, a single token, and an empty sequence
    w = Workload("c1_tiny_f32", overrides=dict(lengths=[1, 2, 15, 16, 17, 31, 32, 33, 48, 200]))
    _full_parity(w, [0, 16, 64])


def test_c2_8b_bf16_full():
    _full_parity(Workload("c2_8b_bf16"), [0, 256])


@pytest.mark.parametrize("variant", ["q64", "q512", "needle", "large"])
def test_c2_shape_stress_variants(variant):
    w = Workload("c2_8b_bf16", variant=variant, overrides=dict(num_seqs=12, num_blocks=4000))
    _full_parity(w, [0, 512])


def test_c4_prefix_sharing_full():
    cache, run = _full_parity(Workload("c4_prefix_bf16"), [0])
    n_cow = sum(len(p) for p in run.cow_log)
    say(f"  c4 copy-on-write pairs over the run: {n_cow}")
    assert n_cow > 0


def test_c5_mixed_bs32_full_10_steps():
    _full_parity(Workload("c5_mixed_bs32_bf16"), [0], check_steps=(0, 9))


@pytest.mark.parametrize("P", [512, 2048, 0])
def test_c3_shape_scaled_split_partitions(P):
    w = Workload("c3_70b_32k_bf16", overrides=dict(lengths=[8192, 5000, 1, 513], num_blocks=1300))
    _full_parity(w, [P])


def test_c3_full_size_every_sequence():
    """The 70B-shaped 32k layer at full size, default launch configuration;
    the output of every sequence against the oracle from its logical tokens."""
    w = Workload("c3_70b_32k_bf16")
    say("case c3 full: building the cache")
    cache = product_cache(w)
    run = OracleRun(w, materialize=False)
    out, slots, pairs = product_step(cache, w, 0)
    rslots, _ = run.step(0)
    assert slots.tolist() == rslots
    q = w.q(0)
    ref = np.stack([run.logical_attention(q, s) for s in range(w.num_seqs)])
    assert_close(out, ref, "bf16", "c3 full, all 16 sequences")


def _fused_parity(w, partition_sizes, steps):
    """Decode steps as the benchmark runs them: the block manager reserves the
    slots, copy-on-write copies run, then one paged_attention_decode_append
    call appends and decodes; outputs against the oracle element by element,
    pools bit for bit at the end."""
    import paged_kv_cache_230_amd as pkv

    c = w.config
    say(f"case fused {w.name} variant={w.variant} seqs={w.num_seqs} P={partition_sizes}")
    cache = product_cache(w)
    run = OracleRun(w)
    for k in range(steps):
        slots, pairs = cache.bm.append_slots(w.decode_seqs, [1] * w.num_seqs)
        rslots, rpairs = run.step(k)
        assert slots.tolist() == rslots and pairs.tolist() == [list(p) for p in rpairs]
        if pairs.shape[0]:
            pkv.paged_kv_copy_blocks(cache.k_cache, cache.v_cache, torch.from_numpy(pairs.copy()).cuda())
        tables, lens, _, lh = cache.tables(w.decode_seqs)
        kn, vn = w.kv(("step", k))
        q = w.q(k)
        ref = run.attention(q)
        for P in partition_sizes:  # a repeated append rewrites the same bytes
            out = torch.full(q.shape, float("nan"), dtype=q.dtype, device="cuda")
            pkv.paged_attention_decode_append(out, q.cuda(), kn.cuda(), vn.cuda(), cache.k_cache, cache.v_cache,
                                              tables, lens, int(lh.max()), partition_size=P)
            torch.cuda.synchronize()
            assert_close(out, ref, c.dtype, f"{w.name}/{w.variant} fused step {k} P={P}")
    assert_pools_equal(cache, run)


@pytest.mark.parametrize("variant", ["q64", "q512", "needle", "large"])
def test_c3_shape_stress_variants_fused(variant):
    """Group size 8 (64 query / 8 kv heads) under scores that matter: larger
    query scales, a planted needle key, logits in the hundreds (the rescale
    path).  Long sequences split into many pieces (P = 512) or over the
    default one-round split, with a single-token and a ragged sequence."""
    w = Workload("c3_70b_32k_bf16", variant=variant,
                 overrides=dict(lengths=[8192, 5000, 1, 513], num_blocks=1300))
    _fused_parity(w, [0, 512], steps=2)


@pytest.mark.parametrize("variant", ["q64", "q512", "needle", "large"])
def test_c5_shape_stress_variants_fused(variant):
    """The mixed-length block-32 shape (64 query / 8 kv heads) under the same
    stress values: 24 log-uniform lengths over 16..16384, two steps."""
    w = Workload("c5_mixed_bs32_bf16", variant=variant, overrides=dict(num_seqs=24, steps=2))
    _fused_parity(w, [0, 512], steps=2)


def test_split_matches_unsplit_fp32():
    w = Workload("c1_tiny_f32", overrides=dict(lengths=[3000, 1000, 17], num_blocks=400))
    cache = product_cache(w)
    out_split, _, _ = product_step(cache, w, 0, partition_size=256)
    tables, lens, _, lh = cache.tables(w.decode_seqs)
    from paged_kv_cache_230_amd import paged_attention_decode

    out_one = torch.empty_like(out_split)
    q = w.q(0).cuda()
    # partition_size >= num_seqs * max_len: one workgroup per kv head, nothing split
    paged_attention_decode(out_one, q, cache.k_cache, cache.v_cache, tables, lens, int(lh.max()),
                           partition_size=len(lh) * int(lh.max()))
    paged_attention_decode(out_split, q, cache.k_cache, cache.v_cache, tables, lens, int(lh.max()),
                           partition_size=256)
    torch.cuda.synchronize()
    diff = (out_split - out_one).abs().max().item()
    say(f"  split vs unsplit max diff {diff:.3e}")
    assert diff <= 2e-6 * max(1.0, out_one.abs().max().item())


def test_block_permutation_is_bit_invariant():
    """Paging only moves data: a scrambled physical placement gives bit-identical outputs."""
    w1 = Workload("c2_8b_bf16", variant="q512", overrides=dict(num_seqs=8, num_blocks=3000))
    w2 = Workload("c2_8b_bf16", variant="q512", overrides=dict(num_seqs=8, num_blocks=3000))
    w2.free_order = np.arange(w2.num_blocks, dtype=np.int32)  # contiguous placement
    outs = []
    for w in (w1, w2):
        cache = product_cache(w)
        out, _, _ = product_step(cache, w, 0, partition_size=512)
        outs.append(storage_np(out))
    assert np.array_equal(outs[0], outs[1])


def test_shared_prefix_equals_private_copies_bitwise():
    w = Workload("c4_prefix_bf16", variant="q64", overrides=dict(num_prompts=6, n_samples=4, num_blocks=5000))
    shared = product_cache(w)
    out_shared, _, pairs = product_step(shared, w, 0)
    assert pairs.shape[0] > 0 or all((2048 + int(s)) % 16 == 0 for s in w.suffix_lens)
    # Same logical content, every sequence holding private blocks.
    from paged_kv_cache_230_amd import PagedKVCache

    c = w.config
    priv = PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, "cuda",
                        w.free_order)
    pk, pv = w.kv(("prefix",))
    i = 0
    for p, s in enumerate(w.suffix_lens):
        sk, sv = w.kv(("suffix", p))
        for _ in range(4):
            sid = w.decode_seqs[i]
            priv.add_seq(sid)
            priv.append([sid], [2048 + int(s)], torch.cat([pk, sk]), torch.cat([pv, sv]))
            i += 1
    out_priv, _, pairs2 = product_step(priv, w, 0)
    assert pairs2.shape[0] == 0
    assert np.array_equal(storage_np(out_shared), storage_np(out_priv))


def test_nan_in_unused_slots_does_not_leak():
    """Slots past a sequence's length may hold anything (here NaN)."""
    w = Workload("c5_mixed_bs32_bf16", variant="q64", overrides=dict(num_seqs=10, steps=1))
    c = w.config
    from paged_kv_cache_230_amd import PagedKVCache

    cache = PagedKVCache(w.num_blocks, c.num_kv_heads, c.head_dim, c.block_size, c.torch_dtype, "cuda", w.free_order)
    cache.k_cache.view(torch.int16).fill_(0x7FC1)
    cache.v_cache.view(torch.int16).fill_(0x7FC1)
    for op in w.setup_ops:
        cache.apply(op, w.kv)
    run = OracleRun(w, materialize=False)
    out, _, _ = product_step(cache, w, 0)
    run.step(0)
    q = w.q(0)
    ref = np.stack([run.logical_attention(q, s) for s in range(w.num_seqs)])
    assert_close(out, ref, "bf16", "NaN-filled unused slots")


def test_zero_length_sequences_give_zero_rows():
    from paged_kv_cache_230_amd import PagedKVCache, paged_attention_decode

    torch.manual_seed(0)
    cache = PagedKVCache(64, 2, 128, 16, torch.bfloat16, "cuda")
    for sid in range(3):
        cache.add_seq(sid)
    k = (torch.randn(40, 2, 128) * 0.1).bfloat16()
    cache.append([1], [40], k, k)
    tables, lens, _, lh = cache.tables([0, 1, 2], max_blocks=4)
    q = torch.randn(3, 8, 128).bfloat16().cuda()
    out = torch.full_like(q, float("nan"))
    paged_attention_decode(out, q, cache.k_cache, cache.v_cache, tables, lens, 64, partition_size=16)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.all(o[0] == 0) and torch.all(o[2] == 0) and torch.isfinite(o[1]).all()


def test_append_and_copy_move_arbitrary_bits():
    """Append and block copy are byte moves: any bit pattern (NaN payloads included) survives."""
    from paged_kv_cache_230_amd import new_pools, paged_kv_append, paged_kv_copy_blocks
    import oracle.pool as opool

    g = torch.Generator().manual_seed(5)
    for dtype, bs in ((torch.bfloat16, 16), (torch.bfloat16, 32), (torch.float32, 16), (torch.float32, 32)):
        nb, H, d, T = 37, 3, 128 if dtype == torch.bfloat16 else 64, 150
        k, v = new_pools(nb, H, d, bs, dtype)
        ib = torch.int16 if dtype == torch.bfloat16 else torch.int32
        lo, hi = (-(1 << 15), 1 << 15) if ib == torch.int16 else (-(1 << 31), (1 << 31) - 1)
        kn = torch.randint(lo, hi, (T, H, d), generator=g, dtype=ib)
        vn = torch.randint(lo, hi, (T, H, d), generator=g, dtype=ib)
        slots = torch.randperm(nb * bs, generator=g)[:T].to(torch.int32)
        slots[::7] = -1  # skipped tokens
        paged_kv_append(kn.cuda().view(dtype), vn.cuda().view(dtype), k, v, slots.cuda())
        pairs = torch.tensor([[3, 30], [5, 31], [0, 36]], dtype=torch.int32)
        paged_kv_copy_blocks(k, v, pairs.cuda())
        torch.cuda.synchronize()
        sd = np.uint16 if dtype == torch.bfloat16 else np.float32
        ok, ov = opool.new_pools(nb, H, d, bs, sd)
        nk = kn.numpy().view(sd)
        nv = vn.numpy().view(sd)
        opool.append(ok, ov, nk, nv, slots.numpy())
        opool.copy_blocks(ok, ov, pairs.numpy())
        assert np.array_equal(bits(storage_np(k)), bits(ok)), f"K pool {dtype} bs{bs}"
        assert np.array_equal(bits(storage_np(v)), bits(ov)), f"V pool {dtype} bs{bs}"
