"""Prefix caching end to end on the GPU: cached admissions share the blocks
an earlier request of the same tenant computed (revived from the eviction
list), the rest of each prompt is appended, and decode attention over the
shared blocks must equal the oracle's, both over the oracle's own pool and
over each request's logical (contiguous) K/V, which no paging touches."""
import numpy as np
import pytest
import torch

from helpers import TOL, assert_close, assert_pools_equal, product_cache, product_step, say
from oracle.runner import OracleRun
from test_gpu_stage import Staged
from workloads import Workload

pytestmark = pytest.mark.gpu

SMALL = dict(prefix_len=160, num_prompts=12, suffix_max=40)


def _tight(overrides, steps):
    """The smallest pool that holds the final state: the warm requests'
    cached blocks must then be evicted on the way."""
    loose = Workload("c6_prefix_cache_bf16", overrides=dict(overrides, num_blocks=4000))
    run = OracleRun(loose, materialize=False)
    for k in range(steps):
        run.step(k)
    in_use = loose.num_blocks - run.bm.num_free()
    return in_use + 1, len(run.bm.evictable())


def test_cached_admission_and_decode_small_tight_pool():
    steps = 3
    nb, evictable_loose = _tight(SMALL, steps)
    w = Workload("c6_prefix_cache_bf16", overrides=dict(SMALL, num_blocks=nb))
    say(f"c6 small: {w.num_seqs} requests, pool {nb} blocks")
    cache = product_cache(w)
    run = OracleRun(w)
    assert cache.admitted == run.admitted
    assert all(run.admitted[s] == 160 for s in w.decode_seqs)
    for k in range(steps):
        out, slots, pairs = product_step(cache, w, k)
        o_slots, o_pairs = run.step(k)
        assert slots.tolist() == o_slots and pairs.tolist() == [list(p) for p in o_pairs]
        assert_close(out, run.attention(w.q(k)), "bf16", f"c6 small step {k} vs oracle pool")
        for i in range(w.num_seqs):
            ref = run.logical_attention(w.q(k), i)
            assert_close(out[i:i + 1], ref[None], "bf16", f"c6 small step {k} seq {i} vs logical K/V")
    assert_pools_equal(cache, run)
    assert cache.bm.evictable() == run.bm.evictable()
    assert len(run.bm.evictable()) < evictable_loose  # cached blocks were evicted to make room
    run.bm.check_invariants()


def test_cached_admission_full_size_logical():
    """50 requests, 2048-token system prompt over two tenants (bs 16)."""
    w = Workload("c6_prefix_cache_bf16")
    say(f"c6 full: {w.num_seqs} requests")
    cache = product_cache(w)
    run = OracleRun(w, materialize=False)
    assert cache.admitted == run.admitted
    tables, lens, _, _ = cache.tables(w.decode_seqs)
    rows, olens = run.tables(max_blocks=tables.shape[1])
    assert np.array_equal(tables.cpu().numpy(), rows) and np.array_equal(lens.cpu().numpy(), olens)
    out, _, _ = product_step(cache, w, 0)
    run.step(0)
    q = w.q(0)
    for i in range(w.num_seqs):
        assert_close(out[i:i + 1], run.logical_attention(q, i)[None], "bf16", f"c6 full seq {i} vs logical K/V")


def test_stage_step_with_token_ids_registers_like_the_model():
    w = Workload("c6_prefix_cache_bf16", overrides=dict(SMALL, num_blocks=600))
    cache = product_cache(w)
    run = OracleRun(w, materialize=False)
    st = Staged(w.num_seqs, maxb=64)
    for k in range(2 * 16):  # two blocks' worth of steps: every sequence fills blocks
        ids = w.step_tokens(k)
        n_cow, max_len = st.step_ids(cache.bm, w.decode_seqs, ids)
        run.step(k)
        assert n_cow == 0 and max_len == max(run.bm.lens[s] for s in w.decode_seqs)
    torch.cuda.synchronize()
    t = st.tables.cpu().numpy()
    for i, sid in enumerate(w.decode_seqs):
        nb = len(run.bm.tables[sid])
        assert t[i, :nb].tolist() == run.bm.tables[sid]
    assert cache.bm.num_cached() == run.bm.num_cached()
    for b in range(w.num_blocks):
        assert cache.bm.cached_digest(b) == run.bm.block_digest[b]


@pytest.mark.parametrize("name,over", [
    ("c6_prefix_cache_bf16", SMALL),
    ("c4_prefix_bf16", dict(prefix_len=300, num_prompts=4, n_samples=4, suffix_max=40, num_blocks=400)),
    ("c2_8b_bf16", dict(lengths=[300, 17, 1, 64, 129, 2000], num_blocks=400)),
    ("c5_mixed_bs32_bf16", dict(lengths=[16, 40, 33, 100, 1000, 64, 65, 31, 2], num_blocks=80)),
    ("c1_tiny_f32", {}),
])
def test_shared_blocks_flag_changes_only_the_schedule(name, over):
    """The decode calls' cache-policy flag (PKV_DECODE_SHARED_BLOCKS: cached
    loads, one kv head per XCD; else non-temporal streaming loads and, at
    block size 16, every head on every XCD) gives bit-identical outputs, on
    a batch whose sequences share prompt blocks and on one whose blocks are
    all private; both equal the oracle."""
    import paged_kv_cache_230_amd as pkv

    w = Workload(name, overrides=over)
    cache = product_cache(w)
    run = OracleRun(w)
    kn, vn = w.kv(("step", 0))
    cache.append(w.decode_seqs, [1] * w.num_seqs, kn, vn, token_ids=w.step_tokens(0))
    run.step(0)
    shared = cache.bm.num_shared()
    say(f"case {name}: {w.num_seqs} sequences, {shared} shared blocks")
    if name in ("c6_prefix_cache_bf16", "c4_prefix_bf16"):
        assert shared > 0
    else:
        assert shared == 0
    kind = "f32" if w.config.dtype == "f32" else "bf16"
    q = w.q(0).to(cache.device)
    tables, lens, _, lh = cache.tables(w.decode_seqs)
    outs = {}
    for flag in (False, True):
        for part in (0, 64):
            out = torch.full_like(q, float("nan"))
            pkv.device_status()
            pkv.paged_attention_decode(out, q, cache.k_cache, cache.v_cache, tables, lens, int(lh.max()),
                                       partition_size=part, shared_blocks=flag)
            assert pkv.device_status() == 0
            outs[(flag, part)] = out
    torch.cuda.synchronize()
    for part in (0, 64):
        a, b = outs[(False, part)], outs[(True, part)]
        bits = torch.int32 if a.dtype == torch.float32 else torch.int16
        assert torch.equal(a.view(bits), b.view(bits)), f"{name} partition {part}: outputs differ between the cache policies"
        assert_close(b, run.attention(w.q(0)), kind, f"{name} partition {part} vs oracle")
