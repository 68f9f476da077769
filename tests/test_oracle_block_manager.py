"""Pins for the oracle's block-manager model (CPU only).

The model is checked against invariants and closed forms the pages fix,
never against itself: a recount of every reference from the tables after
each operation, on-demand growth (L tokens hold ceil(L/bs) blocks), copy on
write only for shared blocks, immediate reuse of released blocks, and the
block count of the shared-prefix workload in closed form.
"""
import copy
import math

import numpy as np
import pytest

import oracle.pool as pool
from oracle.block_manager import BlockManagerModel, Capacity, InvalidArg, OutOfBlocks, UnknownSeq
from oracle.runner import OracleRun
from workloads import Workload


def test_scripted_allocation_order():
    # free order [3,1,4,0,5,2]: 3 is handed out first
    bm = BlockManagerModel(6, 4, [3, 1, 4, 0, 5, 2])
    bm.add_seq(10)
    slots, pairs = bm.append_slots([10], [6])
    assert slots == [12, 13, 14, 15, 4, 5] and pairs == []  # blocks 3 then 1
    assert bm.tables[10] == [3, 1] and bm.num_free() == 4
    bm.add_seq(11)
    slots, _ = bm.append_slots([11, 10], [1, 3])
    assert slots == [16, 6, 7, 0]  # 11 -> block 4; 10 fills block 1 then takes block 0
    bm.free_seq(10)  # releases 3, 1, 0 in logical order: 0 is on top
    assert bm.free_stack()[-3:] == [3, 1, 0]
    bm.add_seq(12)
    s, _ = bm.append_slots([12], [1])
    assert s == [0]  # the most recently released block is reused first
    bm.check_invariants()


def test_on_demand_growth_and_sixty_tokens():
    bm = BlockManagerModel(64, 16)
    bm.add_seq(0)
    for _ in range(60):
        bm.append_slots([0])
        bm.check_invariants()
    assert len(bm.tables[0]) == math.ceil(60 / 16) == 4  # 60 tokens, not max_context
    assert bm.num_free() == 60


def test_fork_and_copy_on_write_rules():
    bm = BlockManagerModel(16, 4)
    bm.add_seq(0)
    bm.append_slots([0], [6])  # two blocks, the second half full
    b0, b1 = bm.tables[0]
    bm.fork(0, 1, 6)
    bm.fork(0, 2, 6)
    assert bm.refcount[b0] == 3 and bm.refcount[b1] == 3
    slots, pairs = bm.append_slots([1, 2, 0], [1, 1, 1])
    # 1 and 2 copy the shared partial block; 0 is then its last holder and writes in place
    assert len(pairs) == 2 and all(src == b1 for src, _ in pairs)
    assert bm.tables[0][1] == b1 and bm.refcount[b1] == 1
    assert slots[2] == b1 * 4 + 2
    assert bm.refcount[b0] == 3  # the full shared block is never copied
    bm.check_invariants()


def test_full_shared_block_allocates_instead_of_copying():
    bm = BlockManagerModel(8, 4)
    bm.add_seq(0)
    bm.append_slots([0], [8])
    bm.fork(0, 1, 8)
    _, pairs = bm.append_slots([1])
    assert pairs == [] and len(bm.tables[1]) == 3
    bm.check_invariants()


def test_fork_inside_a_block():
    bm = BlockManagerModel(8, 4)
    bm.add_seq(0)
    bm.append_slots([0], [7])
    bm.fork(0, 1, 5)  # child shares ceil(5/4) = 2 blocks
    assert bm.tables[1] == bm.tables[0][:2] and bm.lens[1] == 5
    slots, pairs = bm.append_slots([1])
    assert pairs == [(bm.tables[0][1], bm.tables[1][1])]
    assert slots == [bm.tables[1][1] * 4 + 1]
    bm.check_invariants()


def test_cow_leaves_source_block_untouched():
    rng = np.random.default_rng(5)
    bs, H, d = 4, 2, 8
    bm = BlockManagerModel(8, bs)
    k, v = pool.new_pools(8, H, d, bs, np.float32)
    bm.add_seq(0)
    slots, _ = bm.append_slots([0], [6])
    kt = rng.standard_normal((6, H, d)).astype(np.float32)
    pool.append(k, v, kt, kt, slots)
    bm.fork(0, 1, 6)
    src = bm.tables[0][1]
    before_k, before_v = k[src].copy(), v[src].copy()
    slots, pairs = bm.append_slots([1])
    pool.copy_blocks(k, v, pairs)
    new = rng.standard_normal((1, H, d)).astype(np.float32)
    pool.append(k, v, new, new, slots)
    assert np.array_equal(k[src], before_k) and np.array_equal(v[src], before_v)
    kg, _ = pool.gather(k, v, bm.tables[1], 7)
    assert np.array_equal(kg[:6], kt) and np.array_equal(kg[6], new[0])


def test_out_of_blocks_is_atomic():
    bm = BlockManagerModel(5, 4)
    bm.add_seq(0)
    bm.add_seq(1)
    bm.append_slots([0], [7])  # 2 blocks in use, 3 free
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.append_slots([0, 1], [2, 13])  # 1 + 4 blocks > 3 free
    assert bm.__dict__ == snap
    bm.append_slots([0, 1], [2, 8])  # 1 + 2 blocks: exactly fits
    assert bm.num_free() == 0


def test_cow_with_empty_pool_is_atomic():
    bm = BlockManagerModel(2, 4)
    bm.add_seq(0)
    bm.append_slots([0], [6])
    bm.fork(0, 1, 6)
    snap = copy.deepcopy(bm.__dict__)
    with pytest.raises(OutOfBlocks):
        bm.append_slots([1])
    assert bm.__dict__ == snap


def test_errors():
    bm = BlockManagerModel(4, 4)
    bm.add_seq(0)
    with pytest.raises(InvalidArg):
        bm.add_seq(0)
    with pytest.raises(UnknownSeq):
        bm.append_slots([9])
    with pytest.raises(InvalidArg):
        bm.append_slots([0, 0])
    with pytest.raises(InvalidArg):
        bm.fork(0, 1, 3)  # beyond the parent's length
    with pytest.raises(UnknownSeq):
        bm.free_seq(5)
    with pytest.raises(Capacity):
        bm.append_slots([0], [3], slot_capacity=2)
    bm.append_slots([0], [5])
    with pytest.raises(Capacity):
        bm.block_tables([0], 1)
    with pytest.raises(InvalidArg):
        BlockManagerModel(3, 4, [0, 0, 1])


def test_random_operations_keep_invariants():
    rng = np.random.default_rng(230)
    for trial in range(20):
        nb, bs = int(rng.integers(4, 40)), int(rng.choice([1, 2, 4, 16]))
        bm = BlockManagerModel(nb, bs, rng.permutation(nb))
        live, nxt = [], 0
        for _ in range(200):
            op = rng.integers(0, 4)
            try:
                if op == 0 or not live:
                    bm.add_seq(nxt)
                    live.append(nxt)
                    nxt += 1
                elif op == 1:
                    k = int(rng.integers(1, len(live) + 1))
                    sids = list(rng.choice(live, size=k, replace=False))
                    ntoks = list(rng.integers(0, 2 * bs + 2, size=k))
                    before = copy.deepcopy(bm.__dict__)
                    try:
                        bm.append_slots(sids, ntoks)
                    except OutOfBlocks:
                        assert bm.__dict__ == before
                elif op == 2:
                    p = int(rng.choice(live))
                    bm.fork(p, nxt, int(rng.integers(0, bm.lens[p] + 1)))
                    live.append(nxt)
                    nxt += 1
                else:
                    s = int(rng.choice(live))
                    bm.free_seq(s)
                    live.remove(s)
            finally:
                bm.check_invariants()


def test_prefix_workload_closed_form():
    """Shared-prefix workload: blocks in use and copies follow from the lengths alone."""
    w = Workload("c4_prefix_bf16", overrides=dict(num_prompts=12, n_samples=4, prefix_len=64, suffix_max=40,
                                                   num_blocks=400))
    run = OracleRun(w, materialize=False)
    bs, P, n = 16, 12, 4
    prefix_blocks = 64 // bs
    assert all(run.bm.refcount[b] == P * n for b in run.bm.tables[w.decode_seqs[0]][:prefix_blocks])
    used_before = prefix_blocks + sum(math.ceil(int(s) / bs) for s in w.suffix_lens)
    assert run.bm.num_free() == 400 - used_before
    _, pairs = run.step(0)
    partial = [int(s) for s in w.suffix_lens if (64 + int(s)) % bs]
    assert len(pairs) == (n - 1) * len(partial)
    fresh = n * (P - len(partial))
    assert run.bm.num_free() == 400 - used_before - len(pairs) - fresh
    # Saving against private copies: n*P samples each holding their whole
    # prompt would need sum_p n*ceil((prefix+s_p)/bs) blocks; sharing saves
    # (n*P - 1) copies of the prefix and (n - 1) copies of each suffix.
    private = sum(n * math.ceil((64 + int(s)) / bs) for s in w.suffix_lens)
    saved = (n * P - 1) * prefix_blocks + (n - 1) * sum(math.ceil(int(s) / bs) for s in w.suffix_lens)
    assert private - used_before == saved
    run.bm.check_invariants()


def test_kv_bytes_per_token_figure():
    """Llama-3.1-70B in bf16 holds about 0.31 MB of cache per token (aitalk page, introduction)."""
    layers, kv_heads, head_dim, two, bf16 = 80, 8, 128, 2, 2
    per_token = layers * kv_heads * head_dim * two * bf16
    assert per_token == 327_680 and abs(per_token / 2**20 - 0.3125) < 1e-12
    assert abs(per_token * 128_000 / 1e9 - 41.9) < 0.05  # "128k tokens ~ 40 GB"
