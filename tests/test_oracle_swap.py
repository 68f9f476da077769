"""Pins for the oracle's swap to host memory (CPU only).

The pages fix only that, when GPU memory runs out even with paging, pages
go to CPU RAM and come back when needed ("PagedAttention — Gestion mémoire
pour LLM à long contexte", *Mode d'échec*, glossary *Page eviction*).  The
pins: a sequence's logical K/V survive a swap-out / swap-in round trip bit
for bit (gathered through its old and new tables), the blocks it frees are
immediately reusable by others (and those others' K/V stay intact), shared
prefix blocks stay on the GPU for their other holders, counts and
atomicity, and the invariants after random mixes of swaps with the other
operations.
"""
import random

import numpy as np
import pytest

import oracle.pool as pool
from oracle.block_manager import BlockManagerModel, InvalidArg, OutOfBlocks, UnknownSeq

BS, H, D = 4, 2, 8


def _pools(n):
    return pool.new_pools(n, H, D, BS, np.float32)


def _write(bm, k, v, sid, n, rng):
    slots, pairs = bm.append_slots([sid], [n])
    pool.copy_blocks(k, v, pairs)
    kt = rng.standard_normal((n, H, D)).astype(np.float32)
    vt = rng.standard_normal((n, H, D)).astype(np.float32)
    pool.append(k, v, kt, vt, slots)


def _logical(bm, k, v, sid):
    return pool.gather(k, v, np.array(bm.tables[sid]), bm.lens[sid])


def test_round_trip_preserves_logical_kv_and_frees_blocks():
    rng = np.random.default_rng(1)
    bm = BlockManagerModel(12, BS, list(range(12)))
    bm.add_host_pool(6)
    k, v = _pools(12)
    hk, hv = _pools(6)
    bm.add_seq(0)
    bm.add_seq(1)
    _write(bm, k, v, 0, 10, rng)  # 3 blocks
    _write(bm, k, v, 1, 5, rng)
    before = [x.copy() for x in _logical(bm, k, v, 0)]
    pairs = bm.swap_out(0)
    assert [g for g, _ in pairs] == [0, 1, 2] and [h for _, h in pairs] == [0, 1, 2]
    pool.swap_copy(k, v, hk, hv, pairs)
    assert bm.num_free() == 12 - 2 and bm.num_free_host() == 3
    with pytest.raises(InvalidArg):
        bm.append_slots([0], [1])
    with pytest.raises(InvalidArg):
        bm.block_tables([0], 8)
    # another sequence reuses the freed blocks and overwrites them
    bm.add_seq(2)
    _write(bm, k, v, 2, 12, rng)
    other = [x.copy() for x in _logical(bm, k, v, 1)]
    back = bm.swap_in(0)
    assert [h for h, _ in back] == [0, 1, 2]
    pool.swap_copy(hk, hv, k, v, back)
    after = _logical(bm, k, v, 0)
    assert all(np.array_equal(a, b) for a, b in zip(before, after))
    assert all(np.array_equal(a, b) for a, b in zip(other, _logical(bm, k, v, 1)))
    assert bm.num_free_host() == 6
    bm.append_slots([0], [1])  # usable again
    bm.check_invariants()


def test_shared_prefix_stays_on_gpu_for_its_other_holders():
    rng = np.random.default_rng(2)
    bm = BlockManagerModel(16, BS)
    bm.add_host_pool(8)
    k, v = _pools(16)
    hk, hv = _pools(8)
    bm.add_seq(0)
    _write(bm, k, v, 0, 8, rng)
    bm.fork(0, 1, 8)
    prefix = list(bm.tables[0])
    pairs = bm.swap_out(1)
    pool.swap_copy(k, v, hk, hv, pairs)
    assert [g for g, _ in pairs] == prefix and all(bm.refcount[b] == 1 for b in prefix)
    assert bm.tables[0] == prefix
    back = bm.swap_in(1)
    pool.swap_copy(hk, hv, k, v, back)
    assert set(bm.tables[1]).isdisjoint(prefix)  # private copies now
    assert all(np.array_equal(a, b) for a, b in zip(_logical(bm, k, v, 0), _logical(bm, k, v, 1)))
    bm.check_invariants()


def test_swap_is_atomic_and_validated():
    bm = BlockManagerModel(6, BS)
    with pytest.raises(InvalidArg):
        bm.add_host_pool(0)
    bm.add_host_pool(2)
    with pytest.raises(InvalidArg):
        bm.add_host_pool(2)
    bm.add_seq(0)
    bm.append_slots([0], [12])  # 3 blocks > 2 host blocks
    with pytest.raises(OutOfBlocks):
        bm.swap_out(0)
    assert bm.tables[0] and bm.num_free_host() == 2
    with pytest.raises(InvalidArg):
        bm.swap_in(0)  # not swapped out
    with pytest.raises(UnknownSeq):
        bm.swap_out(9)
    bm.add_seq(1)
    bm.append_slots([1], [4])
    bm.swap_out(1)
    bm.add_seq(2)
    bm.append_slots([2], [12])  # the pool is now full
    with pytest.raises(OutOfBlocks):
        bm.swap_in(1)
    assert 1 in bm.host_tables and bm.num_free() == 0
    bm.free_seq(1)  # a swapped-out sequence releases its host blocks
    assert bm.num_free_host() == 2
    bm.check_invariants()


def test_random_mix_keeps_invariants_and_contents():
    rng = np.random.default_rng(3)
    r = random.Random(3)
    bm = BlockManagerModel(40, BS, r.sample(range(40), 40))
    bm.add_host_pool(24)
    k, v = _pools(40)
    hk, hv = _pools(24)
    ref = {}  # sid -> logical (K, V) rows, kept by the test
    nxt = 0
    for _ in range(300):
        live = [s for s in bm.tables]
        op = r.random()
        try:
            if op < 0.25 or not live:
                bm.add_seq(nxt)
                ref[nxt] = (np.zeros((0, H, D), np.float32), np.zeros((0, H, D), np.float32))
                nxt += 1
            elif op < 0.55:
                sid = r.choice(live)
                if sid in bm.host_tables:
                    continue
                n = r.randint(1, 6)
                slots, pairs = bm.append_slots([sid], [n])
                pool.copy_blocks(k, v, pairs)
                kt = rng.standard_normal((n, H, D)).astype(np.float32)
                vt = rng.standard_normal((n, H, D)).astype(np.float32)
                pool.append(k, v, kt, vt, slots)
                ref[sid] = (np.concatenate([ref[sid][0], kt]), np.concatenate([ref[sid][1], vt]))
            elif op < 0.7:
                sid = r.choice(live)
                if sid in bm.host_tables or not bm.tables[sid]:
                    continue
                pool.swap_copy(k, v, hk, hv, bm.swap_out(sid))
            elif op < 0.85:
                swapped = list(bm.host_tables)
                if swapped:
                    sid = r.choice(swapped)
                    pool.swap_copy(hk, hv, k, v, bm.swap_in(sid))
            else:
                sid = r.choice(live)
                bm.free_seq(sid)
                del ref[sid]
        except OutOfBlocks:
            pass
        bm.check_invariants()
        for sid in bm.tables:
            if sid not in bm.host_tables and bm.lens[sid]:
                kk, vv = _logical(bm, k, v, sid)
                assert np.array_equal(kk, ref[sid][0]) and np.array_equal(vv, ref[sid][1])
