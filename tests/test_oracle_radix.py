"""Pins for the oracle's radix-tree prefix index (CPU only).

Against the pages ("PagedAttention et RadixAttention : parlons de KV
Cache", *RadixAttention : un arbre qui n'oublie pas*): the longest cached
prefix is found token by token (brute force: the longest common prefix with
the token sequences inserted so far), prefixes are stored once (an edge
splits exactly where two requests diverge, even inside a block, and the
split shares the blocks), least recently used leaves go first and nodes
that running requests depend on are never evicted.  Block-level effects
go through the block-manager model and its invariants.
"""
import random

import pytest

from oracle.block_manager import BlockManagerModel, InvalidArg, UnknownSeq
from oracle.radix import HOLDER_BASE, RadixCacheModel

BS = 16


def _serve(rc, sid, tokens):
    """One request: admit, append the uncached rest, insert, release, free."""
    m = rc.admit(sid, tokens)
    rc.bm.append_slots([sid], [len(tokens) - m])
    rc.insert(sid, tokens)
    rc.release(sid)
    rc.bm.free_seq(sid)
    return m


def _lcp(a, b):
    n = 0
    while n < len(a) and n < len(b) and a[n] == b[n]:
        n += 1
    return n


def test_token_granular_reuse_shares_the_partial_block():
    rc = RadixCacheModel(BlockManagerModel(64, BS))
    first = list(range(37))  # 2 full blocks + 5 tokens
    assert _serve(rc, 0, first) == 0
    req = first + [900] * 10
    m = rc.admit(1, req)
    assert m == 37  # token granular: beyond the last full block (chained block digests would give 32)
    holder = rc.nodes()[0].holder
    assert rc.bm.tables[1] == rc.bm.tables[holder][:3]
    slots, pairs = rc.bm.append_slots([1], [10])
    assert pairs == [(rc.bm.tables[holder][2], rc.bm.tables[1][2])]  # the partial block is copied on write
    rc.insert(1, req)
    rc.release(1)
    rc.check_invariants()


def test_split_inside_a_block_keeps_the_common_prefix_once():
    bm = BlockManagerModel(64, BS)
    rc = RadixCacheModel(bm)
    p = list(range(20))
    _serve(rc, 0, p + [1, 2, 3])
    _serve(rc, 1, p + [7, 8])
    nodes = rc.nodes()
    assert [len(n.edge) for n in nodes] == [20, 3, 2] and nodes[0].depth == 20
    inner = nodes[0].holder
    for leaf in nodes[1:]:
        assert bm.tables[leaf.holder][0] == bm.tables[inner][0]  # the full block is shared
    assert rc.match(p + [1, 2]) == 22 and rc.match(p + [9]) == 20 and rc.match([5]) == 0
    rc.check_invariants()


def test_matches_equal_brute_force_longest_common_prefix():
    r = random.Random(4)
    rc = RadixCacheModel(BlockManagerModel(4000, BS))
    inserted = []
    roots = [[r.randrange(3) for _ in range(r.randint(0, 40))] for _ in range(5)]
    for sid in range(60):
        toks = r.choice(roots) + [r.randrange(3) for _ in range(r.randint(1, 30))]
        expect = max([_lcp(toks, s) for s in inserted] + [0])
        assert rc.match(toks) == expect
        assert _serve(rc, sid, toks) == expect
        inserted.append(toks)
        rc.check_invariants()
    # every inserted sequence is found in full, and every node path is an inserted prefix
    assert all(rc.match(s) == len(s) for s in inserted)
    assert all(any(s[:len(p)] == p for s in inserted) for p in rc.paths())


def test_eviction_is_lru_over_unlocked_leaves_and_spares_shared_nodes():
    bm = BlockManagerModel(40, BS)
    rc = RadixCacheModel(bm)
    common = list(range(48))  # 3 blocks
    a, b, c = common + [1] * 32, common + [2] * 32, [7] * 64
    _serve(rc, 0, a)
    _serve(rc, 1, b)
    _serve(rc, 2, c)
    rc.admit(10, b)  # a running request depends on the common node and b's leaf
    held_before = bm.num_free()
    freed = rc.evict(held_before + 1)  # one more block is needed than is free
    assert len(freed) == 1 and rc.match(a) == 48  # a's leaf (oldest unlocked) went first, the shared node stays
    freed = rc.evict(10 ** 6)  # everything evictable
    assert rc.match(b) == len(b) and rc.match(c) == 0  # c's leaf evicted; b's path is locked
    rc.release(10)
    rc.evict(10 ** 6)
    assert rc.nodes() == [] and rc.match(b) == 0
    bm.free_seq(10)
    assert bm.num_free() == 40
    rc.check_invariants()


def test_errors():
    rc = RadixCacheModel(BlockManagerModel(8, BS))
    rc.admit(0, [1, 2])
    with pytest.raises(InvalidArg):
        rc.admit(0, [1])
    with pytest.raises(UnknownSeq):
        rc.release(5)
    with pytest.raises(UnknownSeq):
        rc.insert(9, [1])
    with pytest.raises(InvalidArg):
        rc.insert(0, [1, 2, 3])  # more tokens than the sequence holds
    assert HOLDER_BASE > 2 ** 60


def test_random_lifecycles_keep_invariants():
    r = random.Random(7)
    bm = BlockManagerModel(300, BS)
    rc = RadixCacheModel(bm)
    roots = [[r.randrange(4) for _ in range(r.randint(0, 50))] for _ in range(4)]
    running, admitted = {}, {}
    nxt = 0
    for _ in range(300):
        op = r.random()
        if op < 0.4 or not running:
            toks = r.choice(roots) + [r.randrange(4) for _ in range(r.randint(1, 40))]
            need = len(toks) // BS + 2
            if bm.num_free() < need:
                rc.evict(need)
            if bm.num_free() < need:
                continue
            m = rc.admit(nxt, toks)
            bm.append_slots([nxt], [len(toks) - m])
            running[nxt] = toks
            admitted[nxt] = m
            nxt += 1
        elif op < 0.7:
            sid = r.choice(list(running))
            rc.insert(sid, running[sid])
        else:
            sid = r.choice(list(running))
            toks = running.pop(sid)
            rc.insert(sid, toks)
            rc.release(sid)
            bm.free_seq(sid)
        rc.check_invariants()
        # the prefix a running request was admitted on is locked: never evicted
        assert all(rc.match(t) >= admitted[s] for s, t in running.items())


# ---------------------------------------------------------------- mutants
def _walk_whole_edges_only(self, tokens):
    node, i, path = self.root, 0, []
    while i < len(tokens):
        child = node.children.get(tokens[i])
        if child is None or tokens[i:i + len(child.edge)] != child.edge:
            break
        path.append(child)
        i += len(child.edge)
        node = child
    return path, i, len(path[-1].edge) if path else 0


_true_walk = RadixCacheModel._walk


def _walk_block_granular(self, tokens):
    path, i, used = _true_walk(self, tokens)
    return path, i - i % BS, used


def _evict_newest_first(self, num_blocks):
    freed = []
    while self.bm.num_free() < num_blocks:
        leaves = [n for n in self.nodes() if not n.children and n.locks == 0]
        if not leaves:
            break
        victim = max(leaves, key=lambda n: (n.stamp, n.serial))
        self.bm.free_seq(victim.holder)
        del victim.parent.children[victim.edge[0]]
        freed.append(victim.holder)
    return freed


@pytest.mark.parametrize("mutant,pin", [
    ("walk", test_matches_equal_brute_force_longest_common_prefix),
    ("blocks", test_token_granular_reuse_shares_the_partial_block),
    ("evict", test_eviction_is_lru_over_unlocked_leaves_and_spares_shared_nodes),
], ids=["whole-edges-only", "block-granular-match", "evicts-newest"])
def test_pins_catch_planted_mistakes(monkeypatch, mutant, pin):
    import oracle.radix as orx

    if mutant == "walk":
        monkeypatch.setattr(orx.RadixCacheModel, "_walk", _walk_whole_edges_only)
    elif mutant == "blocks":
        monkeypatch.setattr(orx.RadixCacheModel, "_walk", _walk_block_granular)
    else:
        monkeypatch.setattr(orx.RadixCacheModel, "evict", _evict_newest_first)
    with pytest.raises(AssertionError):
        pin()
