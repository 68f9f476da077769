"""Pins for the oracle's prefix cache (chained block digests, CPU only).

What the pages fix ("PagedAttention et RadixAttention : parlons de KV
Cache", on vLLM's automatic prefix caching and on cache salting): equal token
sequences give equal digest chains and so find each other's blocks; each
digest depends on the previous one, so a chain stands for the whole prefix
before it; a tenant salt makes equal requests of different tenants miss.
These tests check those properties, the memory figure of a system prompt
shared by 50 requests ("PagedAttention — Gestion mémoire pour LLM à long
contexte", *Implications*), and, in a random run, every lookup against a
brute force that compares token tuples directly, with no hashing at all.
"""
import hashlib
import random

import pytest

from oracle.block_manager import ZERO_DIGEST, BlockManagerModel, InvalidArg, OutOfBlocks, block_digest

BS = 4


def _bm(n=64, order=None):
    return BlockManagerModel(n, BS, order)


def _prefill(bm, sid, tokens, salt=0):
    n = bm.add_seq_cached(sid, tokens, salt)
    bm.append_slots([sid], [len(tokens) - n], token_ids=tokens[n:])
    return n


def test_digest_encoding_and_primitive():
    # SHA-256 itself: the FIPS 180-2 one-block example
    assert hashlib.sha256(b"abc").hexdigest() == (
        "ba7816bf8f01cfea414140de5dae2223b00361a396177a9cb410ff61f20015ad")
    # the block message: parent || salt (8 bytes LE) || int32 LE tokens
    msg = bytes(32) + bytes([7, 0, 0, 0, 0, 0, 0, 0]) + bytes([1, 0, 0, 0, 0xFF, 0xFF, 0xFF, 0xFF])
    assert block_digest(ZERO_DIGEST, 7, [1, -1]) == hashlib.sha256(msg).digest()
    with pytest.raises(InvalidArg):
        block_digest(b"x", 0, [1])
    with pytest.raises(InvalidArg):
        block_digest(ZERO_DIGEST, 2 ** 64, [1])


def test_same_tokens_find_the_same_blocks():
    bm = _bm()
    prompt = list(range(100, 100 + 5 * BS + 3))
    assert _prefill(bm, 0, prompt) == 0
    assert bm.num_cached() == 5  # five full blocks registered; the partial one is not
    assert bm.match_prefix(prompt) == 5 * BS
    assert _prefill(bm, 1, prompt) == 5 * BS
    assert bm.tables[1][:5] == bm.tables[0][:5] and bm.tables[1][5] != bm.tables[0][5]
    assert all(bm.refcount[b] == 2 for b in bm.tables[0][:5])
    # a longer prompt with the same start shares the same five blocks
    assert bm.match_prefix(prompt + [9] * (2 * BS)) == 5 * BS
    bm.check_invariants()


def test_salt_separates_tenants():
    bm = _bm()
    prompt = list(range(3 * BS))
    _prefill(bm, 0, prompt, salt=11)
    assert bm.match_prefix(prompt, salt=11) == 3 * BS
    assert bm.match_prefix(prompt, salt=12) == 0
    assert bm.match_prefix(prompt, salt=0) == 0
    assert _prefill(bm, 1, prompt, salt=12) == 0  # tenant 12 computes its own copy
    assert set(bm.tables[0]).isdisjoint(bm.tables[1])
    assert bm.match_prefix(prompt, salt=12) == 3 * BS
    bm.check_invariants()


def test_chain_depends_on_every_earlier_block():
    bm = _bm()
    r = random.Random(1)
    prompt = [r.randrange(1000) for _ in range(6 * BS)]
    _prefill(bm, 0, prompt)
    for j in (0, BS - 1, BS, 3 * BS + 2, 6 * BS - 1):
        other = list(prompt)
        other[j] += 1  # one token changed: blocks after j's block are equal but must miss
        assert bm.match_prefix(other) == (j // BS) * BS, j
    # block content equal to the cached blocks 1.. but at another depth
    assert bm.match_prefix(prompt[BS:]) == 0


def test_only_full_blocks_with_known_ids_register():
    bm = _bm()
    bm.add_seq(0)
    bm.append_slots([0], [BS - 1], token_ids=[1] * (BS - 1))
    assert bm.num_cached() == 0
    bm.append_slots([0], [1], token_ids=[1])
    assert bm.num_cached() == 1
    bm.append_slots([0], [2])  # no ids: the chain ends here
    bm.append_slots([0], [3 * BS], token_ids=[1] * (3 * BS))
    assert bm.num_cached() == 1 and len(bm.digests[0]) == 1
    bm.check_invariants()


def test_duplicate_content_stays_unregistered():
    bm = _bm()
    prompt = list(range(2 * BS))
    bm.add_seq(0)
    bm.add_seq(1)
    bm.append_slots([0, 1], [2 * BS, 2 * BS], token_ids=prompt + prompt)  # both compute the same blocks
    assert bm.num_cached() == 2
    assert all(bm.block_digest[b] is not None for b in bm.tables[0])
    assert all(bm.block_digest[b] is None for b in bm.tables[1])
    dup = list(bm.tables[1])
    bm.free_seq(1)  # its duplicates go back to the free stack, not the eviction list
    assert bm.evictable() == [] and bm.free_stack()[-2:] == dup
    bm.check_invariants()


def test_eviction_is_tail_first_and_only_when_the_stack_is_empty():
    n = 8
    bm = _bm(n, list(range(n)))
    prompt = list(range(4 * BS))
    _prefill(bm, 0, prompt)
    blocks = list(bm.tables[0])
    assert blocks == [0, 1, 2, 3]
    bm.free_seq(0)
    assert bm.evictable() == [3, 2, 1, 0]  # deepest block is the oldest
    assert bm.num_free() == n and bm.num_cached() == 4
    # the four never-used blocks go first, without touching the cache
    bm.add_seq(1)
    bm.append_slots([1], [4 * BS])
    assert sorted(bm.tables[1]) == [4, 5, 6, 7] and bm.num_cached() == 4
    # now the stack is empty: the next allocation evicts block 3 (the tail)
    bm.append_slots([1], [1])
    assert bm.tables[1][-1] == 3 and bm.num_cached() == 3
    assert bm.match_prefix(prompt) == 3 * BS
    # a hit revives the evictable blocks
    assert bm.add_seq_cached(2, prompt) == 3 * BS
    assert bm.tables[2] == [0, 1, 2] and bm.evictable() == []
    with pytest.raises(OutOfBlocks):
        bm.append_slots([2], [1])
    bm.check_invariants()


def test_fork_inherits_the_chain():
    bm = _bm()
    prompt = list(range(2 * BS + 2))
    _prefill(bm, 0, prompt, salt=5)
    bm.fork(0, 1, 2 * BS + 1)
    tail = [70, 71, 72]
    bm.append_slots([1], [3], token_ids=tail)  # fills block 2 of the child (a copy)
    child = prompt[:2 * BS + 1] + tail
    assert bm.match_prefix(child, salt=5) == 3 * BS
    assert bm.match_prefix(child, salt=0) == 0
    bm.check_invariants()


def test_shared_system_prompt_closed_form():
    """50 requests with a common 2k-token system prompt (bs 16): one copy of
    its 128 blocks instead of 50, i.e. 49 x 128 blocks saved."""
    rng = random.Random(3)
    bs = 16
    system = [rng.randrange(32000) for _ in range(2048)]
    suffixes = [[rng.randrange(32000) for _ in range(rng.randint(1, 512))] for _ in range(50)]
    bm = BlockManagerModel(20000, bs)
    cached = []
    for i, suf in enumerate(suffixes):
        p = system + suf
        n = bm.add_seq_cached(i, p, salt=0)
        bm.append_slots([i], [len(p) - n], token_ids=p[n:])
        cached.append(n)
    assert cached[0] == 0 and all(c == 2048 for c in cached[1:])
    used = 20000 - bm.num_free()
    unshared = sum(-(-(2048 + len(s)) // bs) for s in suffixes)
    assert used == unshared - 49 * 128
    assert all(bm.refcount[b] == 50 for b in bm.tables[0][:128])
    bm.check_invariants()


def _brute_match(shadow, prompt, salt):
    """Longest cached prefix by token tuples: block i hits iff a registered
    block was filled as block i of a sequence with this salt and exactly
    these first (i+1)*bs tokens."""
    keys = set(shadow.values())
    k = 0
    while (k + 1) * BS <= len(prompt) and (salt, tuple(prompt[:(k + 1) * BS])) in keys:
        k += 1
    return k * BS


def test_random_run_against_token_tuple_brute_force():
    rng = random.Random(12)
    bm = _bm(48, rng.sample(range(48), 48))
    roots = [[rng.randrange(6) for _ in range(rng.randint(0, 5 * BS))] for _ in range(4)]
    shadow = {}  # registered block -> (salt, prefix tokens) seen when it registered
    seen_digest = {}  # ... and the digest it had then (a block can be evicted and registered again)
    live = []
    nxt = 0

    def refresh():
        for b in list(shadow):
            if bm.block_digest[b] != seen_digest[b]:
                del shadow[b]
        for sid, t in bm.tables.items():
            for i, b in enumerate(t):
                if bm.block_digest[b] is not None and b not in shadow and i < len(bm.digests[sid]) and \
                        bm.block_digest[b] == bm.digests[sid][i]:
                    shadow[b] = (bm.salt[sid], tuple(bm.tokens[sid][:(i + 1) * BS]))
                    seen_digest[b] = bm.block_digest[b]

    for it in range(600):
        op = rng.random()
        try:
            if op < 0.3 or not live:
                prompt = rng.choice(roots) + [rng.randrange(6) for _ in range(rng.randint(0, 2 * BS))]
                salt = rng.choice([0, 0, 9])
                expect = _brute_match(shadow, prompt, salt)
                assert bm.match_prefix(prompt, salt) == expect
                n = bm.add_seq_cached(nxt, prompt, salt)
                assert n == expect
                live.append(nxt)
                nxt += 1
                try:
                    bm.append_slots([live[-1]], [len(prompt) - n], token_ids=prompt[n:])
                except OutOfBlocks:
                    pass
            elif op < 0.6:
                sids = rng.sample(live, rng.randint(1, len(live)))
                nt = [rng.randint(0, 3) for _ in sids]
                ids = None if rng.random() < 0.1 else [rng.randrange(6) for _ in range(sum(nt))]
                bm.append_slots(sids, nt, token_ids=ids)
            elif op < 0.75:
                p = rng.choice(live)
                bm.fork(p, nxt, rng.randint(0, bm.lens[p]))
                live.append(nxt)
                nxt += 1
            else:
                sid = live.pop(rng.randrange(len(live)))
                bm.free_seq(sid)
        except OutOfBlocks:
            pass
        refresh()
        bm.check_invariants()
        # a shadow entry's key is unique: two registered blocks never hold the same prefix
        assert len(set(shadow.values())) == len(shadow)
    assert bm.num_cached() > 0 and len(bm.evictable()) >= 0


def test_registered_block_is_copied_even_for_its_last_holder():
    """A fork inside a registered block, then the parent released: the
    child's write must not change the cached block, so it copies it; the
    released block becomes evictable only after the call."""
    bm = _bm(6, list(range(6)))
    prompt = list(range(2 * BS))
    _prefill(bm, 0, prompt)  # blocks 0, 1 registered
    bm.fork(0, 1, 2 * BS - 1)  # child stops inside block 1
    bm.free_seq(0)
    assert bm.refcount[1] == 1 and bm.evictable() == []  # block 0, 1 still held by the child
    slots, pairs = bm.append_slots([1], [1], token_ids=[99])
    assert pairs == [(1, 2)] and slots == [2 * BS + BS - 1]
    assert bm.evictable() == [1] and bm.refcount[1] == 0
    assert bm.match_prefix(prompt) == 2 * BS  # the cached chain is intact
    assert bm.match_prefix(prompt[:-1] + [99]) == 2 * BS  # the child's copy registered its own chain
    assert bm.block_digest[2] is not None and bm.block_digest[2] != bm.block_digest[1]
    bm.check_invariants()
    # the block released by the copy is not handed out again in the same call
    bm2 = _bm(4, list(range(4)))
    _prefill(bm2, 0, prompt)  # blocks 0, 1
    bm2.fork(0, 1, 2 * BS - 1)
    bm2.free_seq(0)
    bm2.add_seq(2)
    bm2.append_slots([2], [BS])  # block 2; the stack now holds only block 3
    with pytest.raises(OutOfBlocks):
        bm2.append_slots([1, 2], [1, 1])  # needs a copy target and a new block: 1 is not reusable yet
    s, p = bm2.append_slots([1], [1], token_ids=[5])
    assert p == [(1, 3)] and bm2.evictable() == [1]
    bm2.check_invariants()


# ---------------------------------------------------------------- mutants
# Each plants one plausible mistake in the oracle and checks that a pin above
# fails under it.

def _digest_without_parent(parent, salt, tokens):
    return block_digest(ZERO_DIGEST, salt, tokens)


def _digest_without_salt(parent, salt, tokens):
    return block_digest(parent, 0, tokens)


def _free_head_first(self, sid):
    table = self.tables[sid]
    for b in table:
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            (self.free if self.block_digest[b] is None else self.lru).append(b)
    for m in (self.tables, self.lens, self.salt, self.tokens, self.digests):
        del m[sid]


def _copy_only_shared(self, b, dropped):
    return self.refcount[b] - dropped.get(b, 0) > 1


@pytest.mark.parametrize("mutant,pin", [
    ("digest", test_chain_depends_on_every_earlier_block),
    ("salt", test_salt_separates_tenants),
    ("evict", test_eviction_is_tail_first_and_only_when_the_stack_is_empty),
    ("inplace", test_registered_block_is_copied_even_for_its_last_holder),
], ids=["digest-ignores-parent", "digest-ignores-salt", "evicts-head-first", "writes-registered-block"])
def test_pins_catch_planted_mistakes(monkeypatch, mutant, pin):
    import oracle.block_manager as obm

    if mutant == "digest":
        monkeypatch.setattr(obm, "block_digest", _digest_without_parent)
    elif mutant == "salt":
        monkeypatch.setattr(obm, "block_digest", _digest_without_salt)
    elif mutant == "evict":
        monkeypatch.setattr(obm.BlockManagerModel, "free_seq", _free_head_first)
    else:
        monkeypatch.setattr(obm.BlockManagerModel, "_must_copy", _copy_only_shared)
    with pytest.raises(AssertionError):
        pin()

