"""Oracle: host block manager model (pure Python, integers only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: a block manager hands out fixed-size physical blocks
from a free pool and takes them back (robocikowo "PagedAttention",
*Komponenty*: block manager); blocks are allocated one at a time as a
sequence grows, with nothing reserved up front, so L tokens occupy
ceil(L / block_size) blocks ("PagedAttention et RadixAttention : parlons de
KV Cache", *PagedAttention : la mémoire comme un système d'exploitation*,
third step); sequences with a common prefix point at the same physical
blocks, tracked by reference counts, and a write into a shared block first
copies it (same section, fourth step; robocikowo *Jak działa* and
*Komponenty*); a finished request's blocks are released one by one and can
be reused at once ("PagedAttention — Gestion mémoire pour LLM à long
contexte", *Pourquoi c'est important*; glossary *Définition*).

Readings where the pages are silent (the C++ manager follows the same ones
so the two can be compared bit for bit):

* Free pool = a stack.  The initial order is given (element 0 is handed out
  first); released blocks are pushed on top and reused first; a released
  sequence gives back its blocks in logical order 0..n-1.
* Appending a token at length L: if ``L % bs == 0`` pop a fresh block and
  append it to the table; otherwise, if the block holding slot L is shared
  (refcount > 1), pop a block n, record the copy pair (old -> n), drop one
  reference from the old block, give n refcount 1 and put n in the table.
  The slot is ``table[L // bs] * bs + L % bs``.  A batch is processed in
  call order, each sequence's tokens in order; the last sharer of a block
  (refcount 1) writes in place; a full shared block never copies.
* ``fork(parent, child, n)`` shares the parent's first ``ceil(n/bs)`` blocks
  (n may stop inside a block; the child's first write there copies it).
* Every call is atomic: on any error nothing changes.

Prefix caching by chained block digests ("PagedAttention et RadixAttention :
parlons de KV Cache", the closing part on vLLM's automatic prefix caching and
the paragraph on cache salting; "PagedAttention — Gestion mémoire pour LLM à
long contexte", *Implications*: pages with identical token content may be
shared between requests).  The pages fix that every completed block gets a
digest of (its parent's digest, its own tokens, extra data), that equal token
sequences therefore give equal chains and find the blocks already computed,
and that a tenant-specific salt folded into the digest keeps equal requests
of different tenants apart.  Readings where they are silent:

* digest = SHA-256 of ``parent (32 bytes; zeros for block 0) || salt
  (uint64, little-endian) || the block's token ids (int32, little-endian)``;
  the salt is the extra data of every block;
* a block is registered when it fills and every token id in it (and every
  earlier block's digest) is known; if the digest is already registered to
  another block the new block stays unregistered (a duplicate);
* a lookup walks the prompt's full blocks from the first and stops at the
  first digest that is not registered; matched blocks are shared as by fork;
* a registered block whose reference count drops to zero is kept, with its
  digest, on an eviction list (oldest first); a released sequence adds its
  registered blocks from its last block to its first, so a chain's deeper
  blocks are evicted before its head (least recently used leaves first,
  shared heads last: same page, RadixAttention's eviction);
* a new block comes from the free stack; only when that is empty is the
  oldest evictable block taken, and its digest forgotten; a lookup hit on
  an evictable block takes it off the list;
* a registered block is immutable (its digest stands for its tokens): a
  write into one, possible after a fork inside it, copies it first even if
  the writer is its only holder; a block released that way joins the
  eviction list after the whole call, so no copy in the call can read a
  block the same call hands out again;
* token ids are recorded only while they are given with every append; an
  append without ids ends the sequence's chain (its later blocks are never
  registered).

Swapping to host memory ("PagedAttention — Gestion mémoire pour LLM à long
contexte", *Mode d'échec* and the glossary's *Page eviction*: when GPU
memory runs out even with paging, cold pages are written to CPU RAM and
read back when needed).  Readings where the pages are silent:

* a host pool of fixed blocks in the pool's own format, with its own free
  stack (element 0 handed out first, released blocks on top);
* ``swap_out(sid)`` gives every block of the sequence, in logical order, a
  fresh host block and reports the (GPU block, host block) copies; the
  sequence then drops its GPU references exactly as ``free_seq`` would
  (shared blocks stay for their other holders, registered ones become
  evictable).  A swapped-out sequence cannot be appended to, forked or
  exported; ``free_seq`` releases its host blocks;
* ``swap_in(sid)`` gives every host block, in logical order, a fresh GPU
  block (free stack first, then the eviction list), reports the (host
  block, GPU block) copies and releases the host blocks; the new blocks are
  unregistered (the sequence's digests are kept for later blocks);
* both are atomic: with too few free blocks on the target side nothing
  changes.

Pins (``tests/test_oracle_block_manager.py``): after every operation the
reference counts equal a from-scratch recount over all tables, free and
used blocks partition the pool, every table has ``ceil(L/bs)`` entries;
copy-on-write leaves the source block untouched; closed-form block counts
for the shared-prefix workload; out-of-blocks leaves the state unchanged.
Prefix cache (``tests/test_oracle_prefix_cache.py``): equal prompts share
blocks, salts separate tenants, one changed token ends the match at its
block, equal blocks at another depth miss, eviction order, the 50-request
system-prompt saving in closed form, and a random run whose every lookup
equals a brute force over token tuples (no hashing); planted mistakes in
the digest or the eviction order fail these pins.
"""
from __future__ import annotations

import hashlib

__all__ = ["BlockManagerModel", "BMError", "OutOfBlocks", "UnknownSeq", "InvalidArg", "Capacity", "block_digest",
           "ZERO_DIGEST"]

ZERO_DIGEST = bytes(32)


def block_digest(parent, salt, tokens):
    """Chain digest of one full block: SHA-256(parent || salt || tokens)."""
    if len(parent) != 32:
        raise InvalidArg("parent digest must be 32 bytes")
    if not 0 <= salt < 2 ** 64:
        raise InvalidArg("salt must fit in 64 unsigned bits")
    msg = bytearray(parent)
    msg += int(salt).to_bytes(8, "little")
    for t in tokens:
        msg += int(t).to_bytes(4, "little", signed=True)
    return hashlib.sha256(bytes(msg)).digest()


class BMError(Exception):
    pass


class InvalidArg(BMError):
    pass


class OutOfBlocks(BMError):
    pass


class UnknownSeq(BMError):
    pass


class Capacity(BMError):
    pass


def _cdiv(a, b):
    return -(-a // b)


class BlockManagerModel:
    def __init__(self, num_blocks, block_size, initial_free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise InvalidArg("num_blocks and block_size must be positive")
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if sorted(order) != list(range(num_blocks)):
            raise InvalidArg("initial free order must be a permutation of the block ids")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free = list(reversed(order))  # top of the stack = end of the list
        self.refcount = [0] * num_blocks
        self.tables = {}
        self.lens = {}
        # prefix cache
        self.salt = {}
        self.tokens = {}  # known leading token ids of each sequence
        self.digests = {}  # chain digests of each sequence's leading full blocks
        self.cached = {}  # digest -> registered block
        self.block_digest = [None] * num_blocks
        self.lru = []  # evictable registered blocks, oldest first
        # host swap pool
        self.num_host_blocks = 0
        self.host_free = []  # stack, top = end
        self.host_tables = {}  # sid -> host blocks of a swapped-out sequence

    def add_host_pool(self, num_host_blocks):
        if self.num_host_blocks:
            raise InvalidArg("the host pool is already set")
        if num_host_blocks <= 0:
            raise InvalidArg("num_host_blocks must be positive")
        self.num_host_blocks = num_host_blocks
        self.host_free = list(reversed(range(num_host_blocks)))

    def _on_gpu(self, sid):
        if sid not in self.tables:
            raise UnknownSeq(f"unknown sequence {sid}")
        if sid in self.host_tables:
            raise InvalidArg(f"sequence {sid} is swapped out")

    def _release(self, table):
        for b in table:
            self.refcount[b] -= 1
            if self.refcount[b] == 0 and self.block_digest[b] is None:
                self.free.append(b)
        for b in reversed(table):
            if self.refcount[b] == 0 and self.block_digest[b] is not None:
                self.lru.append(b)

    def swap_out(self, sid):
        """Move a sequence to the host pool; returns (GPU block, host block) copies."""
        self._on_gpu(sid)
        table = self.tables[sid]
        if len(table) > len(self.host_free):
            raise OutOfBlocks("not enough free host blocks")
        pairs = []
        for b in table:
            h = self.host_free.pop()
            pairs.append((b, h))
        self.host_tables[sid] = [h for _, h in pairs]
        self._release(table)
        self.tables[sid] = []
        return pairs

    def swap_in(self, sid):
        """Bring a swapped-out sequence back; returns (host block, GPU block) copies."""
        if sid not in self.tables:
            raise UnknownSeq(f"unknown sequence {sid}")
        if sid not in self.host_tables:
            raise InvalidArg(f"sequence {sid} is not swapped out")
        hosts = self.host_tables[sid]
        if len(hosts) > self._available():
            raise OutOfBlocks("not enough free blocks")
        pairs = []
        table = []
        for h in hosts:
            b = self._take()
            self.refcount[b] = 1
            table.append(b)
            pairs.append((h, b))
        self.tables[sid] = table
        for h in hosts:
            self.host_free.append(h)
        del self.host_tables[sid]
        return pairs

    def num_free_host(self):
        return len(self.host_free)

    def _take(self):
        if self.free:
            return self.free.pop()
        b = self.lru.pop(0)
        del self.cached[self.block_digest[b]]
        self.block_digest[b] = None
        return b

    def _available(self):
        return len(self.free) + len(self.lru)

    # ------------------------------------------------------------ sequences
    def add_seq(self, sid):
        self.add_seq_cached(sid, [], 0)

    def _match(self, tokens, salt):
        bs = self.block_size
        blocks, digests = [], []
        d = ZERO_DIGEST
        for i in range(len(tokens) // bs):
            d = block_digest(d, salt, tokens[i * bs:(i + 1) * bs])
            b = self.cached.get(d)
            if b is None:
                break
            blocks.append(b)
            digests.append(d)
        return blocks, digests

    def match_prefix(self, tokens, salt=0):
        """Prompt tokens a cached admission would share (a multiple of bs)."""
        return len(self._match([int(t) for t in tokens], salt)[0]) * self.block_size

    def add_seq_cached(self, sid, tokens, salt=0):
        """Add a sequence for a prompt, sharing its registered leading blocks.

        Returns the number of prompt tokens already cached; the sequence
        starts at that length and the caller appends the rest."""
        if sid in self.tables:
            raise InvalidArg(f"sequence {sid} exists")
        if not 0 <= salt < 2 ** 64:
            raise InvalidArg("salt must fit in 64 unsigned bits")
        tokens = [int(t) for t in tokens]
        blocks, digests = self._match(tokens, salt)
        for b in blocks:
            if self.refcount[b] == 0:
                self.lru.remove(b)
            self.refcount[b] += 1
        n = len(blocks) * self.block_size
        self.tables[sid] = list(blocks)
        self.lens[sid] = n
        self.salt[sid] = salt
        self.tokens[sid] = tokens[:n]
        self.digests[sid] = digests
        return n

    def fork(self, parent, child, n):
        if parent not in self.tables:
            raise UnknownSeq(f"unknown parent {parent}")
        self._on_gpu(parent)
        if child in self.tables:
            raise InvalidArg(f"sequence {child} exists")
        if n < 0 or n > self.lens[parent]:
            raise InvalidArg("fork length outside the parent's context")
        shared = self.tables[parent][: _cdiv(n, self.block_size)]
        for b in shared:
            self.refcount[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = n
        self.salt[child] = self.salt[parent]
        self.tokens[child] = self.tokens[parent][:n]
        self.digests[child] = self.digests[parent][: n // self.block_size]

    def free_seq(self, sid):
        if sid not in self.tables:
            raise UnknownSeq(f"unknown sequence {sid}")
        if sid in self.host_tables:
            self.host_free.extend(self.host_tables.pop(sid))
        else:
            self._release(self.tables[sid])
        for m in (self.tables, self.lens, self.salt, self.tokens, self.digests):
            del m[sid]

    # --------------------------------------------------------------- append
    def _must_copy(self, b, dropped):
        return self.block_digest[b] is not None or self.refcount[b] - dropped.get(b, 0) > 1

    def blocks_needed(self, sids, ntoks):
        bs = self.block_size
        need = 0
        dropped = {}
        for sid, n in zip(sids, ntoks):
            if n == 0:
                continue
            L = self.lens[sid]
            if L % bs:
                last = self.tables[sid][L // bs]
                if self._must_copy(last, dropped):
                    need += 1
                    dropped[last] = dropped.get(last, 0) + 1
            need += _cdiv(L + n, bs) - _cdiv(L, bs)
        return need

    def cow_needed(self, sids, ntoks):
        bs = self.block_size
        n_cow = 0
        dropped = {}
        for sid, n in zip(sids, ntoks):
            L = self.lens[sid]
            if n == 0 or L % bs == 0:
                continue
            last = self.tables[sid][L // bs]
            if self._must_copy(last, dropped):
                n_cow += 1
                dropped[last] = dropped.get(last, 0) + 1
        return n_cow

    def append_slots(self, sids, ntoks=None, slot_capacity=None, cow_capacity=None, token_ids=None):
        """Reserve slots for new tokens; returns ``(slots, cow_pairs)``.

        ``slots`` lists the slot of every new token, sequence-major in call
        order; ``cow_pairs`` lists ``(src, dst)`` block copies that must run
        before the tokens are written.  ``token_ids`` (same order as
        ``slots``, or None) are the new tokens' ids, for the prefix cache.
        """
        sids = list(sids)
        ntoks = [1] * len(sids) if ntoks is None else [int(n) for n in ntoks]
        if len(ntoks) != len(sids):
            raise InvalidArg("one token count per sequence")
        if len(set(sids)) != len(sids):
            raise InvalidArg("duplicate sequence in one call")
        for sid, n in zip(sids, ntoks):
            if sid not in self.tables:
                raise UnknownSeq(f"unknown sequence {sid}")
            self._on_gpu(sid)
            if n < 0:
                raise InvalidArg("negative token count")
        total = sum(ntoks)
        if token_ids is not None:
            token_ids = [int(t) for t in token_ids]
            if len(token_ids) != total:
                raise InvalidArg("one token id per new token")
        if slot_capacity is not None and total > slot_capacity:
            raise Capacity("slot buffer too small")
        if cow_capacity is not None and self.cow_needed(sids, ntoks) > cow_capacity:
            raise Capacity("copy-pair buffer too small")
        if self.blocks_needed(sids, ntoks) > self._available():
            raise OutOfBlocks("not enough free blocks")
        bs = self.block_size
        slots, pairs, released = [], [], []
        for sid, n in zip(sids, ntoks):
            table = self.tables[sid]
            known = self.tokens[sid]
            for _ in range(n):
                L = self.lens[sid]
                if L % bs == 0:
                    b = self._take()
                    self.refcount[b] = 1
                    table.append(b)
                else:
                    old = table[L // bs]
                    if self._must_copy(old, {}):
                        b = self._take()
                        pairs.append((old, b))
                        self.refcount[old] -= 1
                        self.refcount[b] = 1
                        table[L // bs] = b
                        if self.refcount[old] == 0:  # registered, last holder gone
                            released.append(old)
                if token_ids is not None and len(known) == L:
                    known.append(token_ids[len(slots)])
                slots.append(table[L // bs] * bs + L % bs)
                self.lens[sid] = L + 1
                if (L + 1) % bs == 0:
                    self._complete(sid, L // bs)
        self.lru.extend(released)
        return slots, pairs

    def _complete(self, sid, i):
        """Block i of sid just filled: give it its digest and register it."""
        bs = self.block_size
        known, digests = self.tokens[sid], self.digests[sid]
        if len(known) < (i + 1) * bs or len(digests) != i:
            return
        parent = digests[i - 1] if i else ZERO_DIGEST
        d = block_digest(parent, self.salt[sid], known[i * bs:(i + 1) * bs])
        digests.append(d)
        if d not in self.cached:
            b = self.tables[sid][i]
            self.cached[d] = b
            self.block_digest[b] = d

    # ---------------------------------------------------------------- query
    def block_tables(self, sids, max_blocks):
        rows, lens = [], []
        for sid in sids:
            self._on_gpu(sid)
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise Capacity("table wider than max_blocks")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[sid])
        return rows, lens

    def num_free(self):
        """Blocks a new allocation can take: the free stack and the evictable list."""
        return self._available()

    def num_cached(self):
        return len(self.cached)

    def evictable(self):
        """Evictable registered blocks, oldest (next evicted) first."""
        return list(self.lru)

    def free_stack(self):
        """Free blocks, bottom to top (the next block handed out is last)."""
        return list(self.free)

    def check_invariants(self):
        """Raise AssertionError if the bookkeeping is inconsistent."""
        recount = [0] * self.num_blocks
        for sid, t in self.tables.items():
            if sid in self.host_tables:
                assert t == [] and len(self.host_tables[sid]) == _cdiv(self.lens[sid], self.block_size)
                continue
            assert len(t) == _cdiv(self.lens[sid], self.block_size), "table length != ceil(L/bs)"
            for b in t:
                recount[b] += 1
        assert recount == self.refcount, "refcount differs from recount"
        free = set(self.free)
        assert len(free) == len(self.free), "block twice in the free pool"
        used = {b for b in range(self.num_blocks) if recount[b] > 0}
        lru = set(self.lru)
        assert len(lru) == len(self.lru), "block twice on the eviction list"
        assert not (free & used) and not (lru & used) and not (free & lru), "block in two of free/evictable/used"
        assert len(free) + len(lru) + len(used) == self.num_blocks, "block neither free, evictable nor in use"
        host_used = [h for t in self.host_tables.values() for h in t]
        assert len(set(host_used)) == len(host_used), "host block held twice"
        assert not (set(host_used) & set(self.host_free)), "host block both free and held"
        assert len(host_used) + len(self.host_free) == self.num_host_blocks, "host block lost"
        # digest registry: a bijection between digests and registered blocks
        assert len(self.cached) == sum(d is not None for d in self.block_digest)
        for d, b in self.cached.items():
            assert self.block_digest[b] == d, "registry and block digests disagree"
        for b in free:
            assert self.block_digest[b] is None, "registered block on the free stack"
        for b in lru:
            assert self.block_digest[b] is not None, "unregistered block on the eviction list"
        # every sequence's chain recomputed from its token ids, and every
        # registered block it holds carries the digest of its position
        bs = self.block_size
        for sid, t in self.tables.items():
            if sid in self.host_tables:
                continue
            known, digests = self.tokens[sid], self.digests[sid]
            assert len(known) <= self.lens[sid] and len(digests) <= self.lens[sid] // bs
            d = ZERO_DIGEST
            for i, di in enumerate(digests):
                d = block_digest(d, self.salt[sid], known[i * bs:(i + 1) * bs])
                assert d == di, "sequence chain digest does not recompute"
                if self.block_digest[t[i]] is not None:
                    assert self.block_digest[t[i]] == di, "shared block registered under another chain"
