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

Pins (``tests/test_oracle_block_manager.py``): after every operation the
reference counts equal a from-scratch recount over all tables, free and
used blocks partition the pool, every table has ``ceil(L/bs)`` entries;
copy-on-write leaves the source block untouched; closed-form block counts
for the shared-prefix workload; out-of-blocks leaves the state unchanged.
"""
from __future__ import annotations

__all__ = ["BlockManagerModel", "BMError", "OutOfBlocks", "UnknownSeq", "InvalidArg", "Capacity"]


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

    # ------------------------------------------------------------ sequences
    def add_seq(self, sid):
        if sid in self.tables:
            raise InvalidArg(f"sequence {sid} exists")
        self.tables[sid] = []
        self.lens[sid] = 0

    def fork(self, parent, child, n):
        if parent not in self.tables:
            raise UnknownSeq(f"unknown parent {parent}")
        if child in self.tables:
            raise InvalidArg(f"sequence {child} exists")
        if n < 0 or n > self.lens[parent]:
            raise InvalidArg("fork length outside the parent's context")
        shared = self.tables[parent][: _cdiv(n, self.block_size)]
        for b in shared:
            self.refcount[b] += 1
        self.tables[child] = list(shared)
        self.lens[child] = n

    def free_seq(self, sid):
        if sid not in self.tables:
            raise UnknownSeq(f"unknown sequence {sid}")
        for b in self.tables[sid]:
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(b)
        del self.tables[sid]
        del self.lens[sid]

    # --------------------------------------------------------------- append
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
                if self.refcount[last] - dropped.get(last, 0) > 1:
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
            if self.refcount[last] - dropped.get(last, 0) > 1:
                n_cow += 1
                dropped[last] = dropped.get(last, 0) + 1
        return n_cow

    def append_slots(self, sids, ntoks=None, slot_capacity=None, cow_capacity=None):
        """Reserve slots for new tokens; returns ``(slots, cow_pairs)``.

        ``slots`` lists the slot of every new token, sequence-major in call
        order; ``cow_pairs`` lists ``(src, dst)`` block copies that must run
        before the tokens are written.
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
            if n < 0:
                raise InvalidArg("negative token count")
        total = sum(ntoks)
        if slot_capacity is not None and total > slot_capacity:
            raise Capacity("slot buffer too small")
        if cow_capacity is not None and self.cow_needed(sids, ntoks) > cow_capacity:
            raise Capacity("copy-pair buffer too small")
        if self.blocks_needed(sids, ntoks) > len(self.free):
            raise OutOfBlocks("not enough free blocks")
        bs = self.block_size
        slots, pairs = [], []
        for sid, n in zip(sids, ntoks):
            table = self.tables[sid]
            for _ in range(n):
                L = self.lens[sid]
                if L % bs == 0:
                    b = self.free.pop()
                    self.refcount[b] = 1
                    table.append(b)
                else:
                    old = table[L // bs]
                    if self.refcount[old] > 1:
                        b = self.free.pop()
                        pairs.append((old, b))
                        self.refcount[old] -= 1
                        self.refcount[b] = 1
                        table[L // bs] = b
                slots.append(table[L // bs] * bs + L % bs)
                self.lens[sid] = L + 1
        return slots, pairs

    # ---------------------------------------------------------------- query
    def block_tables(self, sids, max_blocks):
        rows, lens = [], []
        for sid in sids:
            if sid not in self.tables:
                raise UnknownSeq(f"unknown sequence {sid}")
            t = self.tables[sid]
            if len(t) > max_blocks:
                raise Capacity("table wider than max_blocks")
            rows.append(list(t) + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[sid])
        return rows, lens

    def num_free(self):
        return len(self.free)

    def free_stack(self):
        """Free blocks, bottom to top (the next block handed out is last)."""
        return list(self.free)

    def check_invariants(self):
        """Raise AssertionError if the bookkeeping is inconsistent."""
        recount = [0] * self.num_blocks
        for sid, t in self.tables.items():
            assert len(t) == _cdiv(self.lens[sid], self.block_size), "table length != ceil(L/bs)"
            for b in t:
                recount[b] += 1
        assert recount == self.refcount, "refcount differs from recount"
        free = set(self.free)
        assert len(free) == len(self.free), "block twice in the free pool"
        used = {b for b in range(self.num_blocks) if recount[b] > 0}
        assert not (free & used), "block both free and in use"
        assert len(free) + len(used) == self.num_blocks, "block neither free nor in use"
