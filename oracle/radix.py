"""Oracle: radix-tree prefix index over the block manager (pure Python).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("PagedAttention et RadixAttention : parlons de KV
Cache", section *RadixAttention : un arbre qui n'oublie pas* and the
paragraph after it): the cache becomes a persistent searchable radix tree,
a compressed trie in which each distinct token prefix is stored once and
requests with a common start walk the same branch, splitting exactly where
their tokens first differ; a new request walks the tree token by token for
the longest prefix already present, reuses its K/V, computes only the rest
and inserts its own path for later requests; when memory runs out, the
least recently used leaves are evicted first while internal nodes shared by
several requests are protected; and the tree only points at blocks that the
paged allocator manages.

Readings where the pages are silent:

* every node (but the root) is backed by a block-manager sequence, its
  *holder*, whose first ``depth`` tokens are the node's path; holders are
  made by ``fork`` from the request or from the node they split, so they
  only add reference counts (a split inside a block shares the partial
  block, which is copied only if someone writes into it);
* holder ids are ``HOLDER_BASE + k`` in creation order;
* ``admit(sid, tokens)``: match the longest prefix (token granular, it may
  end inside an edge); a match of ``m > 0`` tokens forks the deepest
  touched node's holder into ``sid`` at ``m`` (else ``sid`` starts empty);
  every node on the matched path is locked for ``sid`` and stamped with the
  current time; the caller appends ``tokens[m:]``;
* ``insert(sid, tokens)``: the request's first ``len(tokens)`` tokens (its
  K/V already in ``sid``) become a path: an edge that diverges part way is
  split at the divergence (the new inner node's holder is forked from the
  split node's holder), and the unmatched rest becomes a new leaf whose
  holder is forked from ``sid``; nodes on the path are stamped;
* ``release(sid)`` unlocks the nodes ``admit`` locked for ``sid``;
* ``evict(n)`` frees holders of unlocked leaves, least recently stamped
  first (ties: the node created first), until ``n`` blocks are free in the
  pool or no unlocked leaf is left; a parent left without children becomes
  a leaf itself;
* time is a counter advanced by every ``admit`` and ``insert``.

Pins (``tests/test_oracle_radix.py``): matches equal the longest common
prefix with the inserted token sequences (brute force), token-granular
reuse beyond the last full block, shared blocks and copy-on-write of the
partial block, eviction order and the protection of locked paths, and the
block-manager invariants after random runs.
"""
from __future__ import annotations

from .block_manager import InvalidArg, UnknownSeq

__all__ = ["RadixCacheModel", "HOLDER_BASE"]

HOLDER_BASE = 1 << 62


class _Node:
    __slots__ = ("edge", "parent", "children", "depth", "holder", "stamp", "locks", "serial")

    def __init__(self, edge, parent, depth, holder, stamp, serial):
        self.edge = list(edge)
        self.parent = parent
        self.children = {}  # first token -> node
        self.depth = depth
        self.holder = holder
        self.stamp = stamp
        self.locks = 0
        self.serial = serial


class RadixCacheModel:
    def __init__(self, bm):
        self.bm = bm
        self.root = _Node([], None, 0, None, 0, 0)
        self.clock = 0
        self.next_holder = 0
        self.serial = 1
        self.locked = {}  # sid -> nodes locked by admit

    # ----------------------------------------------------------- helpers
    def _new_holder(self):
        h = HOLDER_BASE + self.next_holder
        self.next_holder += 1
        return h

    def _node(self, edge, parent, depth, holder):
        n = _Node(edge, parent, depth, holder, self.clock, self.serial)
        self.serial += 1
        return n

    def _walk(self, tokens):
        """(path of fully or partly matched nodes, matched length, tokens of
        the last node's edge matched)."""
        node, i, path, used = self.root, 0, [], 0
        while i < len(tokens):
            child = node.children.get(tokens[i])
            if child is None:
                break
            k = 0
            while k < len(child.edge) and i + k < len(tokens) and child.edge[k] == tokens[i + k]:
                k += 1
            path.append(child)
            i += k
            used = k
            if k < len(child.edge):
                break
            node = child
        return path, i, used

    # -------------------------------------------------------------- API
    def match(self, tokens):
        return self._walk([int(t) for t in tokens])[1]

    def admit(self, sid, tokens):
        tokens = [int(t) for t in tokens]
        if sid in self.locked or sid in self.bm.tables:
            raise InvalidArg(f"sequence {sid} exists")
        path, m, _ = self._walk(tokens)
        self.clock += 1
        if m:
            self.bm.fork(path[-1].holder, sid, m)
        else:
            self.bm.add_seq(sid)
        for n in path:
            n.locks += 1
            n.stamp = self.clock
        self.locked[sid] = path
        return m

    def release(self, sid):
        if sid not in self.locked:
            raise UnknownSeq(f"sequence {sid} holds no locks")
        for n in self.locked.pop(sid):
            n.locks -= 1

    def insert(self, sid, tokens):
        """Make the first len(tokens) tokens of ``sid`` reusable; returns the
        number of tokens newly added to the tree."""
        tokens = [int(t) for t in tokens]
        if sid not in self.bm.tables:
            raise UnknownSeq(f"unknown sequence {sid}")
        if len(tokens) > self.bm.lens[sid]:
            raise InvalidArg("more tokens than the sequence holds")
        if sid in self.bm.host_tables:
            raise InvalidArg(f"sequence {sid} is swapped out")
        path, m, used = self._walk(tokens)
        self.clock += 1
        for n in path:
            n.stamp = self.clock
        parent = self.root
        if path:
            last = path[-1]
            if used < len(last.edge):  # split the edge at the divergence
                inner_depth = last.depth - len(last.edge) + used
                inner = self._node(last.edge[:used], last.parent, inner_depth, self._new_holder())
                self.bm.fork(last.holder, inner.holder, inner_depth)
                inner.stamp = self.clock
                inner.locks = last.locks
                last.parent.children[inner.edge[0]] = inner
                last.edge = last.edge[used:]
                last.parent = inner
                inner.children[last.edge[0]] = last
                for nodes in self.locked.values():  # a request locking `last` also depends on `inner`
                    if last in nodes:
                        nodes.insert(nodes.index(last), inner)
                parent = inner
            else:
                parent = last
        if m == len(tokens):
            return 0
        leaf = self._node(tokens[m:], parent, len(tokens), self._new_holder())
        self.bm.fork(sid, leaf.holder, len(tokens))
        parent.children[leaf.edge[0]] = leaf
        return len(tokens) - m

    def evict(self, num_blocks):
        """Free unlocked leaves, least recently used first, until
        ``num_blocks`` pool blocks are free; returns the holders freed."""
        freed = []
        while self.bm.num_free() < num_blocks:
            leaves = [n for n in self.nodes() if not n.children and n.locks == 0]
            if not leaves:
                break
            victim = min(leaves, key=lambda n: (n.stamp, n.serial))
            self.bm.free_seq(victim.holder)
            del victim.parent.children[victim.edge[0]]
            freed.append(victim.holder)
        return freed

    # ------------------------------------------------------------ queries
    def nodes(self):
        """All nodes but the root, depth-first in first-token order."""
        out, stack = [], [self.root]
        while stack:
            n = stack.pop()
            if n is not self.root:
                out.append(n)
            stack.extend(n.children[t] for t in sorted(n.children, reverse=True))
        return out

    def paths(self):
        """Token path of every node (root excluded), in ``nodes()`` order."""
        res = []
        for n in self.nodes():
            p, x = [], n
            while x is not self.root:
                p = x.edge + p
                x = x.parent
            res.append(p)
        return res

    def check_invariants(self):
        self.bm.check_invariants()
        for n, p in zip(self.nodes(), self.paths()):
            assert n.edge, "empty edge"
            assert len(p) == n.depth, "depth differs from the path length"
            assert self.bm.lens[n.holder] == n.depth, "holder length differs from the node depth"
            assert n.parent.children[n.edge[0]] is n, "child map broken"
            assert n.locks >= 0
        for nodes in self.locked.values():
            for a, b in zip(nodes, nodes[1:]):
                assert b.parent is a, "locked path is not a chain"
