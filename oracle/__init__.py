"""CPU oracle for paged KV-cache decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import or call it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or constant generators); the
only thing both sides consume is the seeded input description in
``workloads.py``.

What it computes, and where each step comes from (page titles and sections
of the four pages on PagedAttention that define the method):

* ``pool``   -- the physical K/V block pools, the cache-append scatter and
  the copy-on-write block copy.  The KV cache is cut into fixed-size blocks
  of token slots (16 or 32) held in GPU memory; a sequence's tokens land in
  the block its table names ("PagedAttention" glossary, *Définition*;
  "PagedAttention — Gestion mémoire pour LLM à long contexte",
  *Points clés*; robocikowo "PagedAttention", *Jak działa*).
* ``block_manager`` -- the host bookkeeping: free pool, on-demand block
  allocation, per-block reference counts, sharing by fork, copy-on-write on
  a write into a shared block, individual release ("PagedAttention et
  RadixAttention : parlons de KV Cache", *PagedAttention : la mémoire comme
  un système d'exploitation*, steps 1-4; robocikowo *Komponenty*).
* ``attention`` -- decode attention: gather each sequence's blocks through
  its table into a contiguous K/V and evaluate softmax(q K^T * scale) V in
  fp64.  Paging leaves the attention result unchanged (aitalk page, end of
  the *PagedAttention* section), so the oracle is the plain definition.

Every function names the pins (tests in ``tests/test_oracle_*.py``) that tie
it to something other than itself; none is "parity unpinned".
"""

from . import attention, block_manager, pool  # noqa: F401
