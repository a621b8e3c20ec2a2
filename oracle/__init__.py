"""Plain CPU oracle for paged decode attention (TEST INFRASTRUCTURE ONLY).

This package is the slow, obviously-correct reference that the GPU library is
checked against.  It is test infrastructure: only the test suite, the smoke
check in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (the HIP library and its Python binding) never
imports, calls or falls back to anything here, and nothing here imports the
product path.

Sources it follows (web pages, cited by title and section):

* [ZQ] zenaique.com, "How does PagedAttention enable prefix sharing across
  requests and what data structure makes it cheap?" -- the two answer
  paragraphs, the TL;DR and the "Most common mistake" note.
* [KG] kgptalkie.com, "Day 28: PagedAttention" -- sections "Split the Cache
  Into Fixed Blocks", "The Block Table Is the Map", "Follow One Token
  Address", "Growth Needs Only Another Free Block", "Batching Becomes More
  Flexible", "Prefix Sharing Is a Natural Extension", "Shared Blocks Must Not
  Be Changed in Place" and "A Tiny Block-Table Example" (whose closing
  paragraphs compare PagedAttention with FlashAttention and say how to test a
  paging implementation).

Modules:

* ``paged``  -- address translation, the in-block layout, history gather,
  attention, KV-write scatter and whole-block copy, in numpy fp64.
* ``blocks`` -- a host model of the block pool: free list, reference counts,
  growth by one block and copy-on-write.

Every function is pinned by tests under ``tests/test_oracle_*.py`` against
values the pages print, closed forms, library routines or brute force.
Parity of attention values at the large synthetic shapes has no printed
example to pin against (the pages print no attention numbers); those are
pinned only through the invariants and the library cross-check.
"""

from . import blocks, paged, prefix_cache  # noqa: F401
