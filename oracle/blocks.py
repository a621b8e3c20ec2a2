"""Host model of the physical block pool (TEST INFRASTRUCTURE ONLY).

A plain Python model of the bookkeeping the pages describe, used by the tests
to check that synthetic workloads follow the pages' sharing rules and to pin
the allocation counts:

* Fixed-size blocks drawn from a pool of free blocks; a sequence grows by
  one block when it reaches the end of its last one, and its history never
  moves ([KG] "Growth Needs Only Another Free Block").
* Requests that share a prefix point at the same physical blocks; nothing is
  duplicated ([ZQ] answer paragraphs, [KG] "Prefix Sharing Is a Natural
  Extension").
* A reference count per block; finishing a request decrements it and the
  block returns to the free pool only at zero ([ZQ] answer, [KG] "Shared
  Blocks Must Not Be Changed in Place").
* Copy-on-write: when a request appends into a block that others still
  reference, it gets a fresh block holding a copy of the shared one, the new
  token goes into the copy, and only that request's table entry is
  repointed; full shared blocks stay shared ([ZQ] answer and "Most common
  mistake", [KG] "Shared Blocks Must Not Be Changed in Place").

The model reports which (src, dst) block copies the device must perform and
the flat slot of each appended token; it moves no data itself.
"""

from __future__ import annotations

from dataclasses import dataclass, field

from .paged import translate


class PoolExhausted(RuntimeError):
    """No free block is left in the pool."""


class RefcountError(RuntimeError):
    """A reference count would go negative, or a freed block is still mapped."""


@dataclass
class Sequence:
    """One request: its block table (logical -> physical) and its length."""

    table: list = field(default_factory=list)
    length: int = 0


@dataclass
class AppendResult:
    slot: int
    allocated: int | None = None          # a block taken for growth
    cow: tuple | None = None              # (src, dst) block copy required first


class BlockPool:
    """Free list plus a reference count per physical block.

    ``free_order`` fixes the order in which free blocks are handed out (any
    free block is a correct choice; a fixed order makes runs repeatable).
    """

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self._free = list(reversed(order))   # pop() from the end gives order[0] first
        self.refcount = [0] * num_blocks

    # -- pool ----------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free)

    def allocate(self) -> int:
        if not self._free:
            raise PoolExhausted("no free block")
        b = self._free.pop()
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def release(self, block: int) -> None:
        if self.refcount[block] <= 0:
            raise RefcountError(f"block {block} released with refcount {self.refcount[block]}")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            self._free.append(block)

    # -- sequences -----------------------------------------------------------
    def new_sequence(self) -> Sequence:
        return Sequence()

    def append(self, seq: Sequence) -> AppendResult:
        """Reserve the slot for one more token of ``seq``.

        At a block boundary one more free block is taken.  Inside a block that
        other requests still reference, copy-on-write gives this request a
        private copy first.  Returns the token's flat slot and the block
        copy, if any, that must happen before the token is written.
        """
        bs = self.block_size
        allocated = None
        cow = None
        if seq.length % bs == 0:
            allocated = self.allocate()
            seq.table.append(allocated)
        else:
            last = seq.table[-1]
            if self.refcount[last] > 1:
                dst = self.allocate()
                self.refcount[last] -= 1          # this request stops using the shared block
                seq.table[-1] = dst
                cow = (last, dst)
        slot = translate(seq.length, seq.table, bs)[3]
        seq.length += 1
        return AppendResult(slot=slot, allocated=allocated, cow=cow)

    def fork(self, seq: Sequence) -> Sequence:
        """A new request that shares every block of ``seq`` by pointer."""
        for b in seq.table:
            self.refcount[b] += 1
        return Sequence(table=list(seq.table), length=seq.length)

    def free(self, seq: Sequence) -> None:
        """The request finishes: drop one reference to each of its blocks.

        The pages fix no order; blocks are released last to first, so the
        free list hands back a request's tail before its head."""
        for b in reversed(seq.table):
            self.release(b)
        seq.table = []
        seq.length = 0
