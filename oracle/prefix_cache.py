"""Content-addressed prefix cache over the block pool (TEST INFRASTRUCTURE ONLY).

A plain Python model, used by the tests as the reference for the native block
manager's prefix cache.  What it follows:

* Blocks are content addressed: each full block gets a hash over its token
  ids chained with the hash of the block before it, and a table maps block
  hash -> physical block ([ZQ] answer and TL;DR).
* On admission the prompt is hashed block by block and each hash is looked
  up; every hit is shared by pointer (its reference count goes up) and the
  prefill for that span is skipped ([ZQ] TL;DR; [KG] "Prefix Sharing Is a
  Natural Extension").  The walk stops at the first miss: a later block can
  only be reused through the same chain of parents.
* Reuse needs the same computation, not merely similar text: the token ids
  and a caller-chosen ``salt`` standing for model state, position rules and
  cache settings enter the key ([KG] "Shared Blocks Must Not Be Changed in
  Place", last paragraphs).
* Reference counts still decide when a block is unused ([ZQ] answer); a
  cached block whose count reaches zero is kept for reuse, and only such
  blocks are ever evicted, oldest first.

Readings where the pages are silent:

* The hash is 64-bit FNV-1a (Fowler, Noll and Vo's published definition)
  over the parent hash (8 bytes, little-endian; the salt for the first
  block) followed by the block's token ids (4 bytes each, little-endian).
  A hit also compares the stored parent hash and token ids, so a hash
  collision can never share the wrong block.
* Only full blocks are cached.  Prompt blocks are registered when they are
  allocated (the caller writes their keys and values before any later call
  reads them); a block filled by decoding is registered when its last slot
  is taken.  If the hash is already registered the new block stays private.
* A finished request releases its blocks last to first, so among blocks that
  became unused together the tail of a chain is evicted before its parents.
* Allocation takes a never-cached free block first and evicts only when none
  is left.
"""

from __future__ import annotations

from collections import OrderedDict
from dataclasses import dataclass, field

from .blocks import AppendResult, BlockPool, PoolExhausted, RefcountError, Sequence
from .paged import translate

FNV64_OFFSET = 0xCBF29CE484222325
FNV64_PRIME = 0x100000001B3
MASK64 = (1 << 64) - 1


def fnv1a64(data: bytes) -> int:
    """64-bit FNV-1a: for each byte, xor it in, then multiply by the prime."""
    h = FNV64_OFFSET
    for byte in data:
        h ^= byte
        h = (h * FNV64_PRIME) & MASK64
    return h


def block_hash(parent: int, tokens) -> int:
    """Hash of one full block: its token ids chained with the parent's hash."""
    data = int(parent).to_bytes(8, "little") + b"".join(
        int(t).to_bytes(4, "little", signed=True) for t in tokens)
    return fnv1a64(data)


@dataclass
class CachedSequence(Sequence):
    tokens: list = field(default_factory=list)
    parent_hash: int = 0        # hash of the last full block (the salt before the first)


class PrefixCachePool(BlockPool):
    """``BlockPool`` plus the hash table of full blocks and an LRU of unused cached blocks."""

    def __init__(self, num_blocks: int, block_size: int, salt: int = 0, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.salt = int(salt) & MASK64
        self.by_hash: dict = {}            # block hash -> physical block
        self.key: dict = {}                # physical block -> (hash, parent hash, token ids)
        self.evictable: OrderedDict = OrderedDict()   # unused cached blocks, oldest first

    # -- pool ----------------------------------------------------------------
    @property
    def num_free(self) -> int:
        return len(self._free) + len(self.evictable)

    def allocate(self) -> int:
        if self._free:
            b = self._free.pop()
        elif self.evictable:
            b, _ = self.evictable.popitem(last=False)
            h = self.key.pop(b)[0]
            del self.by_hash[h]
        else:
            raise PoolExhausted("no free block")
        assert self.refcount[b] == 0
        self.refcount[b] = 1
        return b

    def release(self, block: int) -> None:
        if self.refcount[block] <= 0:
            raise RefcountError(f"block {block} released with refcount {self.refcount[block]}")
        self.refcount[block] -= 1
        if self.refcount[block] == 0:
            if block in self.key:
                self.evictable[block] = None
            else:
                self._free.append(block)

    def _register(self, block: int, parent: int, tokens) -> int:
        h = block_hash(parent, tokens)
        if h not in self.by_hash:
            self.by_hash[h] = block
            self.key[block] = (h, parent, tuple(int(t) for t in tokens))
        return h

    def _lookup(self, parent: int, tokens):
        h = block_hash(parent, tokens)
        b = self.by_hash.get(h)
        if b is not None and self.key[b][1:] == (parent, tuple(int(t) for t in tokens)):
            return h, b
        return h, None

    # -- sequences -----------------------------------------------------------
    def admit(self, tokens) -> tuple:
        """A new request with prompt ``tokens``: returns (sequence, cached tokens).

        Leading full blocks found in the cache are shared; the rest of the
        prompt gets fresh blocks, and its full blocks are registered.
        """
        bs = self.block_size
        tokens = [int(t) for t in tokens]
        n_full = len(tokens) // bs
        seq = CachedSequence(parent_hash=self.salt)
        found = []                            # (hash, block) of the leading hits
        parent = self.salt
        for i in range(n_full):
            h, b = self._lookup(parent, tokens[i * bs:(i + 1) * bs])
            if b is None:
                break
            found.append((h, b))
            parent = h
        hits = len(found)
        revived = sum(1 for _, b in found if self.refcount[b] == 0)
        need = -(-len(tokens) // bs) - hits
        if need > self.num_free - revived:    # checked first: nothing changes on failure
            raise PoolExhausted(f"prompt needs {need} blocks, {self.num_free - revived} free")
        for h, b in found:
            if self.refcount[b] == 0:
                del self.evictable[b]
            self.refcount[b] += 1
            seq.table.append(b)
            seq.parent_hash = h
        for i in range(hits, n_full):
            b = self.allocate()
            seq.table.append(b)
            seq.parent_hash = self._register(b, seq.parent_hash, tokens[i * bs:(i + 1) * bs])
        if len(tokens) % bs:
            seq.table.append(self.allocate())
        seq.tokens = tokens
        seq.length = len(tokens)
        return seq, hits * bs

    def append(self, seq: CachedSequence, token: int) -> AppendResult:
        """One more token: growth or copy-on-write as in ``BlockPool``, then
        registration of the block if this token filled it."""
        res = super().append(seq)
        seq.tokens.append(int(token))
        bs = self.block_size
        if seq.length % bs == 0:
            seq.parent_hash = self._register(seq.table[-1], seq.parent_hash, seq.tokens[-bs:])
        return res

    def fork(self, seq: CachedSequence) -> CachedSequence:
        child = super().fork(seq)
        return CachedSequence(table=child.table, length=child.length, tokens=list(seq.tokens),
                              parent_hash=seq.parent_hash)

    def free(self, seq: CachedSequence) -> None:
        for b in reversed(seq.table):
            self.release(b)
        seq.table = []
        seq.length = 0
        seq.tokens = []

    def slots(self, seq: Sequence, start: int, count: int) -> list:
        return [translate(p, seq.table, self.block_size)[3] for p in range(start, start + count)]
