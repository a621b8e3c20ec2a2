"""The native block manager (``include/pa_blocks.h``) against the oracle's
block model, on the CPU (the manager is host code; no GPU is touched).

Random sequences of admissions, forks, decode steps and frees run on both
``ops.BlockManager`` and ``oracle.blocks.BlockPool`` /
``oracle.prefix_cache.PrefixCachePool``.  Both hand out free blocks in the
same documented order, so after every operation the slots, copy-on-write
pairs, block tables, lengths, reference counts, free counts and cache sizes
must be identical.  Operations the oracle cannot complete (pool exhausted)
must fail in the manager with PA_ERR_NO_SPACE and change nothing.
"""

import copy

import numpy as np
import pytest

from oracle import blocks as oblocks
from oracle import prefix_cache as opc
from paged_kv_cache_252_amd import ops

NO_SPACE, NOT_FOUND, NULL, SHAPE = 9, 10, 1, 2


class Model:
    """The oracle driven through the same operations as the manager."""

    def __init__(self, num_blocks, bs, cache, salt=0):
        self.cache = cache
        self.bs = bs
        self.pool = (opc.PrefixCachePool(num_blocks, bs, salt=salt) if cache
                     else oblocks.BlockPool(num_blocks, bs))
        self.seqs = {}
        self.next_id = 0

    def add(self, tokens):
        if self.cache:
            seq, cached = self.pool.admit(tokens)
        else:
            need = -(-len(tokens) // self.bs)
            if need > self.pool.num_free:
                raise oblocks.PoolExhausted("prompt")
            seq, cached = self.pool.new_sequence(), 0
            for _ in tokens:
                self.pool.append(seq)
        sid = self.next_id
        self.next_id += 1
        self.seqs[sid] = seq
        return sid, cached

    def fork(self, sid):
        child = self.pool.fork(self.seqs[sid])
        cid = self.next_id
        self.next_id += 1
        self.seqs[cid] = child
        return cid

    def free(self, sid):
        self.pool.free(self.seqs.pop(sid))

    def append(self, ids, toks):
        slots, pairs = [], []
        for sid, t in zip(ids, toks):
            r = self.pool.append(self.seqs[sid], t) if self.cache else self.pool.append(self.seqs[sid])
            slots.append(r.slot)
            if r.cow is not None:
                pairs.append(list(r.cow))
        return slots, pairs


def _same_state(bm, model, num_blocks):
    live = sorted(model.seqs)
    if live:
        max_blocks = max(1, max(len(model.seqs[s].table) for s in live))
        tab, lens = bm.tables(live, max_blocks)
        for i, sid in enumerate(live):
            seq = model.seqs[sid]
            row = seq.table + [-1] * (max_blocks - len(seq.table))
            assert tab[i].tolist() == row, (sid, tab[i].tolist(), row)
            assert int(lens[i]) == seq.length
            assert bm.seq_info(sid) == (seq.length, len(seq.table))
    assert bm.num_free == model.pool.num_free
    assert [bm.refcount(b) for b in range(num_blocks)] == model.pool.refcount
    if model.cache:
        assert bm.num_cached == len(model.pool.by_hash)


def _expect_status(status, fn, *args):
    with pytest.raises(ops.PagedKVError) as e:
        fn(*args)
    assert e.value.status == status, e.value


@pytest.mark.parametrize("cache", [False, True])
@pytest.mark.parametrize("seed", range(6))
def test_random_sessions_match_the_model(cache, seed):
    rng = np.random.default_rng(1000 + seed)
    bs = int(rng.choice([1, 2, 4, 16]))
    num_blocks = int(rng.integers(8, 80))
    salt = int(rng.integers(0, 2**63))
    bm = ops.BlockManager(num_blocks, bs, prefix_cache=cache, salt=salt)
    model = Model(num_blocks, bs, cache, salt)
    # prompts drawn from a few shared beginnings, so the cache gets hits
    stems = [rng.integers(0, 50, size=int(rng.integers(0, 5 * bs + 3))).tolist() for _ in range(3)]
    for step in range(160):
        op = rng.choice(["add", "fork", "append", "free"], p=[0.25, 0.15, 0.45, 0.15])
        live = sorted(model.seqs)
        if op == "add":
            stem = stems[int(rng.integers(0, len(stems)))]
            cut = int(rng.integers(0, len(stem) + 1))
            toks = stem[:cut] + rng.integers(0, 50, size=int(rng.integers(0, 2 * bs + 2))).tolist()
            trial = copy.deepcopy(model)
            try:
                want = trial.add(toks)
            except oblocks.PoolExhausted:
                _expect_status(NO_SPACE, bm.add, 0, np.asarray(toks, dtype=np.int32))
                if not cache:
                    _expect_status(NO_SPACE, bm.add, len(toks))
            else:
                got = bm.add(len(toks), np.asarray(toks, dtype=np.int32) if cache else None)
                assert got == want
                model = trial
        elif op == "fork" and live:
            sid = int(rng.choice(live))
            assert bm.fork(sid) == model.fork(sid)
        elif op == "append" and live:
            k = int(rng.integers(1, min(len(live), 6) + 1))
            ids = rng.choice(live, size=k, replace=bool(rng.integers(0, 2))).tolist()
            toks = rng.integers(0, 50, size=k).tolist()
            trial = copy.deepcopy(model)
            try:
                want_slots, want_pairs = trial.append(ids, toks)
            except oblocks.PoolExhausted:
                _expect_status(NO_SPACE, bm.append, ids, toks if cache else None)
            else:
                slots, pairs = bm.append(ids, toks if cache else None)
                assert slots.tolist() == want_slots
                assert pairs.tolist() == want_pairs
                model = trial
        elif op == "free" and live:
            sid = int(rng.choice(live))
            bm.free(sid)
            model.free(sid)
        _same_state(bm, model, num_blocks)
        for sid in sorted(model.seqs)[:2]:
            seq = model.seqs[sid]
            if seq.length:
                want = [b * bs + p % bs for p, b in
                        ((p, seq.table[p // bs]) for p in range(seq.length))]
                assert bm.slots(sid, 0, seq.length).tolist() == want


def test_worked_example_slots():
    """[KG] "A Tiny Block-Table Example": block size 4, a nine-token request
    needs three blocks; with the free list arranged as 9, 2, 14 its positions
    land where the page says (position 6 -> block 2, slot 10)."""
    bm = ops.BlockManager(16, 4)
    # take every block, then free all but 9, 2, 14 in the order that makes the
    # LIFO list hand out 9 first, then 2, then 14
    hold = [bm.add(4)[0] for _ in range(16)]           # request i holds block i
    for b in range(16):
        if b not in (9, 2, 14):
            bm.free(hold[b])
    for b in (14, 2, 9):
        bm.free(hold[b])
    sid, _ = bm.add(9)
    tab, lens = bm.tables([sid], 3)
    assert tab[0].tolist() == [9, 2, 14] and lens[0] == 9
    assert bm.slots(sid, 6, 1).tolist() == [10]
    assert bm.slots(sid, 8, 1).tolist() == [56]
    # growth: positions 9..11 need no block, the 13th position needs a 4th
    free0 = bm.num_free
    bm.append([sid] * 3)
    assert bm.num_free == free0
    bm.append([sid])
    assert bm.num_free == free0 - 1


def test_fanout_copy_on_write():
    """[ZQ] answer: branches of one prompt share its blocks; the first write of
    each branch into the partly filled shared block copies that block once,
    and the full blocks stay shared.  The parent then keeps its block."""
    bm = ops.BlockManager(64, 16)
    parent, _ = bm.add(40)                            # blocks 0, 1, 2 (2 partly filled)
    kids = [bm.fork(parent) for _ in range(4)]
    assert bm.refcount(2) == 5
    slots, pairs = bm.append(kids)
    assert pairs.tolist() == [[2, 3], [2, 4], [2, 5], [2, 6]]
    assert slots.tolist() == [b * 16 + 40 % 16 for b in (3, 4, 5, 6)]
    assert bm.refcount(0) == 5 and bm.refcount(2) == 1
    s2, p2 = bm.append([parent])
    assert p2.size == 0 and s2.tolist() == [2 * 16 + 8]


def test_block_key_matches_oracle():
    rng = np.random.default_rng(5)
    for _ in range(50):
        parent = int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2))
        toks = rng.integers(-2**31, 2**31, size=int(rng.integers(0, 40))).tolist()
        assert ops.block_key(parent, toks) == opc.block_hash(parent, toks)


def test_prefix_cache_session():
    """[ZQ] TL;DR: the second request with the same system prompt finds it in
    the cache and skips its prefill; blocks are freed only at count zero."""
    bs = 16
    bm = ops.BlockManager(32, bs, prefix_cache=True, salt=7)
    system = np.arange(1000, 1000 + 3 * bs, dtype=np.int32)
    a, ca = bm.add(tokens=np.concatenate([system, [1, 2, 3]]))
    b, cb = bm.add(tokens=np.concatenate([system, [4, 5]]))
    assert (ca, cb) == (0, 3 * bs)
    ta, _ = bm.tables([a, b], 4)
    assert ta[0, :3].tolist() == ta[1, :3].tolist() and ta[0, 3] != ta[1, 3]
    assert [bm.refcount(int(x)) for x in ta[0, :3]] == [2, 2, 2]
    bm.free(a)
    bm.free(b)
    assert bm.num_free == 32 and bm.num_cached == 3
    c, cc = bm.add(tokens=system)
    assert cc == 3 * bs
    other = ops.BlockManager(32, bs, prefix_cache=True, salt=8)
    assert other.add(tokens=system)[1] == 0              # another salt, no reuse


def test_errors_leave_state_unchanged():
    bm = ops.BlockManager(4, 4)
    sid, _ = bm.add(12)
    _expect_status(NO_SPACE, bm.add, 8)
    _expect_status(NOT_FOUND, bm.fork, 99)
    _expect_status(NOT_FOUND, bm.free, 99)
    _expect_status(NOT_FOUND, bm.append, [sid, 99])
    _expect_status(SHAPE, bm.slots, sid, 10, 5)
    _expect_status(SHAPE, bm.tables, [sid], 2)
    assert bm.seq_info(sid) == (12, 3) and bm.num_free == 1
    bm.append([sid] * 4)                                 # fills block 3... then needs a 5th
    _expect_status(NO_SPACE, bm.append, [sid])
    assert bm.seq_info(sid) == (16, 4) and bm.num_free == 0
    cache = ops.BlockManager(4, 4, prefix_cache=True)
    _expect_status(NULL, cache.add, 3, None)
    s2, _ = cache.add(tokens=[1, 2, 3])
    _expect_status(NULL, cache.append, [s2], None)
    lib = ops.lib()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.pa_bm_create(0, 4, 0, 0, ctypes.byref(h)) == SHAPE
    assert lib.pa_bm_create(4, 0, 0, 0, ctypes.byref(h)) == SHAPE
    assert lib.pa_bm_create(4, 4, 2, 0, ctypes.byref(h)) == 5
    assert lib.pa_bm_num_free(None) == -1
