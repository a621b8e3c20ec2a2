"""Plausible mistakes planted in the CPU oracle must trip at least one pin.

Each case monkeypatches one oracle function with a wrong variant (a dropped
term, a wrong index, a transposed operand, an off-by-one) and runs every pin
check; the test passes only if some check fails.  This shows the pins are
strong enough to catch the mistake.  Nothing here touches a GPU.
"""

import numpy as np
import pytest

from oracle import blocks as oblocks
from oracle import paged
from oracle import prefix_cache as opc
from tests import pins

_orig_attend = paged.attend
_orig_gather = paged.gather_kv
_orig_block_tokens = paged.block_tokens
_orig_write = paged.write_kv


def _translate_swapped(position, block_table, block_size):
    offset, logical = divmod(int(position), int(block_size))
    phys = int(block_table[min(logical, len(block_table) - 1)])
    return logical, offset, phys, phys * block_size + offset


def _translate_bad_slot(position, block_table, block_size):
    logical, offset = divmod(int(position), int(block_size))
    phys = int(block_table[logical])
    return logical, offset, phys, phys * block_size + logical


def _blocks_needed_floor(n, bs):
    return n // bs


def _attend_no_scale(q, keys, values, scale):
    return _orig_attend(q, keys, values, 1.0)


def _attend_modulo_heads(q, keys, values, scale):
    hq, d = q.shape
    L, hkv, _ = keys.shape
    out = np.zeros((hq, d))
    if L == 0:
        return out
    for h_q in range(hq):
        h = h_q % hkv                              # wrong grouping
        s = scale * (keys[:, h, :] @ q[h_q])
        w = np.exp(s - s.max())
        out[h_q] = (w @ values[:, h, :]) / w.sum()
    return out


def _attend_unnormalised(q, keys, values, scale):
    hq, d = q.shape
    L, hkv, _ = keys.shape
    g = hq // hkv
    out = np.zeros((hq, d))
    if L == 0:
        return out
    for h_q in range(hq):
        s = scale * (keys[:, h_q // g, :] @ q[h_q])
        out[h_q] = np.exp(s - s.max()) @ values[:, h_q // g, :]
    return out


def _attend_drop_last(q, keys, values, scale):
    return _orig_attend(q, keys[:-1], values[:-1], scale) if keys.shape[0] > 1 else \
        _orig_attend(q, keys, values, scale)


def _attend_values_as_keys(q, keys, values, scale):
    return _orig_attend(q, keys, keys, scale)


def _gather_physical_order(k_pool, v_pool, block_table, context_len, **kw):
    n = paged.blocks_needed(context_len, kw["block_size"])
    return _orig_gather(k_pool, v_pool, sorted(block_table[:n]), context_len, **kw)


def _gather_one_extra(k_pool, v_pool, block_table, context_len, **kw):
    bs = kw["block_size"]
    if context_len % bs and context_len:
        return _orig_gather(k_pool, v_pool, block_table, context_len + 1, **kw)
    return _orig_gather(k_pool, v_pool, block_table, context_len, **kw)


def _block_tokens_k_transposed(k_pool, v_pool, physical_block, num_kv_heads, block_size,
                               head_dim, dtype):
    x = 16 // paged.ELEM_BYTES[dtype]
    k5 = np.asarray(k_pool).reshape(-1, num_kv_heads, block_size, head_dim // x, x)
    k_rows = k5[physical_block].transpose(1, 0, 2, 3).reshape(block_size, num_kv_heads,
                                                                head_dim)
    _, v_rows = _orig_block_tokens(k_pool, v_pool, physical_block, num_kv_heads, block_size,
                                   head_dim, dtype)
    return k_rows, v_rows


def _block_tokens_v_rowmajor(k_pool, v_pool, physical_block, num_kv_heads, block_size,
                             head_dim, dtype):
    k_rows, _ = _orig_block_tokens(k_pool, v_pool, physical_block, num_kv_heads, block_size,
                                   head_dim, dtype)
    v_rows = np.asarray(v_pool).reshape(-1, num_kv_heads, block_size, head_dim)[physical_block]
    return k_rows, v_rows.transpose(1, 0, 2)


def _write_wrong_block(k_pool, v_pool, k_new, v_new, slots, num_kv_heads, block_size,
                       head_dim, dtype):
    bad = [(-1 if s < 0 else (s % block_size) * block_size + s // block_size) for s in slots]
    bad = [b if b < np.asarray(k_pool).shape[0] * block_size else -1 for b in bad]
    return _orig_write(k_pool, v_pool, k_new, v_new, bad, num_kv_heads, block_size, head_dim,
                       dtype)


def _copy_reversed(k_pool, v_pool, pairs):
    k = np.array(k_pool, copy=True)
    v = np.array(v_pool, copy=True)
    for src, dst in pairs:
        k[int(src)] = k[int(dst)]
        v[int(src)] = v[int(dst)]
    return k, v


def _append_in_place(self, seq):
    bs = self.block_size
    allocated = None
    if seq.length % bs == 0:
        allocated = self.allocate()
        seq.table.append(allocated)
    slot = paged.translate(seq.length, seq.table, bs)[3]
    seq.length += 1
    return oblocks.AppendResult(slot=slot, allocated=allocated, cow=None)


def _free_without_refcount(self, seq):
    for b in seq.table:
        self.refcount[b] = 0
        self._free.append(b)
    seq.table = []
    seq.length = 0


_orig_fnv = opc.fnv1a64
_orig_register = opc.PrefixCachePool._register
_orig_pc_append = opc.PrefixCachePool.append


def _fnv_plain(data):                      # FNV-1 order: multiply, then xor
    h = opc.FNV64_OFFSET
    for byte in data:
        h = (h * opc.FNV64_PRIME) & opc.MASK64
        h ^= byte
    return h


def _key_without_parent(parent, tokens):
    return _orig_fnv(b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens))


def _lookup_unverified(self, parent, tokens):
    h = opc.block_hash(parent, tokens)
    return h, self.by_hash.get(h)


def _release_evicts_early(self, block):
    if self.refcount[block] <= 0:
        raise oblocks.RefcountError("underflow")
    self.refcount[block] -= 1
    if block in self.key:
        self.evictable[block] = None          # even while still in use
    elif self.refcount[block] == 0:
        self._free.append(block)


def _allocate_newest_first(self):
    if self._free:
        b = self._free.pop()
    elif self.evictable:
        b, _ = self.evictable.popitem(last=True)
        del self.by_hash[self.key.pop(b)[0]]
    else:
        raise oblocks.PoolExhausted("no free block")
    self.refcount[b] = 1
    return b


def _pc_free_head_first(self, seq):
    for b in seq.table:
        self.release(b)
    seq.table, seq.length, seq.tokens = [], 0, []


def _pc_append_no_registration(self, seq, token):
    res = oblocks.BlockPool.append(self, seq)
    seq.tokens.append(int(token))
    return res


def _admit_registers_partial(self, tokens):
    seq, hits = _orig_admit(self, tokens)
    bs = self.block_size
    if len(tokens) % bs:
        _orig_register(self, seq.table[-1], seq.parent_hash, list(tokens[-(len(tokens) % bs):]))
    return seq, hits


def _bf16_as_half(bits):
    return np.asarray(bits).view(np.float16).astype(np.float64)


def _bf16_drops_sign(bits):
    bits = np.asarray(bits)
    return ((bits & np.uint16(0x7FFF)).astype(np.uint32) << np.uint32(16)).view(
        np.float32).astype(np.float64)


_orig_one_head = paged.decode_one_head


def _one_head_drops_newest(q_group, k_pool, v_pool, block_table, context_len, kv_head, scale,
                           num_kv_heads, block_size, head_dim, dtype):
    return _orig_one_head(q_group, k_pool, v_pool, block_table, max(int(context_len) - 1, 0),
                          kv_head, scale, num_kv_heads, block_size, head_dim, dtype)


_orig_admit = opc.PrefixCachePool.admit
_orig_prefill = paged.prefill


def _prefill_positions_from_start(q, q_start, k_pool, v_pool, block_tables, context_lens, scale,
                                  num_kv_heads, block_size, head_dim, dtype):
    out = np.zeros((np.asarray(q).shape[0], np.asarray(q).shape[1], head_dim))
    for i in range(len(q_start) - 1):
        n = int(q_start[i + 1]) - int(q_start[i])
        kc, vc = paged.gather_kv(k_pool, v_pool, block_tables[i], int(context_lens[i]),
                                 num_kv_heads, block_size, head_dim, dtype)
        for j in range(n):
            r = int(q_start[i]) + j
            out[r] = paged.attend(paged.to_f64(np.asarray(q)[r], dtype), paged.to_f64(kc, dtype)[:j + 1],
                                  paged.to_f64(vc, dtype)[:j + 1], scale)
    return out


def _prefill_excludes_self(q, q_start, k_pool, v_pool, block_tables, context_lens, scale,
                           num_kv_heads, block_size, head_dim, dtype):
    lens = [max(int(L) - 1, 0) for L in context_lens]
    return _orig_prefill(q, q_start, k_pool, v_pool, block_tables, lens, scale, num_kv_heads,
                         block_size, head_dim, dtype)


def _prefill_no_causal_mask(q, q_start, k_pool, v_pool, block_tables, context_lens, scale,
                            num_kv_heads, block_size, head_dim, dtype):
    out = np.zeros((np.asarray(q).shape[0], np.asarray(q).shape[1], head_dim))
    for i in range(len(q_start) - 1):
        L = int(context_lens[i])
        kc, vc = paged.gather_kv(k_pool, v_pool, block_tables[i], L, num_kv_heads, block_size,
                                 head_dim, dtype)
        for r in range(int(q_start[i]), int(q_start[i + 1])):
            out[r] = paged.attend(paged.to_f64(np.asarray(q)[r], dtype), paged.to_f64(kc, dtype),
                                  paged.to_f64(vc, dtype), scale)
    return out


MUTATIONS = {
    "translate_swapped_divmod": (paged, "translate", _translate_swapped),
    "translate_slot_uses_logical": (paged, "translate", _translate_bad_slot),
    "blocks_needed_floor": (paged, "blocks_needed", _blocks_needed_floor),
    "attend_drops_scale": (paged, "attend", _attend_no_scale),
    "attend_heads_modulo": (paged, "attend", _attend_modulo_heads),
    "attend_unnormalised": (paged, "attend", _attend_unnormalised),
    "attend_drops_newest_token": (paged, "attend", _attend_drop_last),
    "attend_mixes_keys": (paged, "attend", _attend_values_as_keys),
    "gather_physical_order": (paged, "gather_kv", _gather_physical_order),
    "gather_reads_past_length": (paged, "gather_kv", _gather_one_extra),
    "layout_k_chunks_transposed": (paged, "block_tokens", _block_tokens_k_transposed),
    "layout_v_row_major": (paged, "block_tokens", _block_tokens_v_rowmajor),
    "write_wrong_block": (paged, "write_kv", _write_wrong_block),
    "copy_reversed": (paged, "copy_blocks", _copy_reversed),
    "append_without_cow": (oblocks.BlockPool, "append", _append_in_place),
    "free_ignores_refcount": (oblocks.BlockPool, "free", _free_without_refcount),
    "fnv_multiply_before_xor": (opc, "fnv1a64", _fnv_plain),
    "key_ignores_parent": (opc, "block_hash", _key_without_parent),
    "lookup_trusts_hash": (opc.PrefixCachePool, "_lookup", _lookup_unverified),
    "cached_block_evictable_in_use": (opc.PrefixCachePool, "release", _release_evicts_early),
    "evict_newest_first": (opc.PrefixCachePool, "allocate", _allocate_newest_first),
    "free_head_first": (opc.PrefixCachePool, "free", _pc_free_head_first),
    "decode_blocks_not_registered": (opc.PrefixCachePool, "append", _pc_append_no_registration),
    "partial_block_registered": (opc.PrefixCachePool, "admit", _admit_registers_partial),
    "prefill_positions_from_start": (paged, "prefill", _prefill_positions_from_start),
    "prefill_excludes_own_token": (paged, "prefill", _prefill_excludes_self),
    "prefill_sees_future": (paged, "prefill", _prefill_no_causal_mask),
    "bf16_read_as_half": (paged, "bf16_bits_to_f64", _bf16_as_half),
    "bf16_drops_sign": (paged, "bf16_bits_to_f64", _bf16_drops_sign),
    "one_head_drops_newest_token": (paged, "decode_one_head", _one_head_drops_newest),
}


def _gather_kw_wrapper(fn):
    """gather_kv is called positionally inside the oracle; adapt the mutants."""
    def wrapped(k_pool, v_pool, block_table, context_len, num_kv_heads, block_size, head_dim,
                dtype):
        return fn(k_pool, v_pool, block_table, context_len, num_kv_heads=num_kv_heads,
                  block_size=block_size, head_dim=head_dim, dtype=dtype)
    return wrapped


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    owner, attr, fn = MUTATIONS[name]
    if attr == "gather_kv":
        fn = _gather_kw_wrapper(fn)
    monkeypatch.setattr(owner, attr, fn)
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check()
        except AssertionError:
            failed.append(check.__name__)
            break
    assert failed, f"mutation {name} passed every pin"
