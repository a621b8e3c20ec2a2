"""Oracle for the paged-KV hot path, in numpy fp64 (TEST INFRASTRUCTURE ONLY).

What is computed, and where it comes from:

* Address translation.  [KG] "Follow One Token Address": a token position is
  divided by the block size; the quotient is the logical block, the remainder
  the offset inside it, and the block table maps the logical block to the
  physical block.  The worked example (block size 4, table [9, 2, 14],
  position 6 -> logical 1, offset 2, physical 2) pins it.
* History gather.  [KG] "The Block Table Is the Map" and "Batching Becomes
  More Flexible": the kernel reads the request's block table and gathers the
  history in logical token order, whatever the physical numbering.
* Attention.  [KG] "Follow One Token Address" (closing sentence: the table
  only locates the cached keys and values; once found they are used by the
  usual decode attention of the newest token, with its visibility rule) and
  "The Contiguous Allocation Problem" (paging is about placement, not a
  change of the attention formula).  Read as scaled dot-product softmax
  attention of one decode query over the first ``L`` cached positions, with
  grouped query heads mapped to KV head ``hq // (Hq / Hkv)``.
* KV-write scatter.  The new token's K/V land at ``slot = physical *
  block_size + offset`` ([KG] "Follow One Token Address"); the library
  receives that flat slot per token.
* Block copy.  [ZQ] answer paragraphs and [KG] "Shared Blocks Must Not Be
  Changed in Place": a diverging writer gets a private copy of the shared
  block; only that block is copied ([ZQ] "Most common mistake").

The in-block layout is the library's documented contract (the pages leave it
to the implementation, [KG] "Split the Cache Into Fixed Blocks").  Each pool
(K or V) reaches the oracle as a dense ``[num_blocks][Hkv * block_size * D]``
array (how the library spaces blocks in device memory, its block stride, is
no concern here).  Positions of a block sit in tiles of ``T`` positions
(``T = 16`` when the block size is a multiple of 16, else the whole block).
With ``x = 16 / element_bytes`` (8 for bf16, 4 for fp32), tile ``u = t // T``
and place ``p = t % T``, the element for (block b, kv head h, position t,
dim d) is, inside the pool array,

    K: ((((b * Hkv + h) * (block_size / T) + u) * (D / x) + d / x) * T + p) * x + d % x
    V: (((b * Hkv + h) * (block_size / T) + u) * D + d) * T + p

The oracle reads it through numpy reshapes/transposes, not through those
scalar formulas (tests pin the two against each other).

Floating point: bf16 inputs arrive as their raw ``uint16`` bit patterns and
are widened exactly to fp64; fp32 inputs are widened to fp64.  All attention
arithmetic is fp64.
"""

from __future__ import annotations

import numpy as np

ELEM_BYTES = {"f32": 4, "bf16": 2}


# ----------------------------------------------------------------------------
# value decoding
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to fp64 exactly.

    A bf16 value is the upper half of an IEEE binary32 value, so shifting the
    16 bits into the top of a 32-bit word gives the same number as fp32.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bf16 data must be given as uint16 bit patterns")
    wide = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):     # signalling-NaN patterns widen to NaN quietly
        return wide.astype(np.float64)


def to_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    """Decode cache/query storage of ``dtype`` ('bf16' bits or 'f32') to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(values)
    if dtype == "f32":
        v = np.asarray(values)
        if v.dtype != np.float32:
            raise TypeError("f32 data must be float32")
        return v.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# block arithmetic ([KG] "Follow One Token Address", "Growth Needs Only
# Another Free Block")
# ----------------------------------------------------------------------------

def translate(position: int, block_table, block_size: int):
    """Map a logical token position to (logical block, offset, physical block, slot).

    [KG] "Follow One Token Address": divide the position by the block size;
    the quotient is the logical block and the remainder the offset inside it;
    the table entry for the logical block names the physical block.  The flat
    slot index of the token is ``physical * block_size + offset``.
    """
    pos, size = int(position), int(block_size)
    if size <= 0:
        raise ValueError("block_size must be positive")
    if pos < 0:
        raise ValueError("position must be non-negative")
    quotient = pos // size                  # which entry of the table
    remainder = pos - quotient * size       # where inside that block
    entry = int(block_table[quotient])
    return quotient, remainder, entry, entry * size + remainder


def slot_mapping(block_tables, seq_ids, positions, block_size: int) -> np.ndarray:
    """Flat slot of each token: ``translate`` of (seq_ids[t], positions[t]).

    A negative position marks a padding token and maps to slot -1.
    """
    out = np.empty(len(positions), dtype=np.int64)
    for t, (s, p) in enumerate(zip(seq_ids, positions)):
        if p < 0:
            out[t] = -1
        else:
            out[t] = translate(int(p), block_tables[int(s)], block_size)[3]
    return out


def blocks_needed(num_tokens: int, block_size: int) -> int:
    """Blocks that hold ``num_tokens`` positions: the count rounded up.

    [KG] "Growth Needs Only Another Free Block": nine tokens at four per
    block use three blocks; the thirteenth token needs a fourth.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("need num_tokens >= 0 and block_size > 0")
    return -(-num_tokens // block_size)


def tail_waste(num_tokens: int, block_size: int) -> int:
    """Unused slots in the last block of one unshared sequence.

    [KG] "Growth Needs Only Another Free Block": the slots allocated minus the
    tokens stored; never more than ``block_size - 1``.
    """
    return blocks_needed(num_tokens, block_size) * block_size - num_tokens


# ----------------------------------------------------------------------------
# the in-block layout (library contract) seen through numpy views
# ----------------------------------------------------------------------------

def tile_tokens(block_size: int) -> int:
    """Positions per tile inside a block: 16 when the block is a multiple of
    16 positions, else the whole block."""
    return 16 if block_size % 16 == 0 else block_size


def _k_view(k_pool: np.ndarray, num_kv_heads: int, block_size: int, head_dim: int, dtype: str):
    # [block][head][tile][D/x][position in tile][x]
    x = 16 // ELEM_BYTES[dtype]
    t = tile_tokens(block_size)
    return np.asarray(k_pool).reshape(-1, num_kv_heads, block_size // t, head_dim // x, t, x)


def _v_view(v_pool: np.ndarray, num_kv_heads: int, block_size: int, head_dim: int):
    # [block][head][tile][D][position in tile]
    t = tile_tokens(block_size)
    return np.asarray(v_pool).reshape(-1, num_kv_heads, block_size // t, head_dim, t)


def block_tokens(k_pool, v_pool, physical_block: int, num_kv_heads: int, block_size: int,
                 head_dim: int, dtype: str):
    """All ``block_size`` token rows of one physical block, as raw storage.

    Returns ``(K, V)``, each ``[block_size][num_kv_heads][head_dim]`` in the
    storage dtype (bit patterns untouched).  Position p of the block is
    position p % T of tile p // T (T = ``tile_tokens``).
    """
    k6 = _k_view(k_pool, num_kv_heads, block_size, head_dim, dtype)[physical_block]
    # [Hkv][tiles][D/x][T][x] -> [tiles][T][Hkv][D/x][x] -> [bs][Hkv][D]
    k_rows = k6.transpose(1, 3, 0, 2, 4).reshape(block_size, num_kv_heads, head_dim)
    v5 = _v_view(v_pool, num_kv_heads, block_size, head_dim)[physical_block]
    # [Hkv][tiles][D][T] -> [tiles][T][Hkv][D] -> [bs][Hkv][D]
    v_rows = v5.transpose(1, 3, 0, 2).reshape(block_size, num_kv_heads, head_dim)
    return k_rows, v_rows


def gather_kv(k_pool, v_pool, block_table, context_len: int, num_kv_heads: int,
              block_size: int, head_dim: int, dtype: str):
    """Contiguous history of one request, gathered through its block table.

    [KG] "The Block Table Is the Map" / "Batching Becomes More Flexible": walk
    the logical blocks in order, look each up in the table, and copy its
    tokens; the last block is truncated to the context length.  Returns raw
    storage ``(K, V)``, each ``[context_len][num_kv_heads][head_dim]``.
    """
    x_dtype = np.uint16 if dtype == "bf16" else np.float32
    kc = np.empty((context_len, num_kv_heads, head_dim), dtype=x_dtype)
    vc = np.empty((context_len, num_kv_heads, head_dim), dtype=x_dtype)
    for logical in range(blocks_needed(context_len, block_size)):
        physical = int(block_table[logical])
        lo = logical * block_size
        n = min(block_size, context_len - lo)
        k_rows, v_rows = block_tokens(k_pool, v_pool, physical, num_kv_heads, block_size,
                                      head_dim, dtype)
        kc[lo:lo + n] = k_rows[:n]
        vc[lo:lo + n] = v_rows[:n]
    return kc, vc


# ----------------------------------------------------------------------------
# attention
# ----------------------------------------------------------------------------

def attend(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """One decode query per head against a contiguous history, in fp64.

    ``q`` is ``[Hq][D]``, ``keys``/``values`` are ``[L][Hkv][D]`` (fp64).
    Query head ``hq`` reads KV head ``hq // (Hq / Hkv)``.  For each query head
    the scores are ``scale * <q, k_t>`` over the visible positions
    ``t = 0 .. L-1``; the output is the softmax-weighted mean of the values.
    The maximum score is subtracted before exponentiating (this leaves the
    result unchanged and keeps the exponentials finite).  An empty history
    (L = 0) gives a zero output.
    """
    num_q_heads, head_dim = q.shape
    context_len, num_kv_heads, _ = keys.shape
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_q_heads, head_dim), dtype=np.float64)
    if context_len == 0:
        return out
    for hq in range(num_q_heads):
        h = hq // group
        scores = scale * (keys[:, h, :] @ q[hq])
        weights = np.exp(scores - scores.max())
        out[hq] = (weights @ values[:, h, :]) / weights.sum()
    return out


def decode(q, k_pool, v_pool, block_tables, context_lens, scale: float, num_kv_heads: int,
           block_size: int, head_dim: int, dtype: str) -> np.ndarray:
    """Paged decode attention for a batch: gather each history, then attend.

    ``q`` is ``[S][Hq][D]`` raw storage; returns fp64 ``[S][Hq][D]``.  Paged
    storage changes only where the history lives, so the result is plain
    attention over the gathered contiguous history ([KG] "A Tiny Block-Table
    Example", closing paragraphs).
    """
    q = np.asarray(q)
    num_seqs, num_q_heads, _ = q.shape
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for i in range(num_seqs):
        kc, vc = gather_kv(k_pool, v_pool, block_tables[i], int(context_lens[i]),
                           num_kv_heads, block_size, head_dim, dtype)
        out[i] = attend(to_f64(q[i], dtype), to_f64(kc, dtype), to_f64(vc, dtype), scale)
    return out


def decode_one_head(q_group, k_pool, v_pool, block_table, context_len: int, kv_head: int,
                    scale: float, num_kv_heads: int, block_size: int, head_dim: int,
                    dtype: str) -> np.ndarray:
    """Decode for the query heads of one KV head of one request.

    Same arithmetic as ``decode`` restricted to one (request, KV head), so a
    large batch can be checked one piece at a time.  ``q_group`` is the
    ``[g][D]`` slice of query heads that read ``kv_head``.
    """
    kc, vc = gather_kv(k_pool, v_pool, block_table, context_len, num_kv_heads, block_size,
                       head_dim, dtype)
    keys = to_f64(kc[:, kv_head:kv_head + 1, :], dtype)
    values = to_f64(vc[:, kv_head:kv_head + 1, :], dtype)
    return attend(to_f64(np.asarray(q_group), dtype), keys, values, scale)


def prefill(q, q_start, k_pool, v_pool, block_tables, context_lens, scale: float,
            num_kv_heads: int, block_size: int, head_dim: int, dtype: str) -> np.ndarray:
    """Several new query tokens per request over the paged history.

    ``q`` is ``[T][Hq][D]`` raw storage holding every request's query tokens
    back to back: request i owns rows ``q_start[i] .. q_start[i+1]-1``.  They
    are the request's last ``n_i`` positions (their keys and values are in the
    cache, counted in ``context_lens[i] = L_i``), so its token j sits at
    position ``L_i - n_i + j`` and sees positions ``0 .. L_i - n_i + j``: its
    own and earlier ones, never a later one ([KG] "A Tiny Block-Table Example",
    closing paragraphs).  A token at a negative position sees nothing and
    gives zeros.  Returns fp64 ``[T][Hq][D]``.
    """
    q = np.asarray(q)
    q_start = [int(x) for x in q_start]
    total, num_q_heads, _ = q.shape
    out = np.zeros((total, num_q_heads, head_dim), dtype=np.float64)
    for i in range(len(q_start) - 1):
        n = q_start[i + 1] - q_start[i]
        L = int(context_lens[i])
        kc, vc = gather_kv(k_pool, v_pool, block_tables[i], max(L, 0), num_kv_heads,
                           block_size, head_dim, dtype)
        keys, values = to_f64(kc, dtype), to_f64(vc, dtype)
        for j in range(n):
            visible = max(L - n + j + 1, 0)
            row = q_start[i] + j
            out[row] = attend(to_f64(q[row], dtype), keys[:visible], values[:visible], scale)
    return out


# ----------------------------------------------------------------------------
# cache writes
# ----------------------------------------------------------------------------

def write_kv(k_pool, v_pool, k_new, v_new, slots, num_kv_heads: int, block_size: int,
             head_dim: int, dtype: str):
    """Scatter new tokens' K/V into copies of the pools; returns the copies.

    For each token with ``slot >= 0`` the physical block is ``slot //
    block_size`` and the offset ``slot % block_size`` ([KG] "Follow One Token
    Address" read backwards); every head's row is stored there, bit for bit.
    Tokens with a negative slot are padding and are skipped.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    k6 = _k_view(k_out, num_kv_heads, block_size, head_dim, dtype)
    v5 = _v_view(v_out, num_kv_heads, block_size, head_dim)
    x = 16 // ELEM_BYTES[dtype]
    tt = tile_tokens(block_size)
    k_new = np.asarray(k_new)
    v_new = np.asarray(v_new)
    for t, slot in enumerate(slots):
        slot = int(slot)
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        tile, pos = divmod(offset, tt)
        k6[block, :, tile, :, pos, :] = k_new[t].reshape(num_kv_heads, head_dim // x, x)
        v5[block, :, tile, :, pos] = v_new[t]
    return k_out, v_out


def copy_blocks(k_pool, v_pool, pairs):
    """Whole-block copies ``dst <- src`` on copies of the pools; returns them.

    [ZQ] answer / [KG] "Shared Blocks Must Not Be Changed in Place": before a
    branch changes a shared, partly filled block it gets a private copy of
    that block -- every slot, every head, K and V.  Pairs are applied in
    order.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    nb = k_out.shape[0]
    k2 = k_out.reshape(nb, -1)
    v2 = v_out.reshape(nb, -1)
    for src, dst in pairs:
        k2[int(dst)] = k2[int(src)]
        v2[int(dst)] = v2[int(src)]
    return k_out, v_out
