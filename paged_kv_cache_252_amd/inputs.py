"""Seeded synthetic workloads for paged decode attention.

This module only draws random numbers and lays out the *structure* of a
workload (which physical blocks each request's table names, which blocks are
shared, which blocks a copy-on-write step copies into).  It holds none of the
arithmetic of the method: no address translation, no attention, no scatter.
Both the GPU library's tests/benchmark and the CPU oracle consume what it
produces, so it imports neither of them.

Recipe (all workloads):

* Structure comes from ``numpy.random.Generator(PCG64(seed))``, drawn in the
  order: context lengths, then one permutation of the pool whose entries are
  handed out in (request, logical block) order.  Lengths are integer-uniform
  with inclusive bounds.
* Values (q, cached K/V, new-token K/V) are iid N(0, 1), drawn with a
  ``torch.Generator`` seeded with the same seed on the target device, in the
  order q, K/V of the referenced blocks, new-token K/V, and rounded to the
  storage dtype by torch (round-to-nearest-even for bf16).
* Blocks that no table references are filled with quiet NaN when
  ``poison=True`` (so reading one shows up in the output) and zeros
  otherwise.  Table entries past a request's last block are -1.
* K and V live in one buffer ``[num_blocks, 2, Hkv * block_size * head_dim]``
  (the library's recommended allocation); ``k_cache`` and ``v_cache`` are
  its ``[:, 0]`` and ``[:, 1]`` views.  ``separate_pools`` converts a
  workload to two dense buffers instead.

Named presets follow the five workload descriptions of the paged decode
benchmark: a tiny fp32 example built around the worked block table
[9, 2, 14]; GQA decode (also at head_dim 64 and 256, and in fp32); a long
shared prefix; long-context split-K; and a fan-out step in which four
branches share each prompt and each branch copies the prompt's partly filled
last block before writing its new token.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPE = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclass
class Workload:
    """A batch of decode requests over a paged KV pool (torch tensors)."""

    name: str
    dtype: str                      # storage/compute dtype of q, K, V, out: 'bf16' or 'f32'
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    context_lens: torch.Tensor      # int32 [S]
    block_tables: torch.Tensor      # int32 [S][max_blocks]; -1 past the last block
    q: torch.Tensor                 # [S][Hq][D]
    k_cache: torch.Tensor           # [num_blocks][Hkv * block_size * head_dim] (view)
    v_cache: torch.Tensor           # [num_blocks][Hkv * block_size * head_dim] (view)
    # the token each request writes this step (fan-out step and benchmark step)
    new_k: torch.Tensor | None = None        # [T][Hkv][D]
    new_v: torch.Tensor | None = None        # [T][Hkv][D]
    new_seq: torch.Tensor | None = None      # int32 [T]: request of each new token
    new_pos: torch.Tensor | None = None      # int32 [T]: logical position of each new token
    cow_pairs: torch.Tensor | None = None    # int64 [N][2]: (src, dst) block copies
    # structure, for tests: which blocks are shared by several tables
    shared_blocks: np.ndarray | None = None
    parent_tables: list | None = None        # fan-out: the prompt tables before copy-on-write
    q_chunk: torch.Tensor | None = None      # packed [total, Hq, D] queries of the last positions
    q_start: torch.Tensor | None = None      # int32 [S + 1] row offsets into q_chunk
    max_q_len: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max().item()) if self.num_seqs else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def block_elems(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim

    def referenced_blocks(self) -> np.ndarray:
        bt = self.block_tables.cpu().numpy()
        return np.unique(bt[bt >= 0])


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _table_array(tables, max_blocks: int) -> np.ndarray:
    out = np.full((len(tables), max_blocks), -1, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, :len(t)] = t
    return out


def _values(gen: torch.Generator, shape, dtype: str, device) -> torch.Tensor:
    x = torch.randn(shape, generator=gen, dtype=torch.float32, device=device)
    return x.to(TORCH_DTYPE[dtype])


def _fill_pool(pool: torch.Tensor, blocks: np.ndarray, gen, dtype: str, chunk: int = 4096):
    """N(0,1) values into ``pool`` rows ``blocks`` (in the given order)."""
    ids = torch.as_tensor(np.asarray(blocks, dtype=np.int64), device=pool.device)
    for lo in range(0, len(blocks), chunk):
        sel = ids[lo:lo + chunk]
        pool[sel] = _values(gen, (sel.numel(), pool.shape[1]), dtype, pool.device)


def _finish(name, dtype, bs, hq, hkv, d, num_blocks, lens, tables, max_blocks, seed, device,
            poison, value_blocks, scale=None, **kw) -> Workload:
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    dev = torch.device(device)
    s = len(lens)
    q = _values(gen, (s, hq, d), dtype, dev)
    elems = hkv * bs * d
    buf = torch.full((num_blocks, 2, elems), float("nan") if poison else 0.0,
                     dtype=TORCH_DTYPE[dtype], device=dev)
    k_cache, v_cache = buf[:, 0], buf[:, 1]
    _fill_pool(k_cache, value_blocks, gen, dtype)
    _fill_pool(v_cache, value_blocks, gen, dtype)
    return Workload(
        name=name, dtype=dtype, block_size=bs, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
        num_blocks=num_blocks, scale=(1.0 / math.sqrt(d)) if scale is None else scale,
        context_lens=torch.as_tensor(np.asarray(lens, dtype=np.int32), device=dev),
        block_tables=torch.as_tensor(_table_array(tables, max_blocks), device=dev),
        q=q, k_cache=k_cache, v_cache=v_cache, extra={"seed": seed, "gen": gen}, **kw)


# ----------------------------------------------------------------------------
# presets
# ----------------------------------------------------------------------------

def tiny(seed: int = 0, device="cpu", poison: bool = True) -> Workload:
    """2 requests of 9 and 6 tokens, block size 4, 2 q heads = 2 KV heads,
    head_dim 16, fp32, 16-block pool.  Request 0 uses the table [9, 2, 14];
    request 1 takes the first two blocks of a seeded permutation of the 13
    blocks left.  scale = 1/sqrt(16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [9, 6]
    t0 = [9, 2, 14]
    rest = np.array([b for b in range(16) if b not in t0])
    t1 = [int(b) for b in rest[rng.permutation(len(rest))][:2]]
    tables = [t0, t1]
    used = np.array(t0 + t1)
    return _finish("tiny", "f32", 4, 2, 2, 16, 16, lens, tables, 3, seed, device, poison, used,
                   scale=0.25)


def paged_random(name: str, num_seqs: int, len_lo: int, len_hi: int, num_q_heads: int,
                 num_kv_heads: int, head_dim: int = 128, block_size: int = 16,
                 dtype: str = "bf16", num_blocks: int | None = 65536,
                 max_blocks: int | None = None, seed: int = 1, device="cpu",
                 poison: bool = True, lens=None) -> Workload:
    """Independent requests with lengths U[len_lo, len_hi] and blocks drawn
    shuffled from the pool (``num_blocks=None`` sizes the pool to fit)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if lens is None:
        lens = rng.integers(len_lo, len_hi, size=num_seqs, endpoint=True).tolist()
    counts = [_ceil_div(int(L), block_size) for L in lens]
    total = sum(counts)
    if num_blocks is None:
        num_blocks = max(total, 1)
    if total > num_blocks:
        raise ValueError(f"workload needs {total} blocks, pool has {num_blocks}")
    perm = rng.permutation(num_blocks)
    tables, at = [], 0
    for c in counts:
        tables.append([int(b) for b in perm[at:at + c]])
        at += c
    if max_blocks is None:
        max_blocks = max(1, _ceil_div(len_hi, block_size))
    return _finish(name, dtype, block_size, num_q_heads, num_kv_heads, head_dim, num_blocks,
                   lens, tables, max_blocks, seed, device, poison, perm[:total])


def gqa(seed: int = 1, device="cpu", poison: bool = True, num_seqs: int = 32,
        len_lo: int = 512, len_hi: int = 4096, num_blocks: int = 65536,
        head_dim: int = 128, dtype: str = "bf16") -> Workload:
    """GQA decode: 32 requests, L ~ U[512, 4096], 32 q / 8 KV heads, D 128
    (or ``head_dim``), block size 16, bf16 (or ``dtype``), blocks shuffled
    from a 65536-block pool."""
    name = "gqa" + ("" if head_dim == 128 else f"_d{head_dim}") + ("" if dtype == "bf16" else f"_{dtype}")
    return paged_random(name, num_seqs, len_lo, len_hi, 32, 8, head_dim=head_dim, dtype=dtype,
                        seed=seed, device=device, poison=poison, num_blocks=num_blocks)


def gqa_d64(**kw) -> Workload:
    """The GQA decode workload at head_dim 64."""
    return gqa(head_dim=64, **kw)


def gqa_d256(**kw) -> Workload:
    """The GQA decode workload at head_dim 256."""
    return gqa(head_dim=256, **kw)


def gqa_f32(**kw) -> Workload:
    """The GQA decode workload on an fp32 cache."""
    return gqa(dtype="f32", **kw)


def long_context(seed: int = 3, device="cpu", poison: bool = True, num_seqs: int = 8,
                 len_lo: int = 32768, len_hi: int = 131072) -> Workload:
    """Long-context split-K: 8 requests, L ~ U[32768, 131072], 64 q / 8 KV
    heads, D 128, block size 16, bf16, pool sized to fit, shuffled."""
    return paged_random("long", num_seqs, len_lo, len_hi, 64, 8, seed=seed, device=device,
                        poison=poison, num_blocks=None)


def shared_prefix(seed: int = 2, device="cpu", poison: bool = True, num_seqs: int = 256,
                  prefix_len: int = 2048, suffix_lo: int = 64, suffix_hi: int = 512,
                  num_blocks: int = 65536, num_q_heads: int = 32, num_kv_heads: int = 8) -> Workload:
    """Shared prefix: every request's first ``prefix_len`` tokens live in the
    same physical blocks; each request then has a private suffix of
    U[suffix_lo, suffix_hi] tokens.  ``prefix_len`` is a whole number of
    blocks here (2048 = 128 blocks of 16)."""
    bs = 16
    if prefix_len % bs:
        raise ValueError("the shared prefix must be a whole number of blocks")
    rng = np.random.Generator(np.random.PCG64(seed))
    suffix = rng.integers(suffix_lo, suffix_hi, size=num_seqs, endpoint=True)
    lens = [prefix_len + int(s) for s in suffix]
    n_prefix = prefix_len // bs
    counts = [_ceil_div(int(s), bs) for s in suffix]
    total = n_prefix + sum(counts)
    if total > num_blocks:
        raise ValueError(f"workload needs {total} blocks, pool has {num_blocks}")
    perm = rng.permutation(num_blocks)
    prefix_blocks = [int(b) for b in perm[:n_prefix]]
    tables, at = [], n_prefix
    for c in counts:
        tables.append(prefix_blocks + [int(b) for b in perm[at:at + c]])
        at += c
    max_blocks = _ceil_div(prefix_len + suffix_hi, bs)
    w = _finish("prefix", "bf16", bs, num_q_heads, num_kv_heads, 128, num_blocks, lens, tables,
                max_blocks, seed, device, poison, perm[:total])
    w.shared_blocks = np.asarray(prefix_blocks)
    return w


def fanout(seed: int = 4, device="cpu", poison: bool = True, num_prompts: int = 128,
           branches: int = 4, prompt_lo: int = 256, prompt_hi: int = 2048,
           num_blocks: int = 65536) -> Workload:
    """Fan-out decode step: ``num_prompts`` prompts, each shared by
    ``branches`` sampling branches.  Prompt lengths are U[prompt_lo,
    prompt_hi], redrawn while a multiple of the block size, so the last
    prompt block is partly filled.  Full prompt blocks stay shared; each
    branch gets a fresh block, receives a copy of the prompt's partial last
    block (one copy-on-write pair per branch) and then writes one new token
    at position ``prompt_len``, so the decode runs over ``prompt_len + 1``
    tokens.  Request ``p * branches + b`` is branch ``b`` of prompt ``p``.

    The pre-copy prompt tables are kept in ``parent_tables``; ``block_tables``
    are the branch tables after the copy.
    """
    bs = 16
    rng = np.random.Generator(np.random.PCG64(seed))
    plens = []
    for _ in range(num_prompts):
        n = int(rng.integers(prompt_lo, prompt_hi, endpoint=True))
        while n % bs == 0:
            n = int(rng.integers(prompt_lo, prompt_hi, endpoint=True))
        plens.append(n)
    need = sum(_ceil_div(n, bs) + branches for n in plens)
    if need > num_blocks:
        raise ValueError(f"workload needs {need} blocks, pool has {num_blocks}")
    perm = rng.permutation(num_blocks)
    at = 0
    parent_tables, tables, pairs, lens, seqs, pos = [], [], [], [], [], []
    shared = []
    for p, n in enumerate(plens):
        nb = _ceil_div(n, bs)
        prompt = [int(b) for b in perm[at:at + nb]]
        at += nb
        parent_tables.append(prompt)
        shared.extend(prompt)
        for b in range(branches):
            dst = int(perm[at])
            at += 1
            tables.append(prompt[:-1] + [dst])
            pairs.append((prompt[-1], dst))
            lens.append(n + 1)
            seqs.append(p * branches + b)
            pos.append(n)
    max_blocks = _ceil_div(prompt_hi + 1, bs)
    prompt_blocks = np.asarray(shared)
    w = _finish("fanout", "bf16", bs, 32, 8, 128, num_blocks, lens, tables, max_blocks, seed,
                device, poison, prompt_blocks)
    dev = torch.device(device)
    t = len(lens)
    w.new_k = _values(w.extra["gen"], (t, 8, 128), "bf16", dev)
    w.new_v = _values(w.extra["gen"], (t, 8, 128), "bf16", dev)
    w.new_seq = torch.as_tensor(np.asarray(seqs, dtype=np.int32), device=dev)
    w.new_pos = torch.as_tensor(np.asarray(pos, dtype=np.int32), device=dev)
    w.cow_pairs = torch.as_tensor(np.asarray(pairs, dtype=np.int64).reshape(-1, 2), device=dev)
    w.shared_blocks = prompt_blocks
    w.parent_tables = parent_tables
    w.extra["prompt_lens"] = plens
    w.extra["branches"] = branches
    return w


def separate_pools(w: Workload) -> Workload:
    """Move the caches into two dense buffers (block stride = one block)."""
    w.k_cache = w.k_cache.contiguous()
    w.v_cache = w.v_cache.contiguous()
    return w


def add_step_tokens(w: Workload) -> Workload:
    """Give each request one new token to write at its last position ``L-1``.

    The decode step then writes that token's K/V and attends over ``L``
    positions including it.  Rewriting the same token is idempotent, so the
    step can be repeated.
    """
    dev = w.q.device
    s = w.num_seqs
    gen = w.extra["gen"]
    w.new_k = _values(gen, (s, w.num_kv_heads, w.head_dim), w.dtype, dev)
    w.new_v = _values(gen, (s, w.num_kv_heads, w.head_dim), w.dtype, dev)
    w.new_seq = torch.arange(s, dtype=torch.int32, device=dev)
    w.new_pos = (w.context_lens - 1).to(torch.int32)
    return w


def add_query_chunks(w: Workload, chunk_lens) -> Workload:
    """Give request i a chunk of ``chunk_lens[i]`` query tokens: its last
    positions, whose K/V are already in the cache.  Sets ``w.q_chunk`` (packed
    [total, Hq, D], N(0,1)), ``w.q_start`` (int32 [S + 1]) and
    ``w.max_q_len``."""
    dev = w.q.device
    n = [int(c) for c in chunk_lens]
    if len(n) != w.num_seqs or min(n, default=0) < 0:
        raise ValueError("one non-negative chunk length per request")
    start = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    w.q_chunk = _values(w.extra["gen"], (int(start[-1]), w.num_q_heads, w.head_dim), w.dtype, dev)
    w.q_start = torch.as_tensor(start, device=dev)
    w.max_q_len = max(n, default=0)
    return w


def prefill_chunk(seed: int = 5, device="cpu", poison: bool = True, num_seqs: int = 16,
                  cached_lo: int = 1024, cached_hi: int = 3072, chunk: int = 256,
                  num_blocks: int = 65536, head_dim: int = 128) -> Workload:
    """Chunked prefill after a prefix-cache hit: ``num_seqs`` requests, each
    with U[cached_lo, cached_hi] cached positions followed by ``chunk`` new
    ones whose queries attend causally; 32 q / 8 KV heads, D ``head_dim``
    (128 by default), bs 16, bf16, blocks shuffled from the pool."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = (rng.integers(cached_lo, cached_hi, size=num_seqs, endpoint=True) + chunk).tolist()
    w = paged_random("prefill", num_seqs, 0, cached_hi + chunk, 32, 8, head_dim=head_dim, seed=seed,
                     num_blocks=num_blocks, device=device, poison=poison, lens=lens)
    return add_query_chunks(w, [chunk] * num_seqs)


def replicate(w: Workload, replicas: int, seed_offset: int = 1000) -> list:
    """Tables for ``replicas`` copies of the workload at disjoint physical blocks.

    Copy 0 is the workload's own table set.  Copies 1.. place the same
    logical content (the same bytes, block by block) at blocks drawn
    shuffled from the blocks no table uses yet.  Returns a list of int32
    table tensors; the pools are extended in place.
    """
    if replicas < 1:
        raise ValueError("replicas must be >= 1")
    bt = w.block_tables.cpu().numpy()
    used = w.referenced_blocks()
    free = np.setdiff1d(np.arange(w.num_blocks), used)
    need = used.size * (replicas - 1)
    if need > free.size:
        raise ValueError(f"{replicas} replicas need {need} spare blocks, pool has {free.size}")
    rng = np.random.Generator(np.random.PCG64(w.extra["seed"] + seed_offset))
    free = free[rng.permutation(free.size)]
    out = [w.block_tables]
    dev = w.block_tables.device
    src = torch.as_tensor(used.astype(np.int64), device=dev)
    for r in range(1, replicas):
        ids = free[(r - 1) * used.size: r * used.size]
        remap = np.full(w.num_blocks, -1, dtype=np.int64)
        remap[used] = ids
        t = np.where(bt >= 0, remap[np.maximum(bt, 0)], -1).astype(np.int32)
        dst = torch.as_tensor(ids.astype(np.int64), device=dev)
        w.k_cache[dst] = w.k_cache[src]
        w.v_cache[dst] = w.v_cache[src]
        out.append(torch.as_tensor(t, device=dev))
    return out


PRESETS = {
    "tiny": tiny,
    "gqa": gqa,
    "gqa_d64": gqa_d64,
    "gqa_d256": gqa_d256,
    "gqa_f32": gqa_f32,
    "prefix": shared_prefix,
    "long": long_context,
    "fanout": fanout,
    "prefill": prefill_chunk,
}
