"""Test helpers: move workload tensors into the oracle's numpy form.

bf16 tensors become their raw uint16 bit patterns, fp32 stays float32, so the
oracle sees exactly the bytes the library sees.
"""

import numpy as np
import torch


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_args(w):
    """The keyword arguments shared by the oracle's cache functions."""
    return dict(num_kv_heads=w.num_kv_heads, block_size=w.block_size, head_dim=w.head_dim,
                dtype=w.dtype)


def oracle_decode(w, block_tables=None, k_cache=None, v_cache=None, context_lens=None):
    from oracle import paged
    bt = to_np(w.block_tables if block_tables is None else block_tables)
    return paged.decode(to_np(w.q), to_np(w.k_cache if k_cache is None else k_cache),
                        to_np(w.v_cache if v_cache is None else v_cache), bt,
                        to_np(w.context_lens if context_lens is None else context_lens),
                        w.scale, **oracle_args(w))


def tail_element_mask(w, offset_from: int):
    """Boolean masks over one block's flattened K and V elements selecting the
    token offsets >= offset_from, built through the oracle's layout reading."""
    from oracle import paged
    n = w.block_elems
    idx = np.arange(n, dtype=np.int64)
    k_rows, v_rows = paged.block_tokens(idx.reshape(1, n), idx.reshape(1, n), 0,
                                        w.num_kv_heads, w.block_size, w.head_dim, w.dtype)
    kmask = np.zeros(n, dtype=bool)
    vmask = np.zeros(n, dtype=bool)
    kmask[k_rows[offset_from:].reshape(-1)] = True
    vmask[v_rows[offset_from:].reshape(-1)] = True
    return kmask, vmask


def poison_tails(w):
    """Set every slot at or past each request's length, in its last block, to NaN."""
    bt = w.block_tables.cpu().numpy()
    lens = w.context_lens.cpu().numpy()
    for i, L in enumerate(lens):
        L = int(L)
        if L == 0 or L % w.block_size == 0:
            continue
        last = int(bt[i, (L - 1) // w.block_size])
        kmask, vmask = tail_element_mask(w, L % w.block_size)
        km = torch.as_tensor(kmask, device=w.k_cache.device)
        vm = torch.as_tensor(vmask, device=w.v_cache.device)
        w.k_cache[last, km] = float("nan")
        w.v_cache[last, vm] = float("nan")
    return w
