"""Python binding of libpagedkv (ctypes): argument marshalling only.

Every function here checks that its torch tensors are on the GPU, contiguous
and of the right dtype, passes their device pointers and the current HIP
stream to the C ABI declared in ``include/pa.h``, and raises ``PagedKVError``
with the library's message on a non-zero status.  All computation happens in
the HIP kernels; if ``libpagedkv.so`` is missing, loading fails loudly (there
is no CPU fallback).

Cache tensors are 2-D ``[num_blocks, Hkv * block_size * head_dim]`` views
with unit stride inside a block and ``block_stride`` elements between blocks
(``include/pa.h`` gives the layout).  ``kv_pool`` allocates the recommended
form: one buffer ``[num_blocks, 2, block]`` whose ``[:, 0]`` and ``[:, 1]``
views are the K and V caches.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedkv.so")
HEADERS = [os.path.join(os.path.dirname(HERE), "include", h) for h in ("pa.h", "pa_blocks.h")]

PA_F32, PA_BF16 = 0, 1
PA_DECODE_STREAM_KV = 1
PA_DECODE_GROUP_SHARED = 2
PA_DECODE_PREFIX_RUNS = 4
PA_DECODE_APPEND_TILES = 8
_DTYPES = {"f32": (PA_F32, torch.float32), "bf16": (PA_BF16, torch.bfloat16)}


class PagedKVError(RuntimeError):
    """A libpagedkv call returned a non-zero status."""

    def __init__(self, func: str, status: int, status_name: str, detail: str):
        super().__init__(f"{func} -> {status_name} ({status}): {detail}")
        self.status = status
        self.status_name = status_name
        self.detail = detail


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("block_stride", ctypes.c_int64)]


@dataclass(frozen=True)
class CacheSpec:
    """Shape of one layer's paged KV cache (the C ``pa_cache_desc_t``)."""

    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    dtype: str = "bf16"
    block_stride: int = 0          # elements between blocks; 0 = dense

    @property
    def torch_dtype(self) -> torch.dtype:
        return _DTYPES[self.dtype][1]

    @property
    def block_elems(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim

    @property
    def stride(self) -> int:
        return self.block_stride or self.block_elems

    def desc(self) -> CacheDesc:
        return CacheDesc(self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim,
                         _DTYPES[self.dtype][0], self.block_stride)

    @staticmethod
    def of(w) -> "CacheSpec":
        """The spec of a workload from ``inputs`` (anything with the same fields),
        with the block stride read off its cache tensors."""
        stride = int(w.k_cache.stride(0))
        elems = w.num_kv_heads * w.block_size * w.head_dim
        return CacheSpec(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.dtype,
                         0 if stride == elems else stride)


def kv_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int,
            dtype: str = "bf16", device="cuda", fill=None):
    """The recommended cache allocation: one buffer [num_blocks, 2, block] with
    K and V of a block adjacent.  Returns (spec, k_cache, v_cache) where the
    caches are [num_blocks, block] views into it."""
    elems = num_kv_heads * block_size * head_dim
    tdt = _DTYPES[dtype][1]
    if fill is None:
        buf = torch.empty((num_blocks, 2, elems), dtype=tdt, device=device)
    else:
        buf = torch.full((num_blocks, 2, elems), fill, dtype=tdt, device=device)
    spec = CacheSpec(num_blocks, block_size, num_kv_heads, head_dim, dtype, 2 * elems)
    return spec, buf[:, 0], buf[:, 1]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SIGNATURES = {
    "pa_abi_version": (ctypes.c_int, []),
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_write_kv": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _I32, _P]),
    "pa_copy_blocks": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _P]),
    "pa_slot_mapping": (ctypes.c_int, [_I32, _P, _I32, _I32, _P, _P, _I32, _P, _P]),
    "pa_gather_kv": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _I32, _P, _P, _P]),
    "pa_decode_partition_tokens": (_I32, [ctypes.POINTER(CacheDesc), _I32, _I32, _I32]),
    "pa_decode_workspace_bytes": (ctypes.c_size_t,
                                  [ctypes.POINTER(CacheDesc), _I32, _I32, _I32, _I32]),
    "pa_decode": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _I32, _I32,
                                 _I32, _I32, ctypes.c_float, _P, _P, ctypes.c_size_t, _I32,
                                 ctypes.c_uint32, _P]),
    "pa_decode_append": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _P, _P,
                                        _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P,
                                        ctypes.c_size_t, _I32, ctypes.c_uint32, _P]),
    "pa_decode_step": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _P, _P, _P,
                                      _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P,
                                      ctypes.c_size_t, _I32, ctypes.c_uint32, _P]),
    "pa_decode_step_noalloc": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _P,
                                              _P, _P, _I32, _I32, _I32, _I32, ctypes.c_float, _P,
                                              _I32, ctypes.c_uint32, _P]),
    "pa_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(CacheDesc), _I32, _I32, _I32,
                                                     _I32, _I32, _I32]),
    "pa_prefill": (ctypes.c_int, [ctypes.POINTER(CacheDesc), _P, _P, _P, _P, _P, _P, _I32, _I32,
                                  _I32, _I32, _I32, _I32, ctypes.c_float, _P, _P, ctypes.c_size_t,
                                  _I32, ctypes.c_uint32, _P]),
    # host-side block manager (include/pa_blocks.h)
    "pa_bm_create": (ctypes.c_int, [_I64, _I32, ctypes.c_uint32, ctypes.c_uint64,
                                    ctypes.POINTER(_P)]),
    "pa_bm_destroy": (None, [_P]),
    "pa_bm_num_free": (_I64, [_P]),
    "pa_bm_num_cached": (_I64, [_P]),
    "pa_bm_add": (ctypes.c_int, [_P, _P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "pa_bm_fork": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I64)]),
    "pa_bm_free": (ctypes.c_int, [_P, _I64]),
    "pa_bm_append": (ctypes.c_int, [_P, _P, _P, _I32, _P, _P, ctypes.POINTER(_I32)]),
    "pa_bm_slots": (ctypes.c_int, [_P, _I64, _I64, _I64, _P]),
    "pa_bm_tables": (ctypes.c_int, [_P, _P, _I32, _I32, _P, _P]),
    "pa_bm_seq_info": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "pa_bm_refcount": (ctypes.c_int, [_P, _I64, ctypes.POINTER(_I32)]),
    "pa_bm_block_key": (ctypes.c_uint64, [ctypes.c_uint64, _P, _I32]),
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_252_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list:
    """Names of the functions ``include/pa.h`` and ``include/pa_blocks.h`` declare."""
    names = set()
    for path in HEADERS:
        with open(path) as f:
            text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
        names |= set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def abi_version() -> int:
    return lib().pa_abi_version()


def status_string(status: int) -> str:
    return lib().pa_status_string(status).decode()


def last_error() -> str:
    return lib().pa_last_error().decode()


def _check(func: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(func, status, status_string(status), last_error())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, device=None, contiguous=True):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _cache_pair(spec: CacheSpec, k_cache, v_cache):
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t, name, spec.torch_dtype, k_cache.device, contiguous=False)
        if t.dim() != 2 or tuple(t.shape) != (spec.num_blocks, spec.block_elems):
            raise ValueError(f"{name} must be [num_blocks, Hkv * block_size * head_dim] = "
                             f"{(spec.num_blocks, spec.block_elems)}, got {tuple(t.shape)}")
        if t.stride(1) != 1 or (spec.num_blocks > 1 and t.stride(0) != spec.stride):
            raise ValueError(f"{name} strides {t.stride()} do not match block_stride "
                             f"{spec.stride}")
    return k_cache.device


# ----------------------------------------------------------------------------
# the C ABI, one function each
# ----------------------------------------------------------------------------

def write_kv(spec: CacheSpec, k_cache, v_cache, k_new, v_new, slot_mapping) -> None:
    """``pa_write_kv``: scatter new tokens' K/V through their slots."""
    dev = _cache_pair(spec, k_cache, v_cache)
    _need(k_new, "k_new", spec.torch_dtype, dev)
    _need(v_new, "v_new", spec.torch_dtype, dev)
    _need(slot_mapping, "slot_mapping", torch.int64, dev)
    n = slot_mapping.numel()
    per_tok = spec.num_kv_heads * spec.head_dim
    if k_new.numel() != n * per_tok or v_new.numel() != n * per_tok:
        raise ValueError("k_new/v_new must be [num_tokens, Hkv, head_dim]")
    d = spec.desc()
    _check("pa_write_kv", lib().pa_write_kv(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n,
                                            _stream(dev)))


def copy_blocks(spec: CacheSpec, k_cache, v_cache, block_pairs) -> None:
    """``pa_copy_blocks``: whole-block copies for copy-on-write."""
    dev = _cache_pair(spec, k_cache, v_cache)
    _need(block_pairs, "block_pairs", torch.int64, dev)
    if block_pairs.numel() % 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    d = spec.desc()
    _check("pa_copy_blocks", lib().pa_copy_blocks(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(block_pairs), block_pairs.numel() // 2,
                                                  _stream(dev)))


def slot_mapping(block_size: int, block_tables, positions, seq_ids=None, out=None):
    """``pa_slot_mapping``: flat slot of each (sequence, position); -1 if none."""
    _need(block_tables, "block_tables", torch.int32)
    dev = block_tables.device
    _need(positions, "positions", torch.int32, dev)
    if seq_ids is not None:
        _need(seq_ids, "seq_ids", torch.int32, dev)
        if seq_ids.numel() != positions.numel():
            raise ValueError("seq_ids and positions must have the same length")
    if block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    n = positions.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.int64, device=dev)
    _need(out, "out", torch.int64, dev)
    s, mb = block_tables.shape
    _check("pa_slot_mapping", lib().pa_slot_mapping(block_size, _ptr(block_tables), s, max(mb, 1),
                                                    _ptr(seq_ids), _ptr(positions), n, _ptr(out),
                                                    _stream(dev)))
    return out


def gather_kv(spec: CacheSpec, k_cache, v_cache, block_table, context_len: int):
    """``pa_gather_kv``: contiguous [L, Hkv, D] K and V of one request."""
    dev = _cache_pair(spec, k_cache, v_cache)
    _need(block_table, "block_table", torch.int32, dev)
    shape = (context_len, spec.num_kv_heads, spec.head_dim)
    k_out = torch.empty(shape, dtype=spec.torch_dtype, device=dev)
    v_out = torch.empty(shape, dtype=spec.torch_dtype, device=dev)
    d = spec.desc()
    _check("pa_gather_kv", lib().pa_gather_kv(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache),
                                              _ptr(block_table), context_len, _ptr(k_out),
                                              _ptr(v_out), _stream(dev)))
    return k_out, v_out


def decode_partition_tokens(spec: CacheSpec, num_seqs: int, num_q_heads: int,
                            max_context_len: int) -> int:
    d = spec.desc()
    return int(lib().pa_decode_partition_tokens(ctypes.byref(d), num_seqs, num_q_heads,
                                                max_context_len))


def decode_workspace_bytes(spec: CacheSpec, num_seqs: int, num_q_heads: int,
                           max_context_len: int, partition_tokens: int = 0) -> int:
    d = spec.desc()
    return int(lib().pa_decode_workspace_bytes(ctypes.byref(d), num_seqs, num_q_heads,
                                               max_context_len, partition_tokens))


def decode_workspace(spec: CacheSpec, num_seqs: int, num_q_heads: int, max_context_len: int,
                     partition_tokens: int = 0, device="cuda"):
    """A workspace for ``decode`` (uint8), or None when none is needed."""
    need = decode_workspace_bytes(spec, num_seqs, num_q_heads, max_context_len, partition_tokens)
    return None if need == 0 else torch.empty(need, dtype=torch.uint8, device=device)


def _decode_args(spec, q, k_cache, v_cache, block_tables, context_lens, max_context_len, out,
                 workspace, partition_tokens):
    dev = _cache_pair(spec, k_cache, v_cache)
    _need(q, "q", spec.torch_dtype, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 3 or q.shape[2] != spec.head_dim:
        raise ValueError("q must be [num_seqs, num_q_heads, head_dim]")
    s, hq, _ = q.shape
    if block_tables.dim() != 2 or block_tables.shape[0] != s or context_lens.numel() != s:
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", spec.torch_dtype, dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    if workspace is False:                     # the caller wants none allocated
        return dev, s, hq, out, None, 0
    if workspace is None:
        workspace = decode_workspace(spec, s, hq, max_context_len, partition_tokens, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace is not None:
        _need(workspace, "workspace", workspace.dtype, dev)
    return dev, s, hq, out, workspace, ws_bytes


def _flags(stream_kv: bool, group_shared: bool, prefix_runs: bool = False,
           append_tiles: bool = False) -> int:
    return ((PA_DECODE_STREAM_KV if stream_kv else 0) | (PA_DECODE_GROUP_SHARED if group_shared else 0)
            | (PA_DECODE_PREFIX_RUNS if prefix_runs else 0)
            | (PA_DECODE_APPEND_TILES if append_tiles else 0))


def decode(spec: CacheSpec, q, k_cache, v_cache, block_tables, context_lens,
           max_context_len: int, scale: float, out=None, workspace=None,
           partition_tokens: int = 0, stream_kv: bool = False, group_shared: bool = False,
           prefix_runs: bool = False):
    """``pa_decode``: attention of one query per request over its paged history.

    ``q`` is [num_seqs, Hq, head_dim]; returns ``out`` of the same shape and
    dtype.  ``workspace`` (>= ``decode_workspace_bytes``) is allocated here
    when not given.  ``stream_kv`` sets ``PA_DECODE_STREAM_KV``: a cache hint
    for batches in which no block is read by two requests.  ``group_shared``
    sets ``PA_DECODE_GROUP_SHARED``: consecutive requests that share leading
    blocks are decoded together and read those blocks once.  ``prefix_runs``
    sets ``PA_DECODE_PREFIX_RUNS``: for long runs of requests with a common
    prefix, partitions a whole chunk of requests shares are decoded once for
    all of them.
    """
    dev, s, hq, out, workspace, ws_bytes = _decode_args(
        spec, q, k_cache, v_cache, block_tables, context_lens, max_context_len, out, workspace,
        partition_tokens)
    d = spec.desc()
    _check("pa_decode", lib().pa_decode(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(q),
                                        _ptr(block_tables), _ptr(context_lens), s, hq,
                                        block_tables.shape[1], max_context_len, float(scale),
                                        _ptr(out), _ptr(workspace), ws_bytes,
                                        partition_tokens, _flags(stream_kv, group_shared, prefix_runs),
                                        _stream(dev)))
    return out


def decode_append(spec: CacheSpec, q, k_cache, v_cache, k_new, v_new, block_tables,
                  context_lens, max_context_len: int, scale: float, out=None, workspace=None,
                  partition_tokens: int = 0, stream_kv: bool = False,
                  group_shared: bool = False, prefix_runs: bool = False,
                  append_tiles: bool = False):
    """``pa_decode_append``: append each request's token at position L-1, then decode.

    ``k_new``/``v_new`` are [num_seqs, Hkv, head_dim]; the caches are written.
    ``append_tiles`` sets ``PA_DECODE_APPEND_TILES`` (the token's tile is
    written back whole; same bytes).
    """
    dev, s, hq, out, workspace, ws_bytes = _decode_args(
        spec, q, k_cache, v_cache, block_tables, context_lens, max_context_len, out, workspace,
        partition_tokens)
    _need(k_new, "k_new", spec.torch_dtype, dev)
    _need(v_new, "v_new", spec.torch_dtype, dev)
    per = s * spec.num_kv_heads * spec.head_dim
    if k_new.numel() != per or v_new.numel() != per:
        raise ValueError("k_new/v_new must be [num_seqs, Hkv, head_dim]")
    d = spec.desc()
    _check("pa_decode_append", lib().pa_decode_append(
        ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(q),
        _ptr(block_tables), _ptr(context_lens), s, hq, block_tables.shape[1], max_context_len,
        float(scale), _ptr(out), _ptr(workspace), ws_bytes, partition_tokens,
        _flags(stream_kv, group_shared, prefix_runs, append_tiles), _stream(dev)))
    return out


def decode_step(spec: CacheSpec, q, k_cache, v_cache, k_new, v_new, cow_src, block_tables,
                context_lens, max_context_len: int, scale: float, out=None, workspace=None,
                partition_tokens: int = 0, stream_kv: bool = False, group_shared: bool = False,
                prefix_runs: bool = False, append_tiles: bool = False):
    """``pa_decode_step``: copy-on-write of each request's last block from
    ``cow_src[i]`` (int32 [num_seqs], -1 = none), then append + decode."""
    dev, s, hq, out, workspace, ws_bytes = _decode_args(
        spec, q, k_cache, v_cache, block_tables, context_lens, max_context_len, out, workspace,
        partition_tokens)
    _need(k_new, "k_new", spec.torch_dtype, dev)
    _need(v_new, "v_new", spec.torch_dtype, dev)
    if cow_src is not None:
        _need(cow_src, "cow_src", torch.int32, dev)
        if cow_src.numel() != s:
            raise ValueError("cow_src must be [num_seqs]")
    per = s * spec.num_kv_heads * spec.head_dim
    if k_new.numel() != per or v_new.numel() != per:
        raise ValueError("k_new/v_new must be [num_seqs, Hkv, head_dim]")
    d = spec.desc()
    _check("pa_decode_step", lib().pa_decode_step(
        ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(cow_src),
        _ptr(q), _ptr(block_tables), _ptr(context_lens), s, hq, block_tables.shape[1],
        max_context_len, float(scale), _ptr(out), _ptr(workspace), ws_bytes, partition_tokens,
        _flags(stream_kv, group_shared, prefix_runs, append_tiles), _stream(dev)))
    return out


# the static scratch of pa_decode_step_noalloc (PA_DECODE_NOALLOC_MAX_BYTES in pa.h)
NOALLOC_MAX_BYTES = 64 << 20


def decode_step_noalloc(spec: CacheSpec, q, k_cache, v_cache, k_new, v_new, cow_src,
                        block_tables, context_lens, max_context_len: int, scale: float, out,
                        partition_tokens: int = 0, stream_kv: bool = False,
                        group_shared: bool = False, prefix_runs: bool = False,
                        append_tiles: bool = False):
    """``pa_decode_step_noalloc``: ``decode_step`` with the split-K partials
    in the library's static scratch instead of a workspace.  ``out`` must be
    given (nothing is allocated here either)."""
    if out is None:
        raise ValueError("decode_step_noalloc needs a preallocated out")
    dev, s, hq, out, _, _ = _decode_args(spec, q, k_cache, v_cache, block_tables, context_lens,
                                         max_context_len, out, False, partition_tokens)
    _need(k_new, "k_new", spec.torch_dtype, dev)
    _need(v_new, "v_new", spec.torch_dtype, dev)
    if cow_src is not None:
        _need(cow_src, "cow_src", torch.int32, dev)
        if cow_src.numel() != s:
            raise ValueError("cow_src must be [num_seqs]")
    per = s * spec.num_kv_heads * spec.head_dim
    if k_new.numel() != per or v_new.numel() != per:
        raise ValueError("k_new/v_new must be [num_seqs, Hkv, head_dim]")
    d = spec.desc()
    _check("pa_decode_step_noalloc", lib().pa_decode_step_noalloc(
        ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(cow_src),
        _ptr(q), _ptr(block_tables), _ptr(context_lens), s, hq, block_tables.shape[1],
        max_context_len, float(scale), _ptr(out), partition_tokens,
        _flags(stream_kv, group_shared, prefix_runs, append_tiles), _stream(dev)))
    return out


def prefill_workspace_bytes(spec: CacheSpec, num_seqs: int, total_q: int, max_q_len: int,
                            num_q_heads: int, max_context_len: int,
                            partition_tokens: int = 0) -> int:
    d = spec.desc()
    return int(lib().pa_prefill_workspace_bytes(ctypes.byref(d), num_seqs, total_q, max_q_len,
                                                num_q_heads, max_context_len, partition_tokens))


def prefill(spec: CacheSpec, q, q_start, k_cache, v_cache, block_tables, context_lens,
            max_q_len: int, max_context_len: int, scale: float, out=None, workspace=None,
            partition_tokens: int = 0):
    """``pa_prefill``: each request's last n_i positions as queries (rows
    ``q_start[i] .. q_start[i+1]-1`` of the packed ``q`` [total_q, Hq, head_dim]),
    each seeing its own and earlier positions.  Returns ``out`` like ``q``."""
    dev = _cache_pair(spec, k_cache, v_cache)
    _need(q, "q", spec.torch_dtype, dev)
    _need(q_start, "q_start", torch.int32, dev)
    _need(block_tables, "block_tables", torch.int32, dev)
    _need(context_lens, "context_lens", torch.int32, dev)
    if q.dim() != 3 or q.shape[2] != spec.head_dim:
        raise ValueError("q must be [total_q, Hq, head_dim]")
    s = context_lens.numel()
    if q_start.numel() != s + 1 or block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("q_start must be [num_seqs + 1] and block_tables [num_seqs, max_blocks]")
    total_q, hq = q.shape[0], q.shape[1]
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", spec.torch_dtype, dev)
    need = prefill_workspace_bytes(spec, s, total_q, max_q_len, hq, max_context_len,
                                   partition_tokens)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    d = spec.desc()
    _check("pa_prefill", lib().pa_prefill(ctypes.byref(d), _ptr(k_cache), _ptr(v_cache), _ptr(q),
                                          _ptr(q_start), _ptr(block_tables), _ptr(context_lens), s,
                                          total_q, max_q_len, hq, block_tables.shape[1],
                                          max_context_len, float(scale), _ptr(out),
                                          _ptr(workspace), ws_bytes, partition_tokens, 0,
                                          _stream(dev)))
    return out


# ---- host-side block manager (include/pa_blocks.h) ---------------------------

PA_BM_PREFIX_CACHE = 1


def _host_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


class BlockManager:
    """``pa_bm_*``: the pool's free list, reference counts, tables, growth,
    fork, free, copy-on-write decisions and (optionally) the prefix cache of
    full blocks.  Host-side: arguments and results are numpy arrays."""

    def __init__(self, num_blocks: int, block_size: int, prefix_cache: bool = False,
                 salt: int = 0):
        import numpy as np
        self._np = np
        self.block_size = block_size
        h = ctypes.c_void_p()
        _check("pa_bm_create", lib().pa_bm_create(
            num_blocks, block_size, PA_BM_PREFIX_CACHE if prefix_cache else 0,
            ctypes.c_uint64(salt & ((1 << 64) - 1)), ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if self._h:
            lib().pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_free(self) -> int:
        return int(lib().pa_bm_num_free(self._h))

    @property
    def num_cached(self) -> int:
        return int(lib().pa_bm_num_cached(self._h))

    def add(self, num_tokens: int = 0, tokens=None) -> tuple:
        """Admit a request; returns (seq_id, cached prompt tokens)."""
        np = self._np
        t = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        n = num_tokens if t is None else int(t.size)
        sid, cached = _I64(), _I64()
        _check("pa_bm_add", lib().pa_bm_add(self._h, _host_ptr(t), n, ctypes.byref(sid),
                                             ctypes.byref(cached)))
        return sid.value, cached.value

    def fork(self, parent: int) -> int:
        child = _I64()
        _check("pa_bm_fork", lib().pa_bm_fork(self._h, parent, ctypes.byref(child)))
        return child.value

    def free(self, seq_id: int) -> None:
        _check("pa_bm_free", lib().pa_bm_free(self._h, seq_id))

    def append(self, seq_ids, tokens=None) -> tuple:
        """One decode step; returns (slots int64 [n], cow_pairs int64 [k, 2])."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = int(ids.size)
        t = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
        if t is not None and t.size != n:
            raise ValueError("one token id per request")
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((n, 2), dtype=np.int64)
        k = _I32()
        _check("pa_bm_append", lib().pa_bm_append(self._h, _host_ptr(ids), _host_ptr(t), n,
                                                   _host_ptr(slots), _host_ptr(pairs),
                                                   ctypes.byref(k)))
        return slots, pairs[:k.value].copy()

    def slots(self, seq_id: int, start: int, count: int):
        np = self._np
        out = np.empty(count, dtype=np.int64)
        _check("pa_bm_slots", lib().pa_bm_slots(self._h, seq_id, start, count, _host_ptr(out)))
        return out

    def tables(self, seq_ids, max_blocks: int) -> tuple:
        """(tables int32 [n, max_blocks] with -1 padding, lens int32 [n])."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = int(ids.size)
        tab = np.empty((n, max_blocks), dtype=np.int32)
        lens = np.empty(n, dtype=np.int32)
        _check("pa_bm_tables", lib().pa_bm_tables(self._h, _host_ptr(ids), n, max_blocks,
                                                   _host_ptr(tab), _host_ptr(lens)))
        return tab, lens

    def seq_info(self, seq_id: int) -> tuple:
        length, nb = _I64(), _I64()
        _check("pa_bm_seq_info", lib().pa_bm_seq_info(self._h, seq_id, ctypes.byref(length),
                                                       ctypes.byref(nb)))
        return length.value, nb.value

    def refcount(self, block: int) -> int:
        r = _I32()
        _check("pa_bm_refcount", lib().pa_bm_refcount(self._h, block, ctypes.byref(r)))
        return r.value


def block_key(parent: int, tokens) -> int:
    """``pa_bm_block_key``: the prefix-cache key of one full block."""
    import numpy as np
    t = np.ascontiguousarray(tokens, dtype=np.int32)
    return int(lib().pa_bm_block_key(ctypes.c_uint64(parent & ((1 << 64) - 1)), _host_ptr(t),
                                      int(t.size)))
