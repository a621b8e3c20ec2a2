"""The C-ABI library loads and exports what include/pa.h declares (no GPU needed).

Only host-side paths run here: version and status queries, and argument
checks that reject a call before it touches the HIP runtime.
"""

import ctypes
import os

import pytest

from paged_kv_cache_252_amd import ops


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from paged_kv_cache_252_amd import build
        build.build()
    return ops.lib()


def test_exports_every_declared_function(lib):
    names = ops.header_functions()
    assert {"pa_write_kv", "pa_decode", "pa_copy_blocks"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"{name} declared in pa.h but not exported"
    assert set(ops._SIGNATURES) == set(names), "binding and header disagree"


def test_version_and_status_strings(lib):
    assert ops.abi_version() == 5
    assert ops.status_string(0) == "PA_OK"
    assert ops.status_string(5) == "PA_ERR_UNSUPPORTED"
    assert ops.status_string(8) == "PA_ERR_VALIDATE"
    assert ops.status_string(99) == "PA_ERR_UNKNOWN"


def _desc(**kw):
    base = dict(num_blocks=64, block_size=16, num_kv_heads=8, head_dim=128, dtype=1,
                block_stride=0)
    base.update(kw)
    return ops.CacheDesc(**base)


def _decode(lib, d, num_seqs=2, num_q_heads=32, max_blocks=4, max_len=64, ptr=1 << 20,
            part=16, scale=0.1, flags=0):
    p = ctypes.c_void_p(ptr)
    return lib.pa_decode(ctypes.byref(d) if d is not None else None, p, p, p, p, p, num_seqs,
                         num_q_heads, max_blocks, max_len, scale, p, p, 1 << 30, part, flags,
                         None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 3),
    (dict(num_blocks=0), 2),
    (dict(block_size=0), 5),
    (dict(block_size=512), 5),
    (dict(head_dim=96), 5),
    (dict(num_kv_heads=0), 2),
    (dict(block_stride=1000), 2),                 # smaller than one block (16384)
    (dict(block_stride=16384 + 4), 4),            # not a multiple of 16 bytes
])
def test_bad_descriptor_rejected(lib, kw, status):
    assert _decode(lib, _desc(**kw)) == status
    assert ops.last_error()


def test_decode_argument_checks(lib):
    assert _decode(lib, None) == 1                                  # NULL descriptor
    assert _decode(lib, _desc(), num_q_heads=30) == 2               # not a multiple of Hkv
    assert _decode(lib, _desc(), max_len=65) == 2                   # beyond table capacity
    assert _decode(lib, _desc(), scale=float("nan")) == 2
    assert _decode(lib, _desc(), num_seqs=-1) == 2
    assert _decode(lib, _desc(), part=24) == 2                      # not a multiple of 16
    assert _decode(lib, _desc(), part=2048) == 2                    # above 1024
    # the MFMA decode at other block sizes: whole blocks and tiles, one table
    # entry per lane (at most 64 blocks of 8 = 512 tokens)
    assert _decode(lib, _desc(block_size=8), max_blocks=8, part=1024) == 2
    assert _decode(lib, _desc(block_size=8), max_blocks=8, part=8) == 2
    assert _decode(lib, _desc(block_size=32), max_blocks=2, part=16) == 2
    assert _decode(lib, _desc(), ptr=(1 << 20) + 8) == 4            # misaligned buffers
    assert _decode(lib, _desc(), flags=16) == 5                     # unknown flag bit
    d = _desc()
    assert lib.pa_decode(ctypes.byref(d), None, None, None, None, None, 2, 32, 4, 64, 0.1, None,
                         None, 0, 16, 0, None) == 1
    assert "NULL" in ops.last_error()
    assert _decode(lib, _desc(), num_seqs=0) == 0                   # nothing to do
    assert ops.last_error() == ""


def test_workspace_size_rules(lib):
    d = _desc()
    # one partition: no workspace
    assert lib.pa_decode_workspace_bytes(ctypes.byref(d), 4, 32, 64, 64) == 0
    # 4 partitions of 16 over 64 tokens: S * Hq * parts * (D + 2) floats
    assert lib.pa_decode_workspace_bytes(ctypes.byref(d), 4, 32, 64, 16) == 4 * 32 * 4 * 130 * 4
    p = ctypes.c_void_p(1 << 20)
    st = lib.pa_decode(ctypes.byref(d), p, p, p, p, p, 4, 32, 4, 64, 0.1, p, p, 100, 16, 0, None)
    assert st == 6 and "workspace" in ops.last_error()


def test_cache_op_argument_checks(lib):
    d = _desc()
    p = ctypes.c_void_p(1 << 20)
    assert lib.pa_write_kv(ctypes.byref(d), p, p, p, p, p, -1, None) == 2
    assert lib.pa_write_kv(ctypes.byref(d), p, p, p, p, p, 0, None) == 0
    assert lib.pa_write_kv(ctypes.byref(d), None, p, p, p, p, 3, None) == 1
    assert lib.pa_write_kv(ctypes.byref(d), p, p, ctypes.c_void_p((1 << 20) + 4), p, p, 3,
                           None) == 4
    assert lib.pa_copy_blocks(ctypes.byref(d), p, p, None, 2, None) == 1
    assert lib.pa_copy_blocks(ctypes.byref(d), p, p, p, -2, None) == 2
    assert lib.pa_slot_mapping(0, p, 1, 1, None, p, 1, p, None) == 2
    assert lib.pa_slot_mapping(16, p, 1, 1, None, None, 1, p, None) == 1
    assert lib.pa_gather_kv(ctypes.byref(d), p, p, p, -1, p, p, None) == 2


def _prefill(lib, d, num_seqs=2, total_q=4, max_q_len=2, num_q_heads=32, max_blocks=4,
             max_len=64, part=0, flags=0, scale=0.1, ws=1 << 30):
    p = ctypes.c_void_p(1 << 20)
    return lib.pa_prefill(ctypes.byref(d), p, p, p, p, p, p, num_seqs, total_q, max_q_len,
                          num_q_heads, max_blocks, max_len, scale, p, p, ws, part, flags, None)


def test_prefill_argument_checks(lib):
    """pa_prefill rejects what it cannot run before touching the device."""
    d = _desc()
    f32 = _desc(dtype=0, head_dim=32, block_size=4)
    # shapes outside the MFMA prefill kernels (g = 3; fp32) take the rows-as-
    # decodes route, whose workspace always holds the row tables and lengths
    for dd, hq, mb in ((d, 24, 4), (f32, 32, 16)):
        assert _prefill(lib, dd, num_q_heads=hq, max_blocks=mb, ws=16) == 6
        assert _prefill(lib, dd, num_q_heads=hq, max_blocks=mb, flags=1) == 5
        assert _prefill(lib, dd, num_q_heads=hq, max_blocks=mb, total_q=70000) == 2
    assert _prefill(lib, f32, max_blocks=16, part=6) == 2            # decode's partition rule
    bs = 4
    rb = 64 // bs
    parts = 64 // 16
    want = 4 * rb * 4 + 16 + 4 * 32 * parts * (32 + 2) * 4             # tables, lengths, partials
    assert lib.pa_prefill_workspace_bytes(ctypes.byref(f32), 2, 4, 2, 32, 64, 16) == want
    assert lib.pa_prefill_workspace_bytes(ctypes.byref(f32), 2, 4, 2, 32, 16, 16) == 4 * 4 * 4 + 16
    assert _prefill(lib, d, total_q=-1) == 2
    assert _prefill(lib, d, total_q=70000) == 2
    assert _prefill(lib, d, max_q_len=-3) == 2
    assert _prefill(lib, d, max_len=65) == 2                       # beyond table capacity
    assert _prefill(lib, d, flags=1) == 5
    assert _prefill(lib, d, part=24) == 2
    assert _prefill(lib, d, num_seqs=40000, max_q_len=8) == 2      # grid rows above 65535
    assert _prefill(lib, d, num_seqs=0) == 0                        # nothing to do
    assert _prefill(lib, d, total_q=0) == 0
    ws = lib.pa_prefill_workspace_bytes(ctypes.byref(d), 2, 4, 2, 32, 64, 16)
    assert ws == 4 * 32 * 4 * (128 + 2) * 4 + 16                    # partials + row lengths
    assert lib.pa_prefill_workspace_bytes(ctypes.byref(d), 2, 4, 2, 32, 16, 16) == 0
