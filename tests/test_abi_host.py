"""The C-ABI library loads on a machine without a GPU, exports every function
include/splitzip.h declares, agrees with the binding's struct mirrors, and its
host-side functions (layout size, workspace size, argument checks) behave.
The reference-stream library exports what include/splitzip_ceiling.h
declares.  No device work is launched here."""
import ctypes
import os
import re

import pytest

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
import oracle_pins as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "splitzip.h")


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splitzip_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = S.lib()
    names = declared_functions()
    assert len(names) == 19, names
    for name in names:
        assert hasattr(lib, name), name
        assert name in _abi.SIGNATURES, name
    assert set(_abi.SIGNATURES) == set(names)


def test_reference_stream_symbols_and_argument_errors():
    lib = _abi.ceiling_lib()
    names = declared_functions(os.path.join(ROOT, "include", "splitzip_ceiling.h"))
    assert names == sorted(_abi.CEILING_SIGNATURES), names
    for name in names:
        assert hasattr(lib, name), name
    # sizes that are not whole tiles, null or misaligned pointers: no launch
    assert lib.splitzip_ceiling_read(0, 1 << 20, 0, 0x1000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_read(0x1000, 24, 0, 0x1000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_encode_shape(0x1000, 8191, 0x2000, 0x3000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_encode_shape(0x1008, 8192, 0x2000, 0x3000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_decode_shape(0x1000, 0x2000, 0x3000, 0, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_decode_shape(0x1000, 0, 0x3000, 8192, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_encode_wide(0x1000, 100, 0x2000, 0x3000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_decode_wide(0x1000, 0x2008, 0x3000, 8192, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_encode_fenced(0x1000, 8192, 0, 0x3000, 0) == _abi.ERR_INVALID
    # epoch 0 is not a tag; a misaligned counter array
    assert lib.splitzip_ceiling_encode_arrive(0x1000, 8192, 0x2000, 0x3000, 0x4000, 0x5000,
                                              0x6000, 0, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_encode_arrive(0x1000, 8192, 0x2000, 0x3000, 0x4000, 0x5008,
                                              0x6000, 1, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_atomics(0x1000, 1, 4097, 1, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_atomics(0x1000, 1, 1, (1 << 20) + 1, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_launch(1, 0, 0x1000, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_launch(0, 1, 0x1002, 0) == _abi.ERR_INVALID
    # order probe: run not a power of two, decode without an output, encode without an input
    assert lib.splitzip_ceiling_order(0, 3, 0x1000, 0x2000, 0x3000, 0, 8192, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_order(1, 64, 0, 0x2000, 0x3000, 0, 8192, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_order(0, 64, 0, 0x2000, 0x3000, 0x4000, 8192, 0) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_order(2, 0, 0x1000, 0x2000, 0x3000, 0x4000, 8192, 0) == _abi.ERR_INVALID


def test_struct_layout_matches_header():
    cb, meta = ctypes.c_size_t(), ctypes.c_size_t()
    S.lib().splitzip_struct_sizes(ctypes.byref(cb), ctypes.byref(meta))
    assert cb.value == ctypes.sizeof(_abi.Codebook) == 2856
    assert meta.value == ctypes.sizeof(_abi.Meta) == 104
    assert _abi.Codebook.dec_lut.offset == 512
    assert _abi.Meta.status.offset == 96
    assert ctypes.sizeof(_abi.SlotItem) == 56 and ctypes.sizeof(_abi.Item) == 56
    assert S.lib().splitzip_abi_version() == 2
    assert _abi.Meta.flags.offset == 100


def test_payload_size_matches_golden_layout():
    path = os.path.join(P.GOLDEN, "layout_sizes.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for row in rows:
        n, e, total = int(row[0]), int(row[1]), int(row[7])
        assert S.payload_size(n, e) == total


def test_workspace_size_monotonic():
    prev = 0
    for n in [0, 1, 4095, 4096, 4097, 1 << 20, 33554432, 37748736]:
        w = _abi.splitzip_workspace_size(n)
        assert w >= prev
        prev = w
        # a count per 8192-element tile and at most 512 staged escapes per
        # tile: bounded by half a byte per element beyond the fixed part
        assert w <= _abi.splitzip_workspace_size(0) + n // 2 + 4096
        assert w >= n // 4


def test_argument_errors_need_no_device():
    assert _abi.splitzip_workspace_init(0, 1 << 20, 0) == _abi.ERR_INVALID
    assert _abi.splitzip_calibrate(0, 5, 0, 0, 0, 0) == _abi.ERR_INVALID
    assert _abi.splitzip_encode(0, 5, 0, 0, 0, 0, 0, 0, 0) == _abi.ERR_INVALID
    assert _abi.splitzip_decode(0, 0, 0, 0, 0, 5, 0, 0) == _abi.ERR_INVALID
    # in-place decode: slot below 2n bytes, stash missing, slot and stash overlapping
    assert _abi.splitzip_decode_slot(0x10000, 9, 0x2000, 0x3000, 5, 0x40000, 1 << 10, 0, 0) == \
        _abi.ERR_INVALID
    assert _abi.splitzip_decode_slot(0x10000, 1 << 10, 0x2000, 0x3000, 5, 0, 1 << 10, 0, 0) == \
        _abi.ERR_INVALID
    assert _abi.splitzip_decode_slot(0x10000, 1 << 10, 0x2000, 0x3000, 5, 0x10200, 1 << 10, 0,
                                     0) == _abi.ERR_INVALID
    assert _abi.splitzip_decode_slot(0x10000, 1 << 10, 0x2000, 0x3000, 5, 0x40000, 4, 0, 0) == \
        _abi.ERR_INVALID
    # a batch with one bad item enqueues nothing
    items = (_abi.SlotItem * 2)()
    items[0].slot, items[0].slot_bytes, items[0].meta, items[0].dec_lut = 0x10000, 1 << 10, 0x2000, 0x3000
    items[0].n, items[0].stash, items[0].stash_bytes = 5, 0x40000, 1 << 10
    items[1] = items[0]
    items[1].stash = 0x10100                      # overlaps its slot
    for fn in (_abi.splitzip_decode_slot_batch, _abi.splitzip_decode_slot_batch_resident):
        assert fn(items, 2, 0, 0) == _abi.ERR_INVALID
        assert fn(None, 1, 0, 0) == _abi.ERR_INVALID
    # chunk sizes the wire format cannot carry
    for chunk, n in ((0, 5), (65537, 5), (1, (1 << 31) + 1)):
        assert _abi.splitzip_encode_chunked(0x1000, n, 0x2000, chunk, 0x4000, 1 << 40, 0x3000,
                                            0x5000, 1 << 40, 0) == _abi.ERR_INVALID
    # misaligned tensor pointer
    assert _abi.splitzip_calibrate(0x1002, 5, 0x2000, 0x3000, 1 << 20, 0) == _abi.ERR_INVALID
    # n above the limit
    assert _abi.splitzip_calibrate(0x1000, _abi.MAX_N + 1, 0x2000, 0x3000, 1 << 20, 0) == \
        _abi.ERR_INVALID
    for code in range(7):
        assert _abi.status_string(code)
    assert _abi.status_string(99) == "unknown status"


def test_binding_rejects_non_bf16():
    import torch
    with pytest.raises(ValueError):
        S.codec._bits(torch.zeros(4, dtype=torch.float16))


def test_batch_host_checks_need_no_device():
    assert _abi.splitzip_calibrate_batch(None, 3, 0x1000, 1 << 20, 0) == _abi.ERR_INVALID
    assert _abi.splitzip_encode_batch(None, 3, 0x1000, 1 << 20, 0) == _abi.ERR_INVALID
    assert _abi.splitzip_decode_batch(None, 3, 0, 0) == _abi.ERR_INVALID
    items = (_abi.Item * 2)()
    items[0].x, items[0].n, items[0].cb = 0x1002, 10, 0x2000      # misaligned tensor
    assert _abi.splitzip_calibrate_batch(items, 2, 0x1000, 1 << 20, 0) == _abi.ERR_INVALID
    ns = [5, 8192 * 3, 0, 1 << 20]
    w = _abi.splitzip_workspace_size_batch(ns)
    assert w >= max(_abi.splitzip_workspace_size(n) for n in ns)
    assert w >= _abi.splitzip_workspace_size(sum(ns))
    # 40 tensors run as two launches of at most 32: the larger group decides
    many = [1 << 16] * 40
    assert _abi.splitzip_workspace_size_batch(many) == _abi.splitzip_workspace_size(32 << 16)
