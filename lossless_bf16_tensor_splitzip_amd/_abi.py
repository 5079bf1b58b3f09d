"""ctypes binding of the C ABI in include/splitzip.h.

Argument marshalling only: every step of calibrate / encode / decode runs in
the HIP kernels of ``_lib/libsplitzip.so``.  The library must have been built
(``python -m lossless_bf16_tensor_splitzip_amd._build`` or
``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

from ._build import CEILING_LIB_PATH, LIB_PATH

CHUNK = 1024
MAX_N = 1 << 36
NOALLOC_MAX_N = 133627904        # splitzip_encode_noalloc's limit

OK = 0
ERR_INVALID = 1
ERR_CAPACITY = 2
ERR_CORRUPT = 3
ERR_HIP = 4
ERR_WORKSPACE = 5
ERR_INTERNAL = 6

# splitzip_meta.flags
META_ASCENDING = 1

# decode status bits
DEC_BAD_META = 1
DEC_ESC_OUT_OF_RANGE = 2
DEC_POS_GE_CHUNK = 4
DEC_NOT_INCREASING = 8


class Codebook(ctypes.Structure):
    """Mirror of splitzip_codebook."""
    _fields_ = [
        ("enc_lut", ctypes.c_uint8 * 256),
        ("enc_lut_marked", ctypes.c_uint8 * 256),
        ("dec_lut", ctypes.c_uint8 * 16),
        ("common_lut", ctypes.c_uint8 * 256),
        ("n_codes", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("covered", ctypes.c_uint64),
        ("total", ctypes.c_uint64),
        ("counts", ctypes.c_uint64 * 256),
    ]


class Meta(ctypes.Structure):
    """Mirror of splitzip_meta."""
    _fields_ = [
        ("n", ctypes.c_uint64),
        ("n_pairs", ctypes.c_uint64),
        ("chunk_size", ctypes.c_uint64),
        ("n_esc", ctypes.c_uint64),
        ("comp_bytes", ctypes.c_uint64),
        ("offsets", ctypes.c_uint64 * 5),
        ("covered", ctypes.c_uint64),
        ("total", ctypes.c_uint64),
        ("status", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]


class Item(ctypes.Structure):
    """Mirror of splitzip_item (one tensor of a batched call; device pointers)."""
    _fields_ = [
        ("x", ctypes.c_void_p),
        ("n", ctypes.c_uint64),
        ("cb", ctypes.c_void_p),
        ("payload", ctypes.c_void_p),
        ("capacity", ctypes.c_uint64),
        ("meta", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
    ]


class SlotItem(ctypes.Structure):
    """Mirror of splitzip_slot_item (one payload of a batched in-place decode)."""
    _fields_ = [
        ("slot", ctypes.c_void_p),
        ("slot_bytes", ctypes.c_uint64),
        ("meta", ctypes.c_void_p),
        ("dec_lut", ctypes.c_void_p),
        ("n", ctypes.c_uint64),
        ("stash", ctypes.c_void_p),
        ("stash_bytes", ctypes.c_uint64),
    ]


DEC_LUT_OFFSET = Codebook.dec_lut.offset

# name -> (restype, argtypes), exactly the functions of include/splitzip.h
_P = ctypes.c_void_p
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t
SIGNATURES = {
    "splitzip_abi_version": (ctypes.c_int, []),
    "splitzip_struct_sizes": (None, [ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "splitzip_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "splitzip_payload_size": (_U64, [_U64, _U64]),
    "splitzip_slot_schedule": (ctypes.c_uint32, [_U64, ctypes.c_uint32, ctypes.POINTER(_U64),
                                                ctypes.POINTER(_U64), ctypes.POINTER(_U64)]),
    "splitzip_workspace_size": (_SZ, [_U64]),
    "splitzip_workspace_init": (ctypes.c_int, [_P, _SZ, _P]),
    "splitzip_calibrate": (ctypes.c_int, [_P, _U64, _P, _P, _SZ, _P]),
    "splitzip_encode": (ctypes.c_int, [_P, _U64, _P, _P, _U64, _P, _P, _SZ, _P]),
    "splitzip_encode_chunked": (ctypes.c_int, [_P, _U64, _P, ctypes.c_uint32, _P, _U64, _P, _P, _SZ,
                                               _P]),
    "splitzip_encode_noalloc": (ctypes.c_int, [_P, _U64, _P, _P, _U64, _P, _P]),
    "splitzip_decode": (ctypes.c_int, [_P, _U64, _P, _P, _P, _U64, _P, _P]),
    "splitzip_decode_slot": (ctypes.c_int, [_P, _U64, _P, _P, _U64, _P, _U64, _P, _P]),
    "splitzip_decode_slot_batch": (ctypes.c_int, [_P, ctypes.c_uint32, _P, _P]),
    "splitzip_decode_slot_batch_resident": (ctypes.c_int, [_P, ctypes.c_uint32, _P, _P]),
    "splitzip_workspace_size_batch": (_SZ, [ctypes.POINTER(ctypes.c_uint64), ctypes.c_uint32]),
    "splitzip_calibrate_batch": (ctypes.c_int, [_P, ctypes.c_uint32, _P, _SZ, _P]),
    "splitzip_encode_batch": (ctypes.c_int, [_P, ctypes.c_uint32, _P, _SZ, _P]),
    "splitzip_decode_batch": (ctypes.c_int, [_P, ctypes.c_uint32, _P, _P]),
}

_lib = None


CEILING_SIGNATURES = {
    "splitzip_ceiling_read": (ctypes.c_int, [_P, ctypes.c_uint64, ctypes.c_uint32, _P, _P]),
    "splitzip_ceiling_encode_shape": (ctypes.c_int, [_P, ctypes.c_uint64, _P, _P, _P]),
    "splitzip_ceiling_decode_shape": (ctypes.c_int, [_P, _P, _P, ctypes.c_uint64, _P]),
    "splitzip_ceiling_order": (ctypes.c_int, [ctypes.c_uint32, ctypes.c_uint32, _P, _P, _P, _P,
                                              ctypes.c_uint64, _P]),
    "splitzip_ceiling_encode_wide": (ctypes.c_int, [_P, ctypes.c_uint64, _P, _P, _P]),
    "splitzip_ceiling_decode_wide": (ctypes.c_int, [_P, _P, _P, ctypes.c_uint64, _P]),
    "splitzip_ceiling_encode_arrive": (ctypes.c_int, [_P, ctypes.c_uint64, _P, _P, _P, _P, _P,
                                                      ctypes.c_uint32, _P]),
    "splitzip_ceiling_encode_fenced": (ctypes.c_int, [_P, ctypes.c_uint64, _P, _P, _P]),
    "splitzip_ceiling_atomics": (ctypes.c_int, [_P, ctypes.c_uint32, ctypes.c_uint32,
                                                ctypes.c_uint32, _P]),
    "splitzip_ceiling_launch": (ctypes.c_int, [ctypes.c_uint32, ctypes.c_uint32, _P, _P]),
}

_ceiling = None


def ceiling_lib():
    """Load the reference-stream library (measurement only; raises if it has
    not been built)."""
    global _ceiling
    if _ceiling is not None:
        return _ceiling
    if not os.path.exists(CEILING_LIB_PATH):
        raise RuntimeError("reference-stream library not built (%s missing)" % CEILING_LIB_PATH)
    handle = ctypes.CDLL(CEILING_LIB_PATH)
    for name, (res, args) in CEILING_SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    _ceiling = handle
    return handle


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "SplitZip HIP library not built (%s missing): run "
            "`python -m lossless_bf16_tensor_splitzip_amd._build`" % LIB_PATH)
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    cb_size, meta_size = ctypes.c_size_t(), ctypes.c_size_t()
    handle.splitzip_struct_sizes(ctypes.byref(cb_size), ctypes.byref(meta_size))
    if cb_size.value != ctypes.sizeof(Codebook) or meta_size.value != ctypes.sizeof(Meta):
        raise RuntimeError("struct layout mismatch between the library and the binding")
    _lib = handle
    return handle


class SplitZipError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, status_string(status), status))


def status_string(status: int) -> str:
    return lib().splitzip_status_string(status).decode()


def _check(fn: str, status: int) -> int:
    if status != OK:
        raise SplitZipError(fn, status)
    return status


# Thin wrappers with the C names (raw pointers / ints in, status out).

def splitzip_abi_version() -> int:
    return lib().splitzip_abi_version()


def splitzip_payload_size(n: int, n_esc: int) -> int:
    return lib().splitzip_payload_size(n, n_esc)


def splitzip_slot_schedule(n: int, passes: int):
    """(passes used, t_min, lo, hi) of the in-place decode's pass schedule;
    lo and hi are lists of passes + 1 entries.  None for invalid arguments."""
    t_min = ctypes.c_uint64()
    lo = (ctypes.c_uint64 * (passes + 1))()
    hi = (ctypes.c_uint64 * (passes + 1))()
    used = lib().splitzip_slot_schedule(n, passes, ctypes.byref(t_min), lo, hi)
    if used == 0:
        return None
    return used, t_min.value, list(lo), list(hi)


def splitzip_workspace_size(n: int) -> int:
    return lib().splitzip_workspace_size(n)


def splitzip_workspace_init(d_ws: int, ws_bytes: int, stream: int) -> int:
    return lib().splitzip_workspace_init(d_ws, ws_bytes, stream)


def splitzip_calibrate(d_x: int, n: int, d_cb: int, d_ws: int, ws_bytes: int, stream: int) -> int:
    return lib().splitzip_calibrate(d_x, n, d_cb, d_ws, ws_bytes, stream)


def splitzip_encode(d_x: int, n: int, d_cb: int, d_payload: int, capacity: int, d_meta: int,
                    d_ws: int, ws_bytes: int, stream: int) -> int:
    return lib().splitzip_encode(d_x, n, d_cb, d_payload, capacity, d_meta, d_ws, ws_bytes, stream)


def splitzip_encode_chunked(d_x: int, n: int, d_cb: int, chunk_size: int, d_payload: int,
                            capacity: int, d_meta: int, d_ws: int, ws_bytes: int,
                            stream: int) -> int:
    return lib().splitzip_encode_chunked(d_x, n, d_cb, chunk_size, d_payload, capacity, d_meta,
                                         d_ws, ws_bytes, stream)


def splitzip_encode_noalloc(d_x: int, n: int, d_cb: int, d_payload: int, capacity: int,
                            d_meta: int, stream: int) -> int:
    return lib().splitzip_encode_noalloc(d_x, n, d_cb, d_payload, capacity, d_meta, stream)


def splitzip_decode(d_payload: int, payload_bytes: int, d_meta: int, d_dec_lut: int, d_out: int,
                    n: int, d_status: int, stream: int) -> int:
    return lib().splitzip_decode(d_payload, payload_bytes, d_meta, d_dec_lut, d_out, n, d_status,
                                 stream)


def splitzip_decode_slot(d_slot: int, slot_bytes: int, d_meta: int, d_dec_lut: int, n: int,
                         d_stash: int, stash_bytes: int, d_status: int, stream: int) -> int:
    return lib().splitzip_decode_slot(d_slot, slot_bytes, d_meta, d_dec_lut, n, d_stash,
                                      stash_bytes, d_status, stream)


def splitzip_decode_slot_batch(items, count: int, d_status: int, stream: int) -> int:
    return lib().splitzip_decode_slot_batch(_items_ptr(items), count, d_status, stream)


def splitzip_decode_slot_batch_resident(items, count: int, d_status: int, stream: int) -> int:
    return lib().splitzip_decode_slot_batch_resident(_items_ptr(items), count, d_status, stream)


def splitzip_workspace_size_batch(ns) -> int:
    arr = (ctypes.c_uint64 * max(len(ns), 1))(*ns)
    return lib().splitzip_workspace_size_batch(arr, len(ns))


def _items_ptr(items):
    return ctypes.cast(items, ctypes.c_void_p) if items is not None else None


def splitzip_calibrate_batch(items, count: int, d_ws: int, ws_bytes: int, stream: int) -> int:
    return lib().splitzip_calibrate_batch(_items_ptr(items), count, d_ws, ws_bytes, stream)


def splitzip_encode_batch(items, count: int, d_ws: int, ws_bytes: int, stream: int) -> int:
    return lib().splitzip_encode_batch(_items_ptr(items), count, d_ws, ws_bytes, stream)


def splitzip_decode_batch(items, count: int, d_status: int, stream: int) -> int:
    return lib().splitzip_decode_batch(_items_ptr(items), count, d_status, stream)
