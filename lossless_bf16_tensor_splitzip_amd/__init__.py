"""SplitZip lossless BF16 codec for MI355X (gfx950).

Hand-written HIP kernels behind the C ABI of include/splitzip.h
(``_lib/libsplitzip.so``); this package is the thin Python binding:

* ``_abi``   -- ctypes view of the C functions (same names) and structs;
* ``codec``  -- torch-tensor marshalling: Workspace, calibrate, encode, decode;
* ``persist`` -- codebook / metadata JSON and the 0.99 coverage gate.

The method: page "splitzip_codec.py -- SplitZip codec adapter for
diffusers-dynamic-offloader" and page "SplitZip in DDO -- VMM routes".
"""
from ._abi import CHUNK, Codebook, Meta, SplitZipError, lib  # noqa: F401
from . import persist  # noqa: F401
from .codec import (Batch, Workspace, calibrate, decode, decode_slot, decode_slots,  # noqa: F401
                    encode, payload_for, payload_size, read_codebook, read_meta)

__all__ = ["CHUNK", "Batch", "Codebook", "Meta", "SplitZipError", "Workspace", "calibrate", "encode",
           "decode", "decode_slot", "decode_slots", "payload_for", "payload_size", "read_codebook", "read_meta",
           "lib", "persist"]
