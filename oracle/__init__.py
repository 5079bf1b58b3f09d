"""CPU oracle of the SplitZip lossless BF16 codec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and this package imports
nothing from the product.

The arithmetic lives in ``splitzip_oracle.c`` (plain single-threaded C, built
with gcc); this module only compiles it and marshals numpy arrays through
ctypes.  Every function follows the page "splitzip_codec.py -- SplitZip codec
adapter for diffusers-dynamic-offloader" (functions calibrate_codebook,
assemble_payload, encode_torch, decode_torch) and the wire-format invariant of
the page "SplitZip in DDO -- VMM routes" (section "Invariants common to both
routes", item 1).  Pins: ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "splitzip_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "libsplitzip_oracle.so")

OK, EINVAL, ECAPACITY, ECORRUPT, ENOMEM = 0, 1, 2, 3, 4
CHUNK = 1024


def build() -> str:
    """Compile the oracle with gcc (strict IEEE, no fast-math; integer code)."""
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-fPIC", "-shared",
           _SRC, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_u16(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x))
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise ValueError("oracle expects the 16-bit patterns of a BF16 tensor (uint16)")
    return a.reshape(-1)


@dataclass
class Codebook:
    """Top-16 exponent codebook of one tensor (page 1, SplitZipCodebook)."""
    counts: np.ndarray          # (256,) uint64 exponent histogram
    enc_lut: np.ndarray         # (256,) uint8 value -> code (0 if none)
    enc_lut_marked: np.ndarray  # (256,) uint8 value -> code, 16 = escape
    dec_lut: np.ndarray         # (16,) uint8 code -> value
    common_lut: np.ndarray      # (256,) uint8, 1 if value has a code
    n_codes: int
    covered: int
    total: int

    @property
    def coverage(self) -> float:
        # an empty tensor counts as fully covered
        return 1.0 if self.total == 0 else self.covered / self.total


@dataclass
class Meta:
    """Payload metadata (page 1, PayloadMeta)."""
    n: int
    n_pairs: int
    chunk_size: int
    n_esc: int
    comp_bytes: int
    offsets: tuple


class OracleLib:
    """ctypes view of one build of ``splitzip_oracle.c``.  The default build is
    ``oracle/_build/libsplitzip_oracle.so``; the mutation tests load
    deliberately broken copies through the same class."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = _LIB_PATH
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        u64 = ctypes.c_uint64
        lib.orc_histogram.argtypes = [u16p, u64, u64p]
        lib.orc_histogram.restype = None
        lib.orc_select.argtypes = [u64p, u8p, u8p, u8p, u8p, u32p, u64p]
        lib.orc_select.restype = None
        lib.orc_layout.argtypes = [u64, u64, u64p, u64p]
        lib.orc_layout.restype = None
        lib.orc_encode.argtypes = [u16p, u64, u8p, ctypes.c_uint32, u8p, u64, u64p, u64p,
                                   u64p]
        lib.orc_encode.restype = ctypes.c_int
        lib.orc_decode.argtypes = [u8p, u64, u64, u64, ctypes.c_uint32, u64p, u8p, u16p,
                                   ctypes.c_int]
        lib.orc_decode.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def histogram(self, x) -> np.ndarray:
        a = _as_u16(x)
        cnt = np.zeros(256, dtype=np.uint64)
        self.lib.orc_histogram(_ptr(a, ctypes.c_uint16), a.size, _ptr(cnt, ctypes.c_uint64))
        return cnt

    def select(self, counts) -> Codebook:
        cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.uint64))
        if cnt.shape != (256,):
            raise ValueError("counts must have 256 bins")
        enc = np.empty(256, np.uint8)
        marked = np.empty(256, np.uint8)
        dec = np.empty(16, np.uint8)
        common = np.empty(256, np.uint8)
        n_codes = ctypes.c_uint32()
        covered = ctypes.c_uint64()
        self.lib.orc_select(_ptr(cnt, ctypes.c_uint64), _ptr(enc, ctypes.c_uint8),
                            _ptr(marked, ctypes.c_uint8), _ptr(dec, ctypes.c_uint8),
                            _ptr(common, ctypes.c_uint8), ctypes.byref(n_codes),
                            ctypes.byref(covered))
        return Codebook(cnt.copy(), enc, marked, dec, common, int(n_codes.value),
                        int(covered.value), int(cnt.sum()))

    def calibrate(self, x) -> Codebook:
        """Page 1, calibrate_codebook (tie-break: count desc, exponent asc)."""
        return self.select(self.histogram(x))

    def layout(self, n: int, n_esc: int) -> tuple[tuple, int]:
        off = np.zeros(5, np.uint64)
        total = ctypes.c_uint64()
        self.lib.orc_layout(n, n_esc, _ptr(off, ctypes.c_uint64), ctypes.byref(total))
        return tuple(int(v) for v in off), int(total.value)

    def encode(self, x, codebook: Codebook, chunk_size: int = CHUNK) -> tuple[bytes, Meta]:
        """Page 1, encode_torch + assemble_payload.  Returns (payload, meta)."""
        a = _as_u16(x)
        n = a.size
        # worst case (every element escapes) plus slack for a broken layout rule
        cap = 9 * n + 64
        buf = np.zeros(cap, np.uint8)
        marked = np.ascontiguousarray(codebook.enc_lut_marked, dtype=np.uint8)
        n_esc = ctypes.c_uint64()
        off = np.zeros(5, np.uint64)
        total = ctypes.c_uint64()
        rc = self.lib.orc_encode(_ptr(a, ctypes.c_uint16), n, _ptr(marked, ctypes.c_uint8),
                                 chunk_size, _ptr(buf, ctypes.c_uint8), buf.size,
                                 ctypes.byref(n_esc), _ptr(off, ctypes.c_uint64),
                                 ctypes.byref(total))
        if rc != OK:
            raise RuntimeError("oracle encode failed with status %d" % rc)
        meta = Meta(n=n, n_pairs=(n + 1) // 2, chunk_size=chunk_size,
                    n_esc=int(n_esc.value), comp_bytes=int(total.value),
                    offsets=tuple(int(v) for v in off))
        return bytes(buf[: meta.comp_bytes]), meta

    def decode_status(self, payload, meta: Meta, dec_lut, validate: bool = True):
        """Page 1, decode_torch.  Returns (status, uint16 bit patterns)."""
        buf = np.frombuffer(bytes(payload), dtype=np.uint8).copy()
        blen = buf.size
        if blen == 0:
            buf = np.zeros(1, np.uint8)
        dec = np.ascontiguousarray(np.asarray(dec_lut, dtype=np.uint8))
        off = np.asarray(meta.offsets, dtype=np.uint64)
        out = np.zeros(max(meta.n, 1), np.uint16)
        rc = self.lib.orc_decode(_ptr(buf, ctypes.c_uint8), blen, meta.n, meta.n_esc,
                                 meta.chunk_size, _ptr(off, ctypes.c_uint64),
                                 _ptr(dec, ctypes.c_uint8), _ptr(out, ctypes.c_uint16),
                                 1 if validate else 0)
        return rc, out[: meta.n]

    def decode(self, payload, meta: Meta, dec_lut, validate: bool = True) -> np.ndarray:
        """Page 1, decode_torch; raises ValueError on a corrupt payload."""
        rc, out = self.decode_status(payload, meta, dec_lut, validate)
        if rc != OK:
            raise ValueError("oracle decode rejected the payload (status %d)" % rc)
        return out


_default: OracleLib | None = None


def default() -> OracleLib:
    global _default
    if _default is None:
        _default = OracleLib()
    return _default


def histogram(x):
    return default().histogram(x)


def select(counts):
    return default().select(counts)


def calibrate(x):
    return default().calibrate(x)


def layout(n, n_esc):
    return default().layout(n, n_esc)


def encode(x, codebook, chunk_size=CHUNK):
    return default().encode(x, codebook, chunk_size)


def decode(payload, meta, dec_lut, validate=True):
    return default().decode(payload, meta, dec_lut, validate)


def decode_status(payload, meta, dec_lut, validate=True):
    return default().decode_status(payload, meta, dec_lut, validate)
