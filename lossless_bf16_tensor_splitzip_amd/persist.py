"""Persistence of codebooks and payload metadata, and the coverage gate.

Host-side policy helpers around the C ABI (no codec arithmetic):

* JSON forms with the keys of the page "splitzip_codec.py -- SplitZip codec
  adapter for diffusers-dynamic-offloader" (``SplitZipCodebook.to_json``: the
  coverage and the four tables as base64 of their raw bytes;
  ``PayloadMeta.to_json``: n, n_pairs, chunk_size, n_esc, comp_bytes, offsets,
  coverage).  Our extra exact fields (n_codes, covered, total, counts) ride
  along under their own keys; a reader of the pages' format ignores them.
* The coverage gate of the page "SplitZip in DDO -- VMM routes" ("Build the
  cache"; "Invariants common to both routes", item 3): a tensor whose top-16
  coverage is below 0.99 is left uncompressed: the payload-size estimate no
  longer holds there, and tensors with widely spread exponents can come out
  larger than the raw data.

A payload cannot be decoded without its codebook's dec_lut (same page,
invariant 2): keep the codebook JSON next to every stored payload.
"""
from __future__ import annotations

import base64
import ctypes

from ._abi import META_ASCENDING, Codebook, Meta

COVERAGE_GATE = 0.99

_TABLES = ("enc_lut", "enc_lut_marked", "dec_lut", "common_lut")


def _b64(raw: bytes) -> str:
    return base64.b64encode(raw).decode()


def coverage(cb: Codebook) -> float:
    """Fraction of elements whose exponent has a code (1 for an empty tensor)."""
    return 1.0 if cb.total == 0 else cb.covered / cb.total


def passes_coverage_gate(cb: Codebook, threshold: float = COVERAGE_GATE) -> bool:
    """True when the tensor should be stored compressed."""
    return coverage(cb) >= threshold


def codebook_to_json(cb: Codebook) -> dict:
    d = {"coverage": coverage(cb)}
    for name in _TABLES:
        d[name] = _b64(bytes(getattr(cb, name)))
    d["n_codes"] = int(cb.n_codes)
    d["covered"] = int(cb.covered)
    d["total"] = int(cb.total)
    d["counts"] = [int(c) for c in cb.counts]
    return d


def codebook_from_json(d: dict) -> Codebook:
    """Rebuild a codebook; accepts the pages' four-table form as well (then
    counts are zero, n_codes comes from common_lut and covered/total from the
    coverage only approximately: total is 0)."""
    cb = Codebook()
    sizes = {"enc_lut": 256, "enc_lut_marked": 256, "dec_lut": 16, "common_lut": 256}
    for name in _TABLES:
        raw = base64.b64decode(d[name])
        if len(raw) != sizes[name]:
            raise ValueError("%s must hold %d bytes, got %d" % (name, sizes[name], len(raw)))
        if name == "enc_lut_marked" and max(raw) > 16:
            # page 1, calibrate_codebook: a marked table holds codes 0..15
            # and 16 for an escape; anything else is not such a table
            raise ValueError("enc_lut_marked holds a value above 16")
        ctypes.memmove(ctypes.addressof(getattr(cb, name)), raw, len(raw))
    cb.n_codes = int(d["n_codes"]) if "n_codes" in d else sum(bytes(cb.common_lut))
    cb.covered = int(d.get("covered", 0))
    cb.total = int(d.get("total", 0))
    counts = d.get("counts")
    if counts is not None:
        if len(counts) != 256:
            raise ValueError("counts must have 256 entries")
        for k, c in enumerate(counts):
            cb.counts[k] = int(c)
    return cb


def meta_to_json(m: Meta) -> dict:
    return {
        "n": int(m.n),
        "n_pairs": int(m.n_pairs),
        "chunk_size": int(m.chunk_size),
        "n_esc": int(m.n_esc),
        "comp_bytes": int(m.comp_bytes),
        "offsets": [int(v) for v in m.offsets],
        "coverage": 1.0 if m.total == 0 else m.covered / m.total,
        "covered": int(m.covered),
        "total": int(m.total),
        # this library's flag: the escape stream is in ascending order
        "ascending": bool(m.flags & META_ASCENDING),
    }


def meta_from_json(d: dict) -> Meta:
    m = Meta()
    m.n, m.n_pairs = int(d["n"]), int(d["n_pairs"])
    m.chunk_size, m.n_esc, m.comp_bytes = int(d["chunk_size"]), int(d["n_esc"]), int(d["comp_bytes"])
    offs = [int(v) for v in d["offsets"]]
    if len(offs) != 5:
        raise ValueError("offsets must have 5 entries")
    for k, v in enumerate(offs):
        m.offsets[k] = v
    m.covered = int(d.get("covered", 0))
    m.total = int(d.get("total", 0))
    m.status = 0
    # page-format metadata says nothing about the escape order: left clear,
    # so the decode applies the escapes in any order
    m.flags = META_ASCENDING if d.get("ascending") is True else 0
    return m


def to_device(struct, device) -> "torch.Tensor":  # noqa: F821
    """Copy a Codebook or Meta into a device uint8 tensor for the C ABI."""
    import torch

    raw = bytearray(bytes(struct))
    return torch.frombuffer(raw, dtype=torch.uint8).to(device)


def manifest_entry(name: str, shape, cb: Codebook | None, m: Meta | None) -> dict:
    """Manifest record of one stored tensor: the codebook travels with the
    blob (a blob without its dec_lut cannot be decoded).  ``cb``/``m`` None
    marks a tensor stored raw (it failed the coverage gate)."""
    d = {"name": name, "dtype": "bfloat16", "shape": [int(v) for v in shape]}
    if cb is None:
        d["raw"] = True
        return d
    d["raw"] = False
    d["codebook"] = codebook_to_json(cb)
    d["meta"] = meta_to_json(m)
    return d


def pack(name: str, x, ws, threshold: float = COVERAGE_GATE):
    """Gate, encode and verify one device bfloat16 tensor for storage.

    Returns (manifest entry, blob) where blob is a device uint8 tensor of
    exactly comp_bytes bytes, or a copy of the raw bytes when the tensor fails
    the coverage gate.  The round trip is checked bit for bit on the device
    before the blob is handed out (page "SplitZip in DDO -- VMM routes",
    "Invariants common to both routes", item 4)."""
    import torch

    from . import codec

    cb_dev = codec.calibrate(x, ws)
    cb = codec.read_codebook(cb_dev)
    flat = x.reshape(-1)
    if not passes_coverage_gate(cb, threshold):
        return manifest_entry(name, x.shape, None, None), flat.view(torch.uint8).clone()
    payload, meta_dev = codec.encode(x, cb_dev, ws)
    m = codec.read_meta(meta_dev)
    if m.status != 0:
        raise RuntimeError("encode of %s failed with status %d" % (name, m.status))
    status = torch.zeros(1, dtype=torch.int32, device=x.device)
    back = codec.decode(payload, meta_dev, cb_dev, flat.numel(), status=status)
    if int(status.item()) != 0 or not torch.equal(back.view(torch.int16), flat.view(torch.int16)):
        raise RuntimeError("round trip of %s is not bit-exact" % name)
    return manifest_entry(name, x.shape, cb, m), payload[: m.comp_bytes].clone()


def unpack(entry: dict, blob, out=None, stream=None):
    """Rebuild the bfloat16 tensor of a manifest entry from its device blob."""
    import torch

    from . import codec

    shape = tuple(entry["shape"])
    n = 1
    for v in shape:
        n *= v
    if entry.get("raw"):
        t = blob.view(torch.bfloat16)[:n]
        return t.reshape(shape) if out is None else out.copy_(t.reshape(out.shape))
    cb = codebook_from_json(entry["codebook"])
    m = meta_from_json(entry["meta"])
    if m.n != n:
        raise ValueError("manifest shape and metadata disagree")
    if out is not None and not out.is_contiguous():
        # a reshape of a strided tensor would be a copy, and the decode would
        # land there instead of in `out`
        raise ValueError("out must be a contiguous tensor")
    flat = None if out is None else out.reshape(-1)
    # The validating decode: metadata from storage may describe an escape
    # stream this library did not write (any order, or damaged bytes).
    status = torch.zeros(1, dtype=torch.int32, device=blob.device)
    res = codec.decode(blob, to_device(m, blob.device), to_device(cb, blob.device), n, out=flat,
                       status=status, stream=stream)
    bad = int(status.item())
    if bad:
        raise ValueError("stored payload of %s is corrupt (decode status %d)"
                         % (entry.get("name", "?"), bad))
    return res.reshape(shape) if out is None else out
