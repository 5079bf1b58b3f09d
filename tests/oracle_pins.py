"""Pins of the CPU oracle: checks against what the pages and plain mathematics
fix, never against the oracle itself.

Each ``pin_*`` function takes an ``oracle.OracleLib`` and raises
AssertionError on a mismatch, so the same checks run on the real oracle
(tests/test_oracle_pins.py) and on deliberately broken copies of it
(tests/test_oracle_mutants.py), where at least one of them must fail.

What pins what:
  * hand-derived golden payloads (tests/golden/worked_examples.json): nibble
    order, tie-break, escape order, endianness, section placement, padding;
  * hand-derived layout table (tests/golden/layout_sizes.txt) and the closed
    form total = P + n + 7e + (-P mod 4) + (-n mod 4) + 2 (e mod 2);
  * the exhaustive 65,536-pattern input (every exponent occurs 256 times);
  * an independent rank characterisation of the top-16 select;
  * brute force over a 14-pattern alphabet of special values;
  * losslessness: decode(encode(x)) == x bit for bit.
"""
from __future__ import annotations

import itertools
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# 14 bit patterns: +-0, +-min subnormal, +-max subnormal, +-1.0, +-max finite,
# +-inf and two NaNs.  Their exponent bytes are 0, 127, 254 and 255.
ALPHABET = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x807F, 0x3F80, 0xBF80,
                     0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC1, 0xFF81], dtype=np.uint16)


def _u16(vals) -> np.ndarray:
    return np.array([int(v, 16) if isinstance(v, str) else int(v) for v in vals], dtype=np.uint16)


def closed_form_total(n: int, e: int) -> int:
    p = (n + 1) // 2
    return p + n + 7 * e + ((-p) % 4) + ((-n) % 4) + 2 * (e % 2)


def rank_codes(counts) -> dict:
    """Independent characterisation of the select: exponent v gets code
    rank(v) = #{u : c[u] > c[v] or (c[u] == c[v] and u < v)} when it occurs and
    that rank is below 16; every other exponent escapes."""
    c = [int(v) for v in counts]
    codes = {}
    for v in range(256):
        if c[v] == 0:
            continue
        rank = sum(1 for u in range(256) if c[u] > c[v] or (c[u] == c[v] and u < v))
        if rank < 16:
            codes[v] = rank
    return codes


def exponents(x: np.ndarray) -> np.ndarray:
    # bits 7..14 of the 16-bit pattern (page 1, docstring "Method")
    return ((x.astype(np.uint32) >> 7) & 0xFF).astype(np.int64)


def load_examples():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["examples"]


def example_input(ex) -> np.ndarray:
    if "x" in ex:
        return _u16(ex["x"])
    x = np.full(ex["n"], int(ex["x_base"], 16), dtype=np.uint16)
    for k, v in ex["x_overrides"].items():
        x[int(k)] = int(v, 16)
    return x


def example_payload(ex) -> bytes:
    if "expect_payload_hex" in ex:
        return bytes.fromhex(ex["expect_payload_hex"])
    buf = bytearray(ex["expect_meta"]["comp_bytes"])
    for k, v in ex["expect_payload_sparse"].items():
        buf[int(k)] = int(v, 16)
    return bytes(buf)


def _check_codebook(cb, want):
    k = len(want["dec_lut_prefix"])
    assert list(cb.dec_lut[:k]) == want["dec_lut_prefix"], (list(cb.dec_lut), want)
    assert all(int(v) == 0 for v in cb.dec_lut[k:]), list(cb.dec_lut)
    assert cb.n_codes == want["n_codes"], (cb.n_codes, want)
    assert cb.covered == want["covered"], (cb.covered, want)
    if "counts" in want:
        expect = np.zeros(256, np.uint64)
        for kk, vv in want["counts"].items():
            expect[int(kk)] = vv
        assert np.array_equal(cb.counts, expect)


def pin_worked_examples(o):
    for ex in load_examples():
        x = example_input(ex)
        if ex["codebook_from"] == "self":
            cb = o.calibrate(x)
            _check_codebook(cb, ex["expect_codebook"])
        else:
            cb = o.calibrate(_u16(ex["codebook_from"]["x"]))
            _check_codebook(cb, ex["expect_codebook_of_source"])
        payload, meta = o.encode(x, cb)
        want_meta = ex["expect_meta"]
        assert meta.n == want_meta["n"] and meta.n_pairs == want_meta["n_pairs"], ex["name"]
        assert meta.n_esc == want_meta["n_esc"], (ex["name"], meta)
        assert list(meta.offsets) == want_meta["offsets"], (ex["name"], meta)
        assert meta.comp_bytes == want_meta["comp_bytes"], (ex["name"], meta)
        want = example_payload(ex)
        assert payload == want, (ex["name"], payload.hex(), want.hex())
        out = o.decode(want, meta, cb.dec_lut)
        assert np.array_equal(out, x), ex["name"]


def pin_layout_table(o):
    with open(os.path.join(GOLDEN, "layout_sizes.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert rows
    for row in rows:
        n, e, *rest = (int(v) for v in row)
        off, total = o.layout(n, e)
        assert list(off) == rest[:5] and total == rest[5], (n, e, off, total, rest)
        assert total == closed_form_total(n, e)


def pin_layout_closed_form(o, seed: int = 1, trials: int = 2000):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        n = int(rng.integers(0, 1 << 40))
        e = int(rng.integers(0, n + 1))
        off, total = o.layout(n, e)
        assert total == closed_form_total(n, e), (n, e, total)
        p = (n + 1) // 2
        # sections in order, non-overlapping, 4-aligned where a wide view is taken
        assert off[0] == 0 and off[1] >= p and off[2] >= off[1] + n
        assert off[3] == off[2] + 4 * e and off[4] >= off[3] + 2 * e
        assert off[1] % 4 == 0 and off[2] % 4 == 0 and off[4] % 4 == 0
        assert off[1] - p < 4 and off[2] - off[1] - n < 4 and off[4] - off[3] - 2 * e < 4


def pin_exhaustive_patterns(o):
    x = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    cb = o.calibrate(x)
    assert np.all(cb.counts == 256)
    # all 256 counts tie: codes go to exponents 0..15 in order
    assert list(cb.dec_lut) == list(range(16))
    assert cb.n_codes == 16 and cb.covered == 16 * 256
    for v in range(256):
        assert cb.enc_lut_marked[v] == (v if v < 16 else 16)
        assert cb.enc_lut[v] == (v if v < 16 else 0)
        assert cb.common_lut[v] == (1 if v < 16 else 0)
    payload, meta = o.encode(x, cb)
    assert meta.n_esc == 65536 - 4096 and meta.comp_bytes == 528384
    assert np.array_equal(o.decode(payload, meta, cb.dec_lut), x)


def pin_select_rank(o, seed: int = 2, trials: int = 300):
    rng = np.random.default_rng(seed)
    cases = [np.zeros(256, np.uint64)]
    one = np.zeros(256, np.uint64)
    one[200] = 7
    cases.append(one)
    for t in range(trials):
        c = np.zeros(256, np.uint64)
        k = int(rng.integers(1, 257))
        bins = rng.choice(256, size=k, replace=False)
        hi = int(rng.choice([2, 3, 5, 1000, 1 << 40]))
        c[bins] = rng.integers(1, hi, size=k, dtype=np.uint64)
        cases.append(c)
    for c in cases:
        cb = o.select(c)
        codes = rank_codes(c)
        assert cb.n_codes == len(codes), (cb.n_codes, len(codes))
        assert cb.covered == sum(int(c[v]) for v in codes)
        for v in range(256):
            if v in codes:
                assert cb.enc_lut[v] == codes[v] and cb.enc_lut_marked[v] == codes[v]
                assert cb.common_lut[v] == 1 and cb.dec_lut[codes[v]] == v
            else:
                assert cb.enc_lut[v] == 0 and cb.enc_lut_marked[v] == 16
                assert cb.common_lut[v] == 0
        for code in range(len(codes), 16):
            assert cb.dec_lut[code] == 0


def check_payload_properties(o, x: np.ndarray, cb, payload: bytes, meta):
    """Properties every payload must have, whatever the codebook."""
    n = x.size
    ex = exponents(x)
    marked = cb.enc_lut_marked.astype(np.int64)
    esc = np.nonzero(marked[ex] == 16)[0]
    assert meta.n_esc == esc.size
    assert len(payload) == meta.comp_bytes == closed_form_total(n, esc.size)
    buf = np.frombuffer(payload, np.uint8)
    off = meta.offsets
    e = esc.size
    cid = buf[off[2]: off[2] + 4 * e].view("<i4").astype(np.int64) if e else np.zeros(0, np.int64)
    pos = buf[off[3]: off[3] + 2 * e].view("<u2").astype(np.int64) if e else np.zeros(0, np.int64)
    ev = buf[off[4]: off[4] + e].astype(np.int64)
    idx = cid * meta.chunk_size + pos
    # escape set == elements whose exponent has no code, in ascending order
    assert np.array_equal(idx, esc)
    assert np.all(pos < meta.chunk_size)
    assert np.array_equal(ev, ex[esc])
    # decode reproduces the input bit for bit
    out = o.decode(payload, meta, cb.dec_lut)
    assert np.array_equal(out, x)


def pin_bruteforce_alphabet(o, max_full_n: int = 3, sampled=((4, 1500), (5, 1500)), seed: int = 3):
    """Every sequence over the 14-pattern alphabet for n <= max_full_n, a random
    sample for longer n; each encoded with its own codebook, a foreign codebook
    covering a subset of its exponents and a disjoint one (all-escape)."""
    foreign = [
        o.calibrate(np.array([0x3F80, 0x3F80, 0x0000], np.uint16)),   # exponents {127, 0}
        o.calibrate(np.array([0x4000], np.uint16)),                   # {128}: disjoint
        o.calibrate(np.array([0x7F80, 0x7F7F, 0x7F7F], np.uint16)),   # {254, 255}
    ]
    rng = np.random.default_rng(seed)
    seqs = []
    for n in range(0, max_full_n + 1):
        seqs.extend(itertools.product(range(ALPHABET.size), repeat=n))
    for n, count in sampled:
        seqs.extend(tuple(r) for r in rng.integers(0, ALPHABET.size, size=(count, n)))
    for s in seqs:
        x = ALPHABET[list(s)] if s else np.zeros(0, np.uint16)
        own = o.calibrate(x)
        codes = rank_codes(own.counts)
        assert own.n_codes == len(codes)
        for cb in [own] + foreign:
            payload, meta = o.encode(x, cb)
            check_payload_properties(o, x, cb, payload, meta)
        if x.size:
            assert o.encode(x, own)[1].n_esc == 0  # at most 4 exponents: all coded


def pin_random_roundtrip(o, seed: int = 4, trials: int = 40):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 5000)) | (t & 1)  # odd and even n
        x = rng.integers(0, 65536, size=n, dtype=np.uint32).astype(np.uint16)
        cb = o.calibrate(x)
        codes = rank_codes(cb.counts)
        assert cb.n_codes == len(codes)
        payload, meta = o.encode(x, cb)
        assert meta.n_esc == n - cb.covered
        check_payload_properties(o, x, cb, payload, meta)


ALL_PINS = [pin_worked_examples, pin_layout_table, pin_layout_closed_form,
            pin_exhaustive_patterns, pin_select_rank, pin_bruteforce_alphabet,
            pin_random_roundtrip]
