"""Encode with caller codebooks whose escape-marked table holds arbitrary
bytes, through the C ABI, against the oracle.

Page 1 (encode_torch) escapes an element when its marked code is above 15 and
packs the marked code's low four bits as its nibble, for any byte value of the
table; a codebook loaded from JSON or built by a caller need not hold only
0..16.  Payload bytes [0, comp_bytes), metadata and decoded bits must equal the
oracle's exactly (tolerance 0), on full and partial encode tiles, on sparse
escapes (written per thread) and on escape-dense tiles (staged through LDS).
"""
import sys

import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import persist
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
_WS = {}


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _ws(n):
    key = max(n, 1 << 20).bit_length()
    if key not in _WS:
        _WS[key] = S.Workspace(1 << key, device=DEV)
    return _WS[key]


def _random_bits(n, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randint(-32768, 32768, (n,), dtype=torch.int32, generator=g).to(torch.int16)
    return x.view(torch.bfloat16)


def _tables(kind, seed):
    """(enc_lut_marked, dec_lut) as uint8 arrays."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(0, 256, 16, dtype=np.uint8)
    if kind == "random_bytes":
        marked = rng.integers(0, 256, 256, dtype=np.uint8)
    elif kind == "f0_heavy":
        marked = np.full(256, 0xF0, np.uint8)
        keep = rng.choice(256, 4, replace=False)
        marked[keep] = np.arange(4, dtype=np.uint8) + 3
    elif kind == "all_ff":
        marked = np.full(256, 0xFF, np.uint8)
    elif kind == "escape_nibbles":
        # escapes whose low nibble is not zero (17..31), codes 0..15 elsewhere
        marked = rng.integers(0, 16, 256, dtype=np.uint8)
        esc = rng.choice(256, 200, replace=False)
        marked[esc] = rng.integers(17, 32, esc.size, dtype=np.uint8)
    elif kind == "sparse_high":
        # gaussian data: most exponents coded, a few of the frequent ones
        # marked with large bytes so that tiles hold a few hundred escapes
        marked = np.full(256, 0x80, np.uint8)
        marked[104:124] = np.arange(20, dtype=np.uint8) % 16
        marked[[104, 105, 106, 107]] = [0x21, 0x7F, 0xC4, 0x11]
    else:
        raise ValueError(kind)
    return marked, dec


def _device_codebook(marked, dec):
    cb = S.Codebook()
    for k in range(256):
        cb.enc_lut_marked[k] = int(marked[k])
        cb.enc_lut[k] = int(marked[k]) & 15
        cb.common_lut[k] = 1 if marked[k] <= 15 else 0
    for k in range(16):
        cb.dec_lut[k] = int(dec[k])
    cb.n_codes = 16
    cb.covered, cb.total = 7, 11           # copied into the metadata as they are
    return persist.to_device(cb, DEV)


def _oracle_codebook(marked, dec):
    z = np.zeros(256, np.uint8)
    return oracle.Codebook(np.zeros(256, np.uint64), z, marked.copy(), dec.copy(), z, 16, 0, 0)


CASES = [
    ("random_bytes", "bits", 100_003),
    ("random_bytes", "gauss", 3 * 8192 + 77),
    ("random_bytes", "bits", 5_000),             # one partial tile only
    ("f0_heavy", "bits", 3 * 8192 + 77),         # escape-dense: staged through LDS
    ("f0_heavy", "bits", 8192),
    ("all_ff", "bits", 2 * 8192 + 1),
    ("all_ff", "gauss", 1_001),
    ("escape_nibbles", "bits", 40_961),
    ("sparse_high", "gauss", 6 * 8192 + 3),      # a few hundred escapes per tile
]


@pytest.mark.parametrize("kind,data,n", CASES)
def test_marked_table_bytes_match_oracle(kind, data, n):
    print("codebook-table case %s %s n=%d" % (kind, data, n), flush=True)
    sys.stdout.flush()
    seed = 1000 + n
    x_cpu = _random_bits(n, seed) if data == "bits" else W.gaussian_weight(n, seed=seed)
    xs = W.bits(x_cpu).numpy().view(np.uint16)
    marked, dec = _tables(kind, seed)
    ocb = _oracle_codebook(marked, dec)
    opay, om = oracle.encode(xs, ocb)

    x = x_cpu.to(DEV)
    cb = _device_codebook(marked, dec)
    cap = S.payload_size(n, n) + 64
    payload = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
    payload, meta = S.encode(x, cb, _ws(n), payload=payload)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=status)
    out_fast = S.decode(payload, meta, cb, n)
    torch.cuda.synchronize()

    m = S.read_meta(meta)
    assert m.status == 0
    assert (m.n, m.n_esc, m.comp_bytes) == (om.n, om.n_esc, om.comp_bytes)
    assert tuple(m.offsets) == tuple(om.offsets)
    pay = payload.cpu().numpy()
    got = pay[: m.comp_bytes].tobytes()
    if got != opay:
        a, b = np.frombuffer(got, np.uint8), np.frombuffer(opay, np.uint8)
        bad = np.nonzero(a != b)[0]
        raise AssertionError("payload differs at %d bytes, first at %d (sections %s)"
                             % (bad.size, bad[0], om.offsets))
    # nothing written past the payload
    assert np.all(pay[m.comp_bytes:] == 0xA5)
    want = oracle.decode(opay, om, dec)
    assert int(status.item()) == 0
    assert np.array_equal(W.bits(out.cpu()).numpy().view(np.uint16), want)
    assert np.array_equal(W.bits(out_fast.cpu()).numpy().view(np.uint16), want)
