"""The CPU oracle against its pins (hand-derived payloads, closed forms, an
independent rank characterisation, brute force, losslessness)."""
import numpy as np
import pytest

import oracle
import oracle_pins as P
import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore")


@pytest.fixture(scope="module")
def o():
    oracle.build()
    return oracle.OracleLib()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)


def _ratio(o, x_bf16):
    x = W.bits(x_bf16).numpy()
    cb = o.calibrate(x)
    payload, meta = o.encode(x, cb)
    assert np.array_equal(o.decode(payload, meta, cb.dec_lut), x.view(np.uint16))
    return meta.comp_bytes / (2 * x.size), cb, meta


def test_ratio_weight_like(o):
    # page 1 docstring: about 0.750 (payload / raw) on Gaussian weight-like data
    r, cb, meta = _ratio(o, W.gaussian_weight(1_000_003, seed=0))
    assert 0.749 <= r <= 0.752, r
    # N(0, 0.02): the top-16 exponents are the contiguous block 108..123
    assert sorted(int(v) for v in cb.dec_lut) == list(range(108, 124))


def test_ratio_kv_like(o):
    # page 2, "What it does": about 0.756x of raw expected on KV activations
    r, cb, meta = _ratio(o, W.kv_layer(seed=2, stream=0, seq=1024))
    assert 0.750 <= r <= 0.765, r


def test_escape_heavy_expands(o):
    # page 2, invariant 3: data whose exponents are widely spread can grow
    r, cb, meta = _ratio(o, W.log_uniform_stress(1 << 18, seed=3, stream=0))
    assert r > 1.17, r
    assert meta.n_esc > (1 << 18) // 2


def test_subnormal_heavy(o):
    x = W.bits(W.subnormal_gaussian(1 << 18, seed=3, stream=1)).numpy().view(np.uint16)
    cb = o.calibrate(x)
    # every value is a subnormal or a zero: one exponent (0), no escapes
    assert cb.n_codes == 1 and cb.dec_lut[0] == 0 and cb.covered == x.size
    payload, meta = o.encode(x, cb)
    assert meta.n_esc == 0 and meta.comp_bytes == P.closed_form_total(x.size, 0)
    assert np.array_equal(o.decode(payload, meta, cb.dec_lut), x)
    assert np.count_nonzero(x & 0x7FFF) > 0.9 * x.size  # mostly non-zero subnormals


def test_escapes_at_chunk_edges(o):
    n = 5 * 1024 + 3
    x = np.full(n, 0x3F80, np.uint16)
    edges = [0, 1, 1023, 1024, 1025, 2047, 2048, 4095, 4096, n - 1]
    x[edges] = 0x4000
    cb = o.calibrate(np.array([0x3F80], np.uint16))  # exponent 128 escapes
    payload, meta = o.encode(x, cb)
    assert meta.n_esc == len(edges)
    P.check_payload_properties(o, x, cb, payload, meta)


def test_decode_rejects_corrupt(o):
    # escapes at elements 5 (chunk 0, pos 5), 1500 (chunk 1, pos 476), 2999 (chunk 2, pos 951)
    x = np.full(3000, 0x3F80, np.uint16)
    x[[5, 1500, 2999]] = 0x4000
    cb = o.calibrate(np.array([0x3F80], np.uint16))
    payload, meta = o.encode(x, cb)
    assert meta.n_esc == 3
    cid_at, pos_at = meta.offsets[2], meta.offsets[3]
    assert o.decode_status(payload, meta, cb.dec_lut)[0] == oracle.OK

    def patched(**fields):
        b = bytearray(payload)
        for (at, val, width) in fields.values():
            b[at: at + width] = val.to_bytes(width, "little", signed=val < 0)
        return bytes(b)

    cases = {
        "lpos_ge_chunk": patched(p=(pos_at, 1024, 2)),
        "idx_ge_n": patched(c=(cid_at + 8, 9, 4)),
        # escape 0 -> element 1000, escape 1 -> element 476: order broken
        "not_increasing": patched(p=(pos_at, 1000, 2), c=(cid_at + 4, 0, 4)),
        "duplicate": patched(p=(pos_at + 2, 5, 2), c=(cid_at + 4, 0, 4)),
        "negative_chunk": patched(c=(cid_at, -1, 4)),
    }
    for name, blob in cases.items():
        rc, _ = o.decode_status(blob, meta, cb.dec_lut)
        assert rc == oracle.ECORRUPT, name
    # truncated payload and offsets that break the layout rule
    assert o.decode_status(payload[:-1], meta, cb.dec_lut)[0] == oracle.ECORRUPT
    bad = oracle.Meta(meta.n, meta.n_pairs, meta.chunk_size, meta.n_esc, meta.comp_bytes,
                      (0, meta.offsets[1] + 4) + tuple(meta.offsets[2:]))
    assert o.decode_status(payload, bad, cb.dec_lut)[0] == oracle.ECORRUPT


def test_chunk_size_parameter(o):
    """Page 1, encode(x, codebook, chunk_size): each escape is stored as (chunk
    number, position inside the chunk) of its element; only the escape
    sections depend on the chunk size.  Pinned by planted escape positions and
    the two degenerate chunkings (one element per chunk; one chunk for all)."""
    n = 70_001
    x = np.full(n, 0x3F80, np.uint16)
    planted = np.array([0, 2, 999, 1000, 1023, 1024, 4097, 12344, 12345, 65535, 65536, n - 1])
    x[planted] = 0x4000                  # exponent 128 escapes under this codebook
    cb = o.calibrate(np.array([0x3F80], np.uint16))
    ref, ref_meta = o.encode(x, cb)
    dense = ref_meta.offsets[2]
    for chunk in (1, 3, 1000, 1024, 4096, 12345, 65536):
        payload, meta = o.encode(x, cb, chunk)
        assert meta.chunk_size == chunk and meta.n_esc == planted.size
        assert payload[:dense] == ref[:dense]          # pk, sm and their padding
        cid = np.frombuffer(payload, "<i4", planted.size, meta.offsets[2])
        pos = np.frombuffer(payload, "<u2", planted.size, meta.offsets[3])
        ev = np.frombuffer(payload, np.uint8, planted.size, meta.offsets[4])
        assert np.array_equal(cid, planted // chunk) and np.array_equal(pos, planted % chunk)
        assert np.all(ev == 128)
        if chunk == 1:
            assert np.all(pos == 0) and np.array_equal(cid, planted)
        assert np.array_equal(o.decode(payload, meta, cb.dec_lut), x)
    # one chunk holds everything when chunk_size >= n
    y = x[:60_000]
    payload, meta = o.encode(y, cb, 65536)
    cid = np.frombuffer(payload, "<i4", meta.n_esc, meta.offsets[2])
    pos = np.frombuffer(payload, "<u2", meta.n_esc, meta.offsets[3])
    assert np.all(cid == 0) and np.array_equal(pos, planted[planted < 60_000])
