"""Parity of the HIP path with the CPU oracle, through the C ABI.

Integer work, tolerance 0: codebook bytes, metadata, payload bytes
[0, comp_bytes) and decoded bit patterns must equal the oracle's exactly, and
each side must decode the other's payload.  Small cases span several tiles and
ragged tails; the large cases are the workloads at full size, in the same
launch configuration the benchmark times.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
import oracle
import oracle_pins as P
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


_WS = {}


def workspace(n):
    """One workspace per size class, reused across tests (as a caller would)."""
    key = max(n, 1 << 20).bit_length()
    if key not in _WS:
        _WS[key] = S.Workspace(1 << key, device=DEV)
    return _WS[key]


def host_bits(x_bf16):
    return W.bits(x_bf16.cpu()).numpy().view(np.uint16)


def gpu_run(x_cpu, cb_source=None, ws=None):
    """calibrate (on cb_source or x) -> encode -> decode on the GPU."""
    x = x_cpu.reshape(-1).to(DEV)
    n = x.numel()
    ws = ws or workspace(max(n, 0 if cb_source is None else cb_source.numel()))
    src = x if cb_source is None else cb_source.reshape(-1).to(DEV)
    cb = S.calibrate(src, ws)
    payload, meta = S.encode(x, cb, ws)
    # decode twice: the plain fused path (no status word) and the validating one
    out_fast = S.decode(payload, meta, cb, n)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=status)
    torch.cuda.synchronize()
    m = S.read_meta(meta)
    c = S.read_codebook(cb)
    pay = payload[: m.comp_bytes].cpu().numpy().tobytes()
    return dict(cb=c, meta=m, payload=pay, out=host_bits(out), out_fast=host_bits(out_fast),
                status=int(status.item()), cb_dev=cb, payload_dev=payload, meta_dev=meta)


def check_codebook(c, ocb):
    assert bytes(c.enc_lut) == ocb.enc_lut.tobytes()
    assert bytes(c.enc_lut_marked) == ocb.enc_lut_marked.tobytes()
    assert bytes(c.dec_lut) == ocb.dec_lut.tobytes()
    assert bytes(c.common_lut) == ocb.common_lut.tobytes()
    assert c.n_codes == ocb.n_codes and c.covered == ocb.covered and c.total == ocb.total
    assert np.array_equal(np.frombuffer(bytes(c.counts), np.uint64), ocb.counts)


def check_meta(m, om, ocb_src):
    assert m.status == 0
    assert (m.n, m.n_pairs, m.chunk_size, m.n_esc, m.comp_bytes) == \
        (om.n, om.n_pairs, om.chunk_size, om.n_esc, om.comp_bytes)
    assert tuple(m.offsets) == tuple(om.offsets)
    assert (m.covered, m.total) == (ocb_src.covered, ocb_src.total)


def meta_to_device(om, ascending=False) -> torch.Tensor:
    """Device metadata for an oracle payload: the page's fields only, unless
    ``ascending`` marks the escape stream as sorted (this library's flag)."""
    m = _abi.Meta()
    m.n, m.n_pairs, m.chunk_size, m.n_esc, m.comp_bytes = (om.n, om.n_pairs, om.chunk_size,
                                                          om.n_esc, om.comp_bytes)
    for k in range(5):
        m.offsets[k] = om.offsets[k]
    m.flags = _abi.META_ASCENDING if ascending else 0
    raw = bytes(m)
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)


def gpu_decode_bytes(payload: bytes, om, dec_lut, validate=True, ascending=False) -> tuple:
    pay = torch.frombuffer(bytearray(payload + b"\0" * 16), dtype=torch.uint8).to(DEV)
    meta = meta_to_device(om, ascending)
    lut = torch.tensor(np.asarray(dec_lut, np.uint8)).to(DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV) if validate else None
    out = torch.empty(om.n, dtype=torch.bfloat16, device=DEV)
    if om.n:
        S.decode(pay[: len(payload)], meta, lut, om.n, out=out, status=status)
    torch.cuda.synchronize()
    return host_bits(out), (int(status.item()) if validate else 0)


def full_parity(x_cpu, cb_source=None, name=""):
    _say("parity case %s n=%d" % (name, x_cpu.numel()))
    xs = host_bits(x_cpu)
    g = gpu_run(x_cpu, cb_source)
    src = xs if cb_source is None else host_bits(cb_source)
    ocb = oracle.calibrate(src)
    check_codebook(g["cb"], ocb)
    opay, om = oracle.encode(xs, ocb)
    check_meta(g["meta"], om, ocb)
    if g["payload"] != opay:
        a = np.frombuffer(g["payload"], np.uint8)
        b = np.frombuffer(opay, np.uint8)
        bad = np.nonzero(a != b)[0]
        raise AssertionError("payload differs at %d bytes, first at %d (sections %s)"
                             % (bad.size, bad[0], om.offsets))
    assert g["status"] == 0
    assert np.array_equal(g["out"], xs)
    assert np.array_equal(g["out_fast"], xs)
    # cross-decoding: oracle decodes the GPU payload, the GPU decodes the oracle's
    assert np.array_equal(oracle.decode(g["payload"], om, ocb.dec_lut), xs)
    out2, st2 = gpu_decode_bytes(opay, om, ocb.dec_lut)
    assert st2 == 0 and np.array_equal(out2, xs)
    # without a status word: page-format metadata (escapes applied in any
    # order) and the same metadata marked ascending (patched per tile)
    out3, _ = gpu_decode_bytes(opay, om, ocb.dec_lut, validate=False)
    assert np.array_equal(out3, xs)
    out4, _ = gpu_decode_bytes(opay, om, ocb.dec_lut, validate=False, ascending=True)
    assert np.array_equal(out4, xs)
    assert g["meta"].flags == _abi.META_ASCENDING
    return g, om


SIZES = [0, 1, 2, 3, 5, 7, 8, 9, 15, 16, 17, 31, 33, 1023, 1024, 1025, 2047, 4095, 4096, 4097,
         8191, 8192, 8193, 12289, 65536, 100_003]


@pytest.mark.parametrize("n", SIZES)
def test_sizes_gaussian(n):
    full_parity(W.gaussian_weight(n, seed=11), name="gauss")


@pytest.mark.parametrize("n", [1, 7, 4097, 8193, 100_003, 300_001])
def test_sizes_escape_heavy(n):
    full_parity(W.log_uniform_stress(n, seed=12), name="loguniform")


@pytest.mark.parametrize("n", [3, 4096, 77_777])
def test_random_bits(n):
    g = torch.Generator().manual_seed(n)
    x = torch.randint(-32768, 32768, (n,), dtype=torch.int32, generator=g).to(torch.int16)
    full_parity(x.view(torch.bfloat16), name="randbits")


def test_subnormal_only():
    full_parity(W.subnormal_gaussian(70_001, seed=3, stream=1), name="subnormal")


def test_constant_tensor():
    full_parity(torch.full((50_001,), -3.5, dtype=torch.bfloat16), name="constant")


def test_exhaustive_patterns():
    x = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    g, om = full_parity(x, name="exhaustive")
    assert om.n_esc == 61440 and om.comp_bytes == 528384


def test_foreign_codebook_all_escape():
    x = W.gaussian_weight(50_003, seed=13)
    src = W.subnormal_gaussian(1000, seed=3, stream=1)   # only exponent 0 has a code
    g, om = full_parity(x, cb_source=src, name="all-escape")
    assert om.n_esc > 49_000


def test_golden_examples():
    for ex in P.load_examples():
        x = torch.from_numpy(P.example_input(ex).astype(np.int16)).view(torch.bfloat16)
        src = None
        if ex["codebook_from"] != "self":
            src = torch.from_numpy(P._u16(ex["codebook_from"]["x"]).astype(np.int16)).view(
                torch.bfloat16)
        if x.numel() == 0:
            continue
        g = gpu_run(x, src)
        assert g["payload"] == P.example_payload(ex), ex["name"]
        assert np.array_equal(g["out"], P.example_input(ex))


def test_escapes_at_chunk_and_tile_edges():
    n = 3 * 4096 + 5
    x = torch.full((n,), 1.0, dtype=torch.bfloat16)
    edges = [0, 1, 1023, 1024, 2047, 2048, 4095, 4096, 4097, 8191, 8192, 12287, 12288, n - 1]
    x[edges] = 2.0
    src = torch.ones(8, dtype=torch.bfloat16)
    g, om = full_parity(x, cb_source=src, name="edges")
    assert om.n_esc == len(edges)


@pytest.mark.parametrize("counts", [
    # escapes per 8192-element encode tile around the staging cap of 512
    [0, 1, 511, 512, 513, 2048, 8191, 8192, 700],
    [513, 0, 0, 0, 5, 512, 0, 8192, 1],
    [8192] * 5 + [3000],
])
def test_staging_cap_edges(counts):
    """Tiles whose escapes are staged (at most 512) and tiles whose escapes
    the placement derives from the input again (more than 512), mixed in one
    placement block and across blocks; the last tile is partial."""
    src = torch.ones(8, dtype=torch.bfloat16)          # codes exponent 127 only
    tail = 4321
    n = (len(counts) - 1) * 8192 + tail
    rng = np.random.default_rng(sum(counts))
    b = np.full(n, 0x3F80, np.uint16)
    for t, c in enumerate(counts):
        size = 8192 if t < len(counts) - 1 else tail
        c = min(c, size)
        pos = t * 8192 + rng.choice(size, c, replace=False)
        b[pos] = (rng.integers(0, 2, c) << 15) | (rng.integers(128, 256, c) << 7) | \
            rng.integers(0, 128, c)
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    g, om = full_parity(x, cb_source=src, name="staging-cap")
    assert om.n_esc == sum(min(c, 8192 if t < len(counts) - 1 else tail)
                           for t, c in enumerate(counts))


def test_decode_patch_paths():
    """Each way the decode applies escapes, byte for byte: scattered from
    registers (a tile with few, and a tile whose position the interpolation
    misses by far), through the tile's sign/mantissa bytes staged in LDS (a
    tile with more than 512 while the tensor averages fewer), and with the
    whole tile built in LDS (more than 512 per tile on average)."""
    src = torch.ones(8, dtype=torch.bfloat16)          # codes exponent 127 only
    n = 6 * 8192 + 100
    b = np.full(n, 0x3F80, np.uint16)
    j = np.arange(100)
    few = 8192 + 37 * j                                 # tile 1: 100 escapes
    b[few] = ((j % 2) << 15) | (((j % 120) + 1) << 7) | (j & 0x7F)
    j = np.arange(2048)
    many = 2 * 8192 + 4 * j                             # tile 2: 2048 escapes
    b[many] = ((j % 3 == 0) << 15) | ((130 + j % 100) << 7) | ((j * 7) & 0x7F)
    b[[n - 1, n - 2, 5 * 8192]] = [0x0001, 0xFF80, 0x8000]
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    _, om = full_parity(x, cb_source=src, name="patch paths")
    assert om.n_esc == 100 + 2048 + 3 and om.n_esc * 8192 <= 512 * n
    # more than 512 per tile on average: every third element escapes
    n = 4 * 8192 + 333
    b = np.full(n, 0x3F80, np.uint16)
    k = np.arange(0, n, 3)
    b[k] = ((k & 1) << 15) | ((k % 126) << 7) | (k & 0x7F)
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    _, om = full_parity(x, cb_source=src, name="tile in LDS")
    assert om.n_esc == len(k) and om.n_esc * 8192 > 512 * n


@pytest.mark.parametrize("per_tile", [1, 31, 32, 33, 63, 64, 65])
def test_decode_escapes_per_tile(per_tile):
    """Tiles with the same number of escapes each, around the search's 64-entry
    window (so that the interpolated rank of a tile's first escape is close:
    the window settles it, or its 64 samples do), and a ragged last tile
    that takes the element path."""
    src = torch.ones(8, dtype=torch.bfloat16)          # codes exponent 127 only
    n = 9 * 8192 + 1234
    b = np.full(n, 0x3F80, np.uint16)
    for t in range(10):
        lo, hi = t * 8192, min(n, (t + 1) * 8192)
        pos = lo + (np.arange(per_tile) * ((hi - lo) // per_tile)) + (t * 7) % 13
        pos = pos[pos < hi]
        j = np.arange(len(pos))
        b[pos] = (((j + t) & 1) << 15) | (((j * 5 + t) % 120 + 1) << 7) | ((j * 3 + t) & 0x7F)
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    _, om = full_parity(x, cb_source=src, name="escapes per tile %d" % per_tile)
    assert om.n_esc >= 9 * per_tile


def test_determinism_and_workspace_reuse():
    big = W.log_uniform_stress(1 << 20, seed=14)
    small = W.gaussian_weight(5_001, seed=15)
    ws = workspace(1 << 20)
    runs = [gpu_run(big, ws=ws), gpu_run(small, ws=ws), gpu_run(big, ws=ws), gpu_run(big, ws=ws)]
    assert runs[0]["payload"] == runs[2]["payload"] == runs[3]["payload"]
    xs = host_bits(small)
    opay, _ = oracle.encode(xs, oracle.calibrate(xs))
    assert runs[1]["payload"] == opay


@pytest.mark.parametrize("make,extra", [
    (W.log_uniform_stress, 0),      # escape-dense tiles: derived again by the placement
    (W.log_uniform_stress, 2),      # capacity not a whole number of chunk ids
    (W.log_uniform_stress, 3),
    (W.gaussian_weight, 0),         # few escapes: staged ones placed by the tail
])
def test_capacity_overflow(make, extra):
    n = 20_001 if make is W.log_uniform_stress else 600_001
    x = make(n, seed=16).to(DEV)
    ws = workspace(n)
    cb = S.calibrate(x, ws)
    xs = host_bits(x)
    opay, om = oracle.encode(xs, oracle.calibrate(xs))
    cap = om.offsets[2] + 4 * (om.n_esc // 2) + extra   # room for half of the chunk ids
    guard = 64
    buf = torch.full((cap + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    meta = torch.zeros(S.codec.META_BYTES, dtype=torch.uint8, device=DEV)
    rc = _abi.splitzip_encode(x.view(torch.int16).data_ptr(), x.numel(), cb.data_ptr(),
                              buf.data_ptr(), cap, meta.data_ptr(), ws.ptr(), ws.nbytes,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    m = S.read_meta(meta)
    assert m.status == _abi.ERR_CAPACITY and m.comp_bytes == om.comp_bytes
    host = buf.cpu().numpy()
    assert bool((host[cap:] == 0xA5).all())          # nothing written past capacity
    # the dense sections and every chunk id that fits whole are the oracle's
    whole = om.offsets[2] + 4 * ((cap - om.offsets[2]) // 4)
    assert host[:whole].tobytes() == opay[:whole]
    assert bool((host[whole:cap] == 0xA5).all())
    # synchronous check: below the dense size
    rc = _abi.splitzip_encode(x.view(torch.int16).data_ptr(), x.numel(), cb.data_ptr(),
                              buf.data_ptr(), om.offsets[2] - 1, meta.data_ptr(), ws.ptr(),
                              ws.nbytes, torch.cuda.current_stream().cuda_stream)
    assert rc == _abi.ERR_CAPACITY


def test_decode_flags_corrupt_streams():
    n = 3000
    x = torch.full((n,), 1.0, dtype=torch.bfloat16)
    x[[5, 1500, 2999]] = 2.0
    xs = host_bits(x)
    ocb = oracle.calibrate(np.array([0x3F80], np.uint16))
    opay, om = oracle.encode(xs, ocb)
    cid_at, pos_at = om.offsets[2], om.offsets[3]

    def patched(edits):
        b = bytearray(opay)
        for at, val, width in edits:
            b[at: at + width] = val.to_bytes(width, "little", signed=val < 0)
        return bytes(b)

    cases = {
        _abi.DEC_POS_GE_CHUNK: [(pos_at, 1024, 2)],
        _abi.DEC_ESC_OUT_OF_RANGE: [(cid_at + 8, 9, 4)],
        _abi.DEC_NOT_INCREASING: [(pos_at, 1000, 2), (cid_at + 4, 0, 4)],
    }
    for bit, edits in cases.items():
        _, st = gpu_decode_bytes(patched(edits), om, ocb.dec_lut)
        assert st & bit, (bit, st)
    bad = oracle.Meta(om.n, om.n_pairs, om.chunk_size, om.n_esc, om.comp_bytes,
                      (0, om.offsets[1] + 4) + tuple(om.offsets[2:]))
    _, st = gpu_decode_bytes(opay, bad, ocb.dec_lut)
    assert st & _abi.DEC_BAD_META
    _, st = gpu_decode_bytes(opay, om, ocb.dec_lut)
    assert st == 0


def test_unsorted_escape_stream_with_validation():
    """A stream whose escapes are not in ascending order is flagged, and the
    validating decode (which re-applies every escape by scatter) still
    reproduces the tensor."""
    n = 3 * 8192 + 77
    x = torch.full((n,), 1.0, dtype=torch.bfloat16)
    pos = [3, 900, 5000, 8191, 8192, 9000, 17000, 24000, n - 1]
    x[pos] = torch.tensor([2.0, -4.0, 8.0, 0.5, 16.0, -0.25, 3.0, 64.0, -2.0],
                          dtype=torch.bfloat16)
    xs = host_bits(x)
    ocb = oracle.calibrate(np.array([0x3F80], np.uint16))
    opay, om = oracle.encode(xs, ocb)
    e = om.n_esc
    assert e == len(pos)
    buf = bytearray(opay)
    order = list(range(e))[::-1]          # reverse the escape stream
    for sec, width in ((2, 4), (3, 2), (4, 1)):
        at = om.offsets[sec]
        items = [bytes(buf[at + width * r: at + width * (r + 1)]) for r in range(e)]
        for k, r in enumerate(order):
            buf[at + width * k: at + width * (k + 1)] = items[r]
    out, st = gpu_decode_bytes(bytes(buf), om, ocb.dec_lut)
    assert st & _abi.DEC_NOT_INCREASING
    assert np.array_equal(out, xs)
    # no status word: the metadata does not mark the stream ascending, so
    # the escapes are applied by index in any order (page 1, decode_torch)
    out, _ = gpu_decode_bytes(bytes(buf), om, ocb.dec_lut, validate=False)
    assert np.array_equal(out, xs)


def _shuffle_escapes(opay: bytes, om, rng) -> bytes:
    buf = bytearray(opay)
    e = om.n_esc
    order = rng.permutation(e)
    for sec, width in ((2, 4), (3, 2), (4, 1)):
        at = om.offsets[sec]
        items = np.frombuffer(bytes(buf[at: at + width * e]), np.uint8).reshape(e, width)
        buf[at: at + width * e] = items[order].tobytes()
    return bytes(buf)


@pytest.mark.parametrize("make,n", [
    (W.log_uniform_stress, 3 * 8192 + 77),      # dense escapes, all tiles
    (W.gaussian_weight, 1_000_003),             # a few escapes
    (W.log_uniform_stress, 100_003),
])
def test_shuffled_escape_stream_without_status(make, n):
    """An escape stream in random order, with page-format metadata (no
    ascending flag) and no status word, decodes bit for bit: plain, and in
    place from the head of the output buffer."""
    x = make(n, seed=77)
    xs = host_bits(x)
    ocb = oracle.calibrate(xs)
    opay, om = oracle.encode(xs, ocb)
    assert om.n_esc > 0
    shuffled = _shuffle_escapes(opay, om, np.random.default_rng(n))
    assert np.array_equal(oracle.decode(shuffled, om, ocb.dec_lut, validate=False), xs)
    out, _ = gpu_decode_bytes(shuffled, om, ocb.dec_lut, validate=False)
    assert np.array_equal(out, xs)
    # in place
    slot = torch.zeros(max(2 * n, om.comp_bytes), dtype=torch.uint8)
    slot[: om.comp_bytes] = torch.frombuffer(bytearray(shuffled), dtype=torch.uint8)
    slot = slot.to(DEV)
    stash = torch.empty(om.comp_bytes, dtype=torch.uint8, device=DEV)
    lut = torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV)
    res = S.decode_slot(slot, meta_to_device(om), lut, n, stash)
    torch.cuda.synchronize()
    assert np.array_equal(W.bits(res.cpu()).numpy().view(np.uint16), xs)


@pytest.mark.parametrize("tiles", [255, 256, 257, 513])
def test_escape_placement_across_tail_blocks(tiles):
    """Escapes spread over more tiles than one placement block handles."""
    n = tiles * 4096 - 5
    full_parity(W.log_uniform_stress(n, seed=30 + tiles), name="tail blocks %d" % tiles)


@pytest.mark.parametrize("n", [300 * 4096 * 8 - 3, 8 * 4096 * 1024 - 8, 17 * 4096 * 8 + 5])
def test_calibrate_grid_edges(n):
    """Calibrate grids of a full 512 workgroups with an uneven last group."""
    full_parity(W.gaussian_weight(n, seed=40), name="calibrate grid")


def test_argument_errors():
    x = torch.zeros(64, dtype=torch.bfloat16, device=DEV)
    ws = workspace(64)
    cbt = torch.empty(S.codec.CODEBOOK_BYTES, dtype=torch.uint8, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    xp = x.view(torch.int16).data_ptr()
    assert _abi.splitzip_calibrate(xp + 2, 63, cbt.data_ptr(), ws.ptr(), ws.nbytes, s) == \
        _abi.ERR_INVALID
    assert _abi.splitzip_calibrate(0, 64, cbt.data_ptr(), ws.ptr(), ws.nbytes, s) == \
        _abi.ERR_INVALID
    assert _abi.splitzip_calibrate(xp, 64, cbt.data_ptr(), ws.ptr(), 100, s) == \
        _abi.ERR_WORKSPACE
    assert _abi.splitzip_calibrate(xp, 64, cbt.data_ptr(), ws.ptr(), ws.nbytes, s) == _abi.OK
    with pytest.raises(ValueError):
        S.calibrate(torch.zeros(8, dtype=torch.float16, device=DEV), ws)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def test_workload_weight_1m_odd():
    g, om = full_parity(W.gaussian_weight(1_000_003, seed=0), name="weight_1m_odd")
    assert 0.749 < om.comp_bytes / (2 * 1_000_003) < 0.752


@pytest.mark.parametrize("kv", [0, 1])
def test_workload_kv_layer(kv):
    full_parity(W.kv_layer(seed=2, stream=kv), name="kv_layer_%d" % kv)


def test_workload_stress_log_uniform():
    g, om = full_parity(W.log_uniform_stress(1 << 24, seed=3, stream=0), name="stress_loguniform")
    assert om.n_esc > (1 << 23)


def test_workload_stress_subnormal():
    g, om = full_parity(W.subnormal_gaussian(1 << 24, seed=3, stream=1), name="stress_subnormal")
    assert om.n_esc == 0


def test_workload_linear_weight_decode_100x():
    x_cpu = W.weight_with_outliers(seed=4)
    _say("parity case linear_weight n=%d" % x_cpu.numel())
    g, om = full_parity(x_cpu, name="linear_weight")
    n = x_cpu.numel()
    arena = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    for _ in range(100):
        S.decode(g["payload_dev"], g["meta_dev"], g["cb_dev"], n, out=arena, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(host_bits(arena), host_bits(x_cpu))


def test_workload_kv_stream_4gib():
    """32 layers x (K, V) [1, 8, 32768, 128], one codebook each.  Every tensor
    is round-tripped on the GPU and checked against the closed-form size and
    the escape-count identity; three of them are compared byte for byte with
    the oracle."""
    n = 8 * 32768 * 128
    ws = workspace(n)
    payload = torch.empty(S.payload_size(n, n), dtype=torch.uint8, device=DEV)
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    full = {(0, 0), (17, 1), (31, 1)}
    for layer in range(32):
        for kv in range(2):
            x = W.kv_cache_tensor(layer, kv, device=DEV)
            cb = S.calibrate(x, ws)
            _, meta = S.encode(x, cb, ws, payload=payload)
            S.decode(payload, meta, cb, n, out=out, status=status)
            assert torch.equal(out.view(torch.int16), x.reshape(-1).view(torch.int16))
            m = S.read_meta(meta)
            c = S.read_codebook(cb)
            assert m.status == 0 and m.n_esc == n - c.covered
            assert m.comp_bytes == P.closed_form_total(n, m.n_esc)
            if (layer, kv) in full:
                _say("parity case kv_stream layer=%d kv=%d" % (layer, kv))
                xs = host_bits(x)
                ocb = oracle.calibrate(xs)
                check_codebook(c, ocb)
                opay, om = oracle.encode(xs, ocb)
                check_meta(m, om, ocb)
                assert payload[: m.comp_bytes].cpu().numpy().tobytes() == opay
    assert int(status.item()) == 0
