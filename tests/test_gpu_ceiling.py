"""The reference memory streams the bench measures the codec against run and
touch exactly the bytes their header states: outputs equal the stated XORs
of the inputs, computed here with torch, and bytes past the stated ranges
stay untouched."""
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
from test_gpu_parity import DEV, _say

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _abi.ceiling_lib()


def _u32(t):
    return t.view(torch.int32).to(torch.int64) & 0xFFFFFFFF


@pytest.mark.parametrize("tiles", [1, 3, 37])
def test_encode_and_decode_shapes(tiles):
    lib = _abi.ceiling_lib()
    n = 8192 * tiles
    _say("reference streams n=%d" % n)
    g = torch.Generator().manual_seed(tiles)
    x = torch.randint(-(1 << 15), 1 << 15, (n,), generator=g, dtype=torch.int32)
    x = x.to(torch.int16).to(DEV)
    guard = 64
    pk = torch.full((n // 2 + guard,), 0x33, dtype=torch.uint8, device=DEV)
    sm = torch.full((n + guard,), 0x44, dtype=torch.uint8, device=DEV)
    out = torch.full((n + guard,), 0x55, dtype=torch.int16, device=DEV)
    sh = int(torch.cuda.current_stream().cuda_stream)
    assert lib.splitzip_ceiling_encode_shape(x.data_ptr(), n, pk.data_ptr(), sm.data_ptr(), sh) == 0
    assert lib.splitzip_ceiling_decode_shape(pk.data_ptr(), sm.data_ptr(), out.data_ptr(), n,
                                             sh) == 0
    torch.cuda.synchronize()
    q = _u32(x.view(torch.int32)).reshape(-1, 4).cpu()        # one 16-byte load per row
    want_pk = q[:, 0] ^ q[:, 1] ^ q[:, 2] ^ q[:, 3]
    want_sm = torch.stack([q[:, 0] ^ q[:, 2], q[:, 1] ^ q[:, 3]], 1)
    assert torch.equal(_u32(pk[: n // 2]).cpu(), want_pk)
    assert torch.equal(_u32(sm[:n]).cpu().reshape(-1, 2), want_sm)
    assert bool((pk[n // 2:] == 0x33).all()) and bool((sm[n:] == 0x44).all())
    o = _u32(out[:n]).cpu().reshape(-1, 4)
    assert torch.equal(o[:, 0], want_pk ^ want_sm[:, 0])
    assert torch.equal(o[:, 1], want_pk ^ want_sm[:, 1])
    assert torch.equal(o[:, 2], want_sm[:, 0] ^ 0x5A5A5A5A)
    assert torch.equal(o[:, 3], want_sm[:, 1] ^ 0xA5A5A5A5)
    assert bool((out[n:] == 0x55).all())


@pytest.mark.parametrize("nbytes,grid", [(16, 0), (1 << 20, 0), (1 << 20, 7), (4096, 1000)])
def test_read_stream(nbytes, grid):
    lib = _abi.ceiling_lib()
    _say("read stream bytes=%d grid=%d" % (nbytes, grid))
    x = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)   # XOR 0: the sink is never written
    sink = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    assert lib.splitzip_ceiling_read(x.data_ptr(), nbytes, grid, sink.data_ptr(),
                                     int(torch.cuda.current_stream().cuda_stream)) == 0
    torch.cuda.synchronize()
    assert int(sink.item()) == 7


@pytest.mark.parametrize("tiles", [1, 5])
def test_wide_shapes_touch_their_bytes(tiles):
    """Thread-contiguous 32-element units: the stated XORs over the stated
    ranges, nothing past them."""
    lib = _abi.ceiling_lib()
    n = 8192 * tiles
    _say("wide reference streams n=%d" % n)
    g = torch.Generator().manual_seed(50 + tiles)
    x = torch.randint(-(1 << 15), 1 << 15, (n,), generator=g, dtype=torch.int32)
    x = x.to(torch.int16).to(DEV)
    guard = 64
    pk = torch.full((n // 2 + guard,), 0x33, dtype=torch.uint8, device=DEV)
    sm = torch.full((n + guard,), 0x44, dtype=torch.uint8, device=DEV)
    out = torch.full((n + guard,), 0x55, dtype=torch.int16, device=DEV)
    sh = int(torch.cuda.current_stream().cuda_stream)
    assert lib.splitzip_ceiling_encode_wide(x.data_ptr(), n, pk.data_ptr(), sm.data_ptr(), sh) == 0
    assert lib.splitzip_ceiling_decode_wide(pk.data_ptr(), sm.data_ptr(), out.data_ptr(), n, sh) == 0
    torch.cuda.synchronize()
    q = _u32(x.view(torch.int32)).reshape(-1, 4, 4).cpu()     # per thread: 4 loads of 4 words
    want_pk = q[:, :, 0] ^ q[:, :, 1]                           # one 16-byte store per thread
    want_s0 = torch.stack([q[:, 0, 0] ^ q[:, 0, 2], q[:, 0, 1] ^ q[:, 0, 3],
                           q[:, 1, 0] ^ q[:, 1, 2], q[:, 1, 1] ^ q[:, 1, 3]], 1)
    want_s1 = torch.stack([q[:, 2, 0] ^ q[:, 2, 2], q[:, 2, 1] ^ q[:, 2, 3],
                           q[:, 3, 0] ^ q[:, 3, 2], q[:, 3, 1] ^ q[:, 3, 3]], 1)
    assert torch.equal(_u32(pk[: n // 2]).cpu().reshape(-1, 4), want_pk)
    s = _u32(sm[:n]).cpu().reshape(-1, 8)
    assert torch.equal(s[:, :4], want_s0) and torch.equal(s[:, 4:], want_s1)
    assert bool((pk[n // 2:] == 0x33).all()) and bool((sm[n:] == 0x44).all())
    p, s0, s1 = want_pk, want_s0, want_s1
    o = _u32(out[:n]).cpu().reshape(-1, 16)
    assert torch.equal(o[:, 0:4], p ^ s0) and torch.equal(o[:, 4:8], p ^ s1)
    assert torch.equal(o[:, 8:12], torch.stack([s0[:, 0], s0[:, 1] ^ p[:, 0], s1[:, 2],
                                                s1[:, 3] ^ p[:, 1]], 1))
    assert torch.equal(o[:, 12:16], torch.stack([s1[:, 0] ^ p[:, 2], s0[:, 2], s0[:, 3] ^ p[:, 3],
                                                 s1[:, 1]], 1))
    assert bool((out[n:] == 0x55).all())


def test_fused_arrival_fence_atomics_and_launch_probes():
    """The probes run and do what their header states: the encode pattern's
    bytes with the arrival or the fence, tile counts and the ready word from
    the last arrival (two calls, counters not cleared between them), every
    atomic add counted, and both launch forms."""
    lib = _abi.ceiling_lib()
    tiles = 37
    n = 8192 * tiles
    _say("probes n=%d" % n)
    sh = int(torch.cuda.current_stream().cuda_stream)
    g = torch.Generator().manual_seed(77)
    x = torch.randint(-(1 << 15), 1 << 15, (n,), generator=g, dtype=torch.int32).to(torch.int16).to(DEV)
    pk0 = torch.zeros(n // 2, dtype=torch.uint8, device=DEV)
    sm0 = torch.zeros(n, dtype=torch.uint8, device=DEV)
    assert lib.splitzip_ceiling_encode_shape(x.data_ptr(), n, pk0.data_ptr(), sm0.data_ptr(), sh) == 0
    pk, sm = torch.zeros_like(pk0), torch.zeros_like(sm0)
    counts = torch.full((tiles + 3,), -1, dtype=torch.int32, device=DEV)
    ctrs = torch.full((8 * (1 + (tiles + 15) // 16),), 12345, dtype=torch.int64, device=DEV)
    ready = torch.zeros(4, dtype=torch.int32, device=DEV)
    for epoch in (1, 2):
        assert lib.splitzip_ceiling_encode_arrive(x.data_ptr(), n, pk.data_ptr(), sm.data_ptr(),
                                                  counts.data_ptr(), ctrs.data_ptr(),
                                                  ready.data_ptr(), epoch, sh) == 0
        torch.cuda.synchronize()
        assert int(ready[0].item()) == epoch
    assert torch.equal(pk, pk0) and torch.equal(sm, sm0)
    assert bool(((counts[:tiles] >= 0) & (counts[:tiles] < 256)).all())
    assert bool((counts[tiles:] == -1).all())
    pk.zero_()
    sm.zero_()
    assert lib.splitzip_ceiling_encode_fenced(x.data_ptr(), n, pk.data_ptr(), sm.data_ptr(), sh) == 0
    torch.cuda.synchronize()
    assert torch.equal(pk, pk0) and torch.equal(sm, sm0)
    ac = torch.zeros(8 * 64, dtype=torch.int64, device=DEV)
    assert lib.splitzip_ceiling_atomics(ac.data_ptr(), 100, 7, 3, sh) == 0
    torch.cuda.synchronize()
    a = ac.cpu().reshape(64, 8)
    want = [3 * len(range(k, 100, 7)) for k in range(7)]
    assert a[:7, 0].tolist() == want and int(a[7:].sum()) == 0 and int(a[:, 1:].sum()) == 0
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    for coop in (0, 1):
        assert lib.splitzip_ceiling_launch(coop, 64, sink.data_ptr(), sh) == 0
    torch.cuda.synchronize()
    assert int(sink[0].item()) == 2
    assert lib.splitzip_ceiling_launch(0, 2000, sink.data_ptr(), sh) == _abi.ERR_INVALID
    assert lib.splitzip_ceiling_atomics(ac.data_ptr(), 1, 0, 1, sh) == _abi.ERR_INVALID


@pytest.mark.parametrize("run", [0, 1, 8, 64])
def test_tile_orders_cover_every_tile_once(run):
    """The order probe in any order writes what the plain-order shapes write
    (every tile exactly once), 1,100 tiles: with run 64 the first 1,024
    workgroups take runs of 64 tiles per XCD and the last 76 the plain
    order."""
    lib = _abi.ceiling_lib()
    n = 8192 * 1100
    _say("tile order run=%d n=%d" % (run, n))
    g = torch.Generator().manual_seed(90 + run)
    x = torch.randint(-(1 << 15), 1 << 15, (n,), generator=g, dtype=torch.int32).to(torch.int16).to(DEV)
    sh = int(torch.cuda.current_stream().cuda_stream)
    pk0 = torch.zeros(n // 2, dtype=torch.uint8, device=DEV)
    sm0 = torch.zeros(n, dtype=torch.uint8, device=DEV)
    out0 = torch.zeros(n, dtype=torch.int16, device=DEV)
    assert lib.splitzip_ceiling_encode_shape(x.data_ptr(), n, pk0.data_ptr(), sm0.data_ptr(), sh) == 0
    assert lib.splitzip_ceiling_decode_shape(pk0.data_ptr(), sm0.data_ptr(), out0.data_ptr(), n, sh) == 0
    pk, sm = torch.zeros_like(pk0), torch.zeros_like(sm0)
    out = torch.zeros_like(out0)
    assert lib.splitzip_ceiling_order(0, run, x.data_ptr(), pk.data_ptr(), sm.data_ptr(), 0, n, sh) == 0
    assert lib.splitzip_ceiling_order(1, run, 0, pk.data_ptr(), sm.data_ptr(), out.data_ptr(), n, sh) == 0
    torch.cuda.synchronize()
    assert torch.equal(pk, pk0) and torch.equal(sm, sm0) and torch.equal(out, out0)
