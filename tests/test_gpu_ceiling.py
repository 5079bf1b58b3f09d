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
