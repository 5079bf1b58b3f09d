"""Escape streams with other chunk sizes (page 1, encode, parameter
chunk_size) and single tensors large enough that escape placement sums the
tile counts per placement workgroup first: byte for byte against the oracle."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
import oracle
import workloads as W
from test_gpu_parity import DEV, _say, check_codebook, check_meta, host_bits, workspace

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def chunk_case(x_cpu, chunk, name):
    x = x_cpu.reshape(-1).to(DEV)
    n = x.numel()
    _say("chunk case %s n=%d chunk=%d" % (name, n, chunk))
    ws = workspace(n)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws, chunk_size=chunk)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=st)
    fast = S.decode(payload, meta, cb, n)
    torch.cuda.synchronize()
    xs = host_bits(x_cpu.reshape(-1))
    ocb = oracle.calibrate(xs)
    opay, om = oracle.encode(xs, ocb, chunk)
    m = S.read_meta(meta)
    check_codebook(S.read_codebook(cb), ocb)
    check_meta(m, om, ocb)
    assert m.chunk_size == chunk
    assert payload[: m.comp_bytes].cpu().numpy().tobytes() == opay
    assert int(st.item()) == 0
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
    assert torch.equal(fast.view(torch.int16), x.view(torch.int16))
    # in place, from the head of the output buffer
    slot = torch.zeros(max(2 * n, m.comp_bytes, S.payload_size(n, 0)), dtype=torch.uint8,
                       device=DEV)
    slot[: m.comp_bytes].copy_(payload[: m.comp_bytes])
    stash = torch.empty(max(m.comp_bytes, 16), dtype=torch.uint8, device=DEV)
    st.zero_()
    res = S.decode_slot(slot, meta, cb, n, stash, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(res.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("chunk", [1, 7, 1000, 1024, 4096, 8192, 12345, 65536])
def test_chunk_sizes_escape_heavy(chunk):
    chunk_case(W.log_uniform_stress(3 * 8192 + 77, seed=600), chunk, "escape heavy")


@pytest.mark.parametrize("chunk", [1, 333, 2048, 65536])
def test_chunk_sizes_weight(chunk):
    chunk_case(W.gaussian_weight(1_000_003, seed=601), chunk, "weight")


def test_large_single_tensor_summed_placement():
    """2^28 + 5 elements: 32,769 encode tiles, 129 placement workgroups, so
    the placement first sums the counts per workgroup.  Escapes are planted
    every 997 elements on top of N(0, 0.02) values."""
    n = (1 << 28) + 5
    b = host_bits(W.gaussian_weight(n, seed=602)).copy()
    k = np.arange(0, n, 997)
    b[k] = ((k & 1) << 15) | ((150 + (k // 997) % 40) << 7) | (k & 0x7F)
    xs = b
    x_cpu = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    _say("large single tensor n=%d" % n)
    x = x_cpu.to(DEV)
    ws = S.Workspace(n, DEV)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    out = S.decode(payload, meta, cb, n)
    torch.cuda.synchronize()
    m = S.read_meta(meta)
    ocb = oracle.calibrate(xs)
    check_codebook(S.read_codebook(cb), ocb)
    opay, om = oracle.encode(xs, ocb)
    check_meta(m, om, ocb)
    assert om.n_esc > 200_000
    got = payload[: m.comp_bytes].cpu().numpy().tobytes()
    assert got == opay
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
