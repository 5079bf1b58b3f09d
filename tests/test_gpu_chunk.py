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
    """2^28 + 5 elements: 32,769 encode tiles, 1,025 placement workgroups of
    32 tiles, so the placement first sums the counts per workgroup and per
    superblock (read directly, the counts would cost 33.6M loads).  Escapes
    are planted every 997 elements on top of N(0, 0.02) values."""
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


def test_two_billion_element_tensor_sampled_against_oracle():
    """n = 2^31 + 5 (4 GiB of bf16, element indices past int32) in one call:
    the codebook equals the oracle's over the whole tensor, the escape count
    and payload size obey their identities, the decode round-trips, and four
    2^20-element windows of the payload (chunk aligned, the last one near the
    end) equal what the oracle encodes for those windows with the same
    codebook: the dense bytes at their offsets and the escapes with chunk ids
    shifted by the window start."""
    n = (1 << 31) + 5
    _say("2G tensor n=%d" % n)
    x = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    step = 1 << 27
    for s0 in range(0, n, step):   # N(0, 0.02), generated in slices to bound memory
        m0 = min(step, n - s0)
        x[s0: s0 + m0] = W.to_bf16(0.02 * W.normal(m0, 610, 0, DEV, start=s0))
    xv = x.view(torch.int16)
    k = torch.arange(0, n, 4099, device=DEV)
    xv[k] = ((((k >> 3) % 40) + 150) << 7).to(torch.int16)     # planted escapes
    xv[n - 4] = 200 << 7                                          # and past index 2^31
    xv[n - 1] = -(0x8000 - (201 << 7) - 5)                        # sign set, mantissa 5
    del k
    torch.cuda.empty_cache()
    ws = S.Workspace(n, DEV)
    cb = S.calibrate(x, ws)
    cap = S.payload_size(n, n // 1000)
    payload, meta = S.encode(x, cb, ws, payload=torch.empty(cap, dtype=torch.uint8, device=DEV))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(out.view(torch.int16), xv)
    del out, ws
    m = S.read_meta(meta)
    c = S.read_codebook(cb)
    assert m.status == 0 and m.n_esc == n - c.covered and m.n_esc > 500_000
    assert m.comp_bytes == S.payload_size(n, m.n_esc)
    xs = xv.cpu().numpy().view(np.uint16)
    ocb = oracle.calibrate(xs)
    check_codebook(c, ocb)
    off = [int(v) for v in m.offsets]
    e = m.n_esc
    esc_cid = payload[off[2]: off[2] + 4 * e].cpu().numpy().view("<i4").astype(np.int64)
    esc_pos = payload[off[3]: off[3] + 2 * e].cpu().numpy().view("<u2").astype(np.int64)
    esc_ev = payload[off[4]: off[4] + e].cpu().numpy()
    esc_idx = esc_cid * 1024 + esc_pos
    assert np.all(np.diff(esc_idx) > 0)
    assert esc_idx[-1] == n - 1 and esc_idx[-2] == n - 4
    win = 1 << 20
    for start, end in ((0, win), (1 << 30, (1 << 30) + win),
                       (1024 * 1_900_001, 1024 * 1_900_001 + win), ((1 << 31) - win, n)):
        _say("2G tensor window [%d, %d)" % (start, end))
        opay, om = oracle.encode(xs[start: end], ocb)
        assert payload[start // 2: (end + 1) // 2].cpu().numpy().tobytes() == \
            opay[: om.n_pairs]
        assert payload[off[1] + start: off[1] + end].cpu().numpy().tobytes() == \
            opay[om.offsets[1]: om.offsets[1] + end - start]
        sel = (esc_idx >= start) & (esc_idx < end)
        ocid = np.frombuffer(opay, "<i4", om.n_esc, om.offsets[2]).astype(np.int64)
        opos = np.frombuffer(opay, "<u2", om.n_esc, om.offsets[3]).astype(np.int64)
        oev = np.frombuffer(opay, np.uint8, om.n_esc, om.offsets[4])
        assert int(sel.sum()) == om.n_esc > 0
        assert np.array_equal(esc_idx[sel] - start, ocid * 1024 + opos)
        assert np.array_equal(esc_ev[sel], oev)
