"""Batched calibrate / encode / decode (one codebook per tensor) through the
C ABI: every item must equal the oracle exactly and equal the single-tensor
calls byte for byte, across batches that need several launches."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
import oracle
import oracle_pins as P
import workloads as W
from test_gpu_parity import DEV, check_codebook, check_meta, host_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def mixed_inputs():
    g = torch.Generator().manual_seed(5)
    rb = torch.randint(-32768, 32768, (9_999,), dtype=torch.int32, generator=g).to(torch.int16)
    return [
        W.gaussian_weight(100_003, seed=50),
        torch.zeros(0, dtype=torch.bfloat16),
        W.log_uniform_stress(8192 * 3 + 1, seed=51),
        W.gaussian_weight(1, seed=52),
        W.subnormal_gaussian(70_001, seed=53),
        rb.view(torch.bfloat16),
        W.kv_layer(seed=2, stream=1, seq=512),
        W.gaussian_weight(1_000_003, seed=54),
        W.gaussian_weight(7, seed=55),
    ]


def run_batch(xs_cpu, status=True):
    xs = [x.reshape(-1).to(DEV) for x in xs_cpu]
    b = S.Batch(xs)
    ws = S.Workspace(0, device=DEV, batch_ns=b.ns)
    b.calibrate(ws)
    b.encode(ws)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    b.decode(status=st if status else None)
    torch.cuda.synchronize()
    return b, int(st.item())


def check_item(b, k, x_cpu):
    xs = host_bits(x_cpu.reshape(-1))
    ocb = oracle.calibrate(xs)
    c = S.read_codebook(b.cbs[k])
    check_codebook(c, ocb)
    opay, om = oracle.encode(xs, ocb)
    m = S.read_meta(b.metas[k])
    check_meta(m, om, ocb)
    assert b.payloads[k][: m.comp_bytes].cpu().numpy().tobytes() == opay, k
    assert np.array_equal(host_bits(b.outs[k]), xs), k


def test_mixed_batch_matches_oracle():
    xs = mixed_inputs()
    b, st = run_batch(xs)
    assert st == 0
    for k, x in enumerate(xs):
        check_item(b, k, x)


def test_batch_equals_single_calls():
    xs = mixed_inputs()
    b, _ = run_batch(xs, status=False)
    for k, x in enumerate(xs):
        n = x.numel()
        xd = x.reshape(-1).to(DEV)
        ws = S.Workspace(n, device=DEV)
        cb = S.calibrate(xd, ws) if n else None
        if n == 0:
            continue
        pay, meta = S.encode(xd, cb, ws)
        torch.cuda.synchronize()
        m = S.read_meta(meta)
        assert bytes(S.read_codebook(cb)) == bytes(S.read_codebook(b.cbs[k]))
        assert bytes(m) == bytes(S.read_meta(b.metas[k]))
        assert torch.equal(pay[: m.comp_bytes], b.payloads[k][: m.comp_bytes])


def test_large_launch_tile_order():
    """A launch of at least 32,768 tiles takes its tiles in runs of 64 per
    XCD, and its last (G mod 512) workgroups in the plain order: 32,821
    encode and decode tiles over items with ragged last tiles, each item
    equal to the oracle and decoded exactly."""
    xs = [W.gaussian_weight((1 << 27) + 12_345, seed=70),
          W.log_uniform_stress(8192 * 37 + 5, seed=71),
          W.gaussian_weight((1 << 27) - 1, seed=72),
          W.gaussian_weight(100_003, seed=73)]
    tiles = sum((x.numel() + 8191) // 8192 for x in xs)
    assert tiles == 32_821 and tiles % 512 == 53
    b, st = run_batch(xs)
    assert st == 0
    for k, x in enumerate(xs):
        check_item(b, k, x)


def test_batch_of_forty_needs_two_launches():
    xs = [W.gaussian_weight(20_000 + 517 * k, seed=60 + k) if k % 3 else
          W.log_uniform_stress(9_000 + 77 * k, seed=60 + k) for k in range(40)]
    b, st = run_batch(xs)
    assert st == 0
    for k in (0, 1, 2, 31, 32, 33, 39):
        check_item(b, k, xs[k])
    for k, x in enumerate(xs):
        assert torch.equal(b.outs[k].view(torch.int16).cpu(), W.bits(x))


def test_batch_decode_flags_bad_item():
    xs = [W.gaussian_weight(50_001, seed=70), W.gaussian_weight(60_001, seed=71)]
    b, st = run_batch(xs)
    assert st == 0
    # break the second item's metadata: its n no longer matches
    m = S.read_meta(b.metas[1])
    m.n = m.n - 1
    b.metas[1].copy_(torch.frombuffer(bytearray(bytes(m)), dtype=torch.uint8).to(DEV))
    st_t = torch.zeros(1, dtype=torch.int32, device=DEV)
    b.outs[0].zero_()
    b.decode(status=st_t)
    torch.cuda.synchronize()
    assert int(st_t.item()) & _abi.DEC_BAD_META
    assert torch.equal(b.outs[0].view(torch.int16).cpu(), W.bits(xs[0]))


def test_batch_workspace_too_small():
    xs = [W.gaussian_weight(3 * 8192, seed=72).to(DEV), W.gaussian_weight(3 * 8192, seed=73).to(DEV)]
    b = S.Batch(xs)
    ws = S.Workspace(3 * 8192, device=DEV)      # sized for one tensor, not both
    b.calibrate(ws)
    rc = _abi.splitzip_encode_batch(b.items, b.count, ws.ptr(), ws.nbytes,
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == _abi.ERR_WORKSPACE
    torch.cuda.synchronize()


def test_workload_kv_stream_batched():
    """The 4 GiB streaming KV cache through the batched calls, as timed by the
    benchmark: every tensor round-trips, obeys the size identities and is
    compared byte for byte with the oracle (codebook, metadata, payload)."""
    xs = [W.kv_cache_tensor(layer, kv, device=DEV).reshape(-1)
          for layer in range(32) for kv in range(2)]
    b = S.Batch(xs)
    ws = S.Workspace(0, device=DEV, batch_ns=b.ns)
    b.calibrate(ws)
    b.encode(ws)
    b.decode()
    torch.cuda.synchronize()
    for k, x in enumerate(xs):
        assert torch.equal(b.outs[k].view(torch.int16), x.view(torch.int16)), k
        m = S.read_meta(b.metas[k])
        c = S.read_codebook(b.cbs[k])
        assert m.status == 0 and m.n_esc == m.n - c.covered
        assert m.comp_bytes == P.closed_form_total(m.n, m.n_esc)
    for k in range(len(xs)):
        xh = host_bits(xs[k])
        ocb = oracle.calibrate(xh)
        opay, om = oracle.encode(xh, ocb)
        check_codebook(S.read_codebook(b.cbs[k]), ocb)
        m = S.read_meta(b.metas[k])
        check_meta(m, om, ocb)
        assert b.payloads[k][: m.comp_bytes].cpu().numpy().tobytes() == opay, k


def test_batch_decode_streams_not_marked_ascending():
    """A batched decode whose items mix streams marked ascending (patched per
    tile) with streams whose metadata lacks the flag (applied by the last
    workgroup of each tensor, in any order), one of them shuffled; no status
    word; twice in a row (the arrival counters carry no state between
    calls)."""
    xs_cpu = [W.log_uniform_stress(8192 * 5 + 3, seed=61), W.gaussian_weight(200_003, seed=62),
              W.log_uniform_stress(50_001, seed=63), W.kv_layer(seed=2, stream=0, seq=256),
              W.log_uniform_stress(8192 * 9, seed=64)]
    xs = [x.reshape(-1).to(DEV) for x in xs_cpu]
    b = S.Batch(xs)
    ws = S.Workspace(0, device=DEV, batch_ns=b.ns)
    b.calibrate(ws)
    b.encode(ws)
    torch.cuda.synchronize()
    flags_at = _abi.Meta.flags.offset
    rng = np.random.default_rng(6)
    for k in (1, 2, 4):
        b.metas[k][flags_at: flags_at + 4] = 0
    # item 2: escape stream in random order
    m = S.read_meta(b.metas[2])
    e = m.n_esc
    assert e > 1000
    pay = b.payloads[2][: m.comp_bytes].cpu().numpy().copy()
    order = rng.permutation(e)
    for sec, width in ((2, 4), (3, 2), (4, 1)):
        at = m.offsets[sec]
        items = pay[at: at + width * e].reshape(e, width)
        pay[at: at + width * e] = items[order].reshape(-1)
    b.payloads[2][: m.comp_bytes] = torch.from_numpy(pay).to(DEV)
    for rep in range(2):
        for o in b.outs:
            o.fill_(0)
        b.decode(status=None)
        torch.cuda.synchronize()
        for k, x in enumerate(xs):
            assert torch.equal(b.outs[k].view(torch.int16), x.view(torch.int16)), (rep, k)


def test_fit_payloads_sizes_each_buffer_exactly():
    """Batch.fit_payloads after a calibrate: every payload buffer is exactly
    its payload's length (n_esc = total - covered under the tensor's own
    codebook), the encode fits with status 0 and the round trip is bit for
    bit; a codebook calibrated on a tensor of another length keeps the
    all-escape bound."""
    xs = [W.gaussian_weight(1_000_003, seed=71, device=DEV),
          W.log_uniform_stress(77_777, seed=72, device=DEV),
          W.kv_cache_tensor(3, 1, device=DEV).reshape(-1)[: 3 * 8192 + 5].contiguous()]
    b = S.Batch(xs, capacities=[16] * len(xs))
    ws = S.Workspace(max(b.ns), device=DEV, batch_ns=b.ns)
    b.calibrate(ws)
    b.fit_payloads()
    b.encode(ws)
    b.decode()
    torch.cuda.synchronize()
    for k, x in enumerate(xs):
        m = S.read_meta(b.metas[k])
        c = S.read_codebook(b.cbs[k])
        assert m.status == 0
        assert m.n_esc == c.total - c.covered
        assert b.payloads[k].numel() == max(m.comp_bytes, 16)
        assert torch.equal(b.outs[k].view(torch.int16), x.view(torch.int16))
    # tensor 1 given tensor 0's codebook (another length): the bound stays
    b.cbs[1].copy_(b.cbs[0])
    b.fit_payloads()
    assert b.payloads[1].numel() == S.payload_size(b.ns[1], b.ns[1])


def test_payload_for_is_the_payload_length():
    """payload_for after a calibrate on the same tensor: the encode fits a
    buffer of exactly comp_bytes and decodes bit for bit."""
    x = W.kv_cache_tensor(5, 0, device=DEV).reshape(-1)[: 40 * 8192 + 3].contiguous()
    ws = S.Workspace(x.numel(), device=DEV)
    cb = S.calibrate(x, ws)
    buf = S.payload_for(cb, x.numel())
    pay, meta = S.encode(x, cb, ws, payload=buf)
    m = S.read_meta(meta)
    assert m.status == 0 and buf.numel() == max(m.comp_bytes, 16)
    out = S.decode(pay, meta, cb, x.numel())
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
