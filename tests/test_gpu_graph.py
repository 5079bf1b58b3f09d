"""The codec inside a captured HIP graph (no allocation, synchronisation or
memset nodes: every call is kernels only), replayed several times with eager
work in between, and two streams with their own workspaces running at once.
Every replay and every stream is checked against eager results."""
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
import workloads as W
from test_gpu_parity import DEV, _say

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def eager(x, ws):
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    out = S.decode(payload, meta, cb, x.numel())
    torch.cuda.synchronize()
    m = S.read_meta(meta)
    return cb.clone(), payload[: m.comp_bytes].clone(), meta.clone(), out


@pytest.mark.parametrize("n", [1_000_003, 8 * 32768 * 128])
def test_graph_replays(n):
    _say("graph case n=%d" % n)
    inputs = [W.gaussian_weight(n, seed=800 + k, device=DEV) for k in range(3)]
    inputs[2] = W.log_uniform_stress(n, seed=803, device=DEV)    # many escapes
    ws = S.Workspace(n, DEV)
    refs = [eager(x, ws) for x in inputs]

    x = inputs[0].clone()
    cb = torch.empty_like(refs[0][0])
    payload = torch.empty(S.payload_size(n, n), dtype=torch.uint8, device=DEV)
    meta = torch.empty_like(refs[0][2])
    out = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.calibrate(x, ws, cb=cb)
        S.encode(x, cb, ws, payload=payload, meta=meta)
        S.decode(payload, meta, cb, n, out=out, status=status)
    for rep in range(6):
        k = rep % 3
        # eager work between the replays: new input, scrambled outputs
        x.copy_(inputs[k])
        out.fill_(0)
        payload[:1024].fill_(0xFF)
        status.zero_()
        g.replay()
        torch.cuda.synchronize()
        ref_cb, ref_pay, ref_meta, ref_out = refs[k]
        assert torch.equal(cb, ref_cb), rep
        assert torch.equal(meta, ref_meta), rep
        assert torch.equal(payload[: ref_pay.numel()], ref_pay), rep
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(out.view(torch.int16), inputs[k].view(torch.int16)), rep
        assert int(status.item()) == 0


def test_two_streams_own_workspaces():
    n = 4_000_037
    xs = [W.gaussian_weight(n, seed=810, device=DEV), W.log_uniform_stress(n, seed=811, device=DEV)]
    refs = []
    for x in xs:
        ws = S.Workspace(n, DEV)
        refs.append(eager(x, ws))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [S.Workspace(n, DEV, stream=st) for st in streams]
    torch.cuda.synchronize()
    res = [None, None]
    for rep in range(3):
        for k in range(2):
            with torch.cuda.stream(streams[k]):
                cb = S.calibrate(xs[k], wss[k])
                payload, meta = S.encode(xs[k], cb, wss[k])
                out = S.decode(payload, meta, cb, n)
                res[k] = (cb, payload, meta, out)
        torch.cuda.synchronize()
        for k in range(2):
            cb, payload, meta, out = res[k]
            ref_cb, ref_pay, ref_meta, ref_out = refs[k]
            assert torch.equal(cb, ref_cb) and torch.equal(meta, ref_meta), (rep, k)
            assert torch.equal(payload[: ref_pay.numel()], ref_pay), (rep, k)
            assert torch.equal(out.view(torch.int16), xs[k].view(torch.int16)), (rep, k)


@pytest.mark.parametrize("resident", [False, True])
def test_graph_replays_slot_decode(resident):
    """A group of two in-place decodes captured in a graph (multi-pass or
    resident form: the resident barrier's counters are put back by each
    launch, so every replay starts clean), replayed six times over three
    different payloads copied into the slot heads between the replays."""
    n = 5 * 8192 + 777
    _say("graph slot decode resident=%s" % resident)
    inputs = [W.gaussian_weight(n, seed=820, device=DEV), W.log_uniform_stress(n, seed=821, device=DEV),
              W.gaussian_weight(n, seed=822, device=DEV)]
    ws = S.Workspace(n, DEV)
    refs = [eager(x, ws) for x in inputs]     # (cb, payload, meta, out)
    comp_max = max(r[1].numel() for r in refs)
    slots = [torch.empty(max(2 * n, comp_max), dtype=torch.uint8, device=DEV) for _ in range(2)]
    stashes = [torch.empty(comp_max, dtype=torch.uint8, device=DEV) for _ in range(2)]
    cbs = [torch.empty_like(refs[0][0]) for _ in range(2)]
    metas = [torch.empty_like(refs[0][2]) for _ in range(2)]

    def load(j, k):
        """payload k into slot j (the rest of the slot scrambled), with its
        codebook and metadata"""
        slots[j].fill_(0xA5)
        slots[j][: refs[k][1].numel()].copy_(refs[k][1])
        cbs[j].copy_(refs[k][0])
        metas[j].copy_(refs[k][2])

    # one eager call first (the library caches its device queries)
    load(0, 0)
    load(1, 1)
    S.decode_slots(slots, metas, cbs, [n, n], stashes, resident=resident)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        S.decode_slots(slots, metas, cbs, [n, n], stashes, resident=resident)
    for rep in range(6):
        ks = (rep % 3, (rep + 1) % 3)
        load(0, ks[0])
        load(1, ks[1])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, k in enumerate(ks):
            got = slots[j][: 2 * n].view(torch.bfloat16)
            assert torch.equal(got.view(torch.int16), inputs[k].reshape(-1).view(torch.int16)), (rep, j)
