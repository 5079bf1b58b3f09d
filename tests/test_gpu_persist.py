"""Codebook and metadata that went through their JSON form still decode the
payload the GPU wrote; the coverage gate agrees with the GPU codebook."""
import json

import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import persist
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("make,n,passes", [
    (W.gaussian_weight, 300_007, True),
    (W.log_uniform_stress, 200_003, False),
])
def test_json_round_trip_decodes(make, n, passes):
    x = make(n, seed=90).to(DEV)
    ws = S.Workspace(n, DEV)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    host_cb, host_meta = S.read_codebook(cb), S.read_meta(meta)
    assert persist.passes_coverage_gate(host_cb) is passes
    cb_json = json.dumps(persist.codebook_to_json(host_cb))
    meta_json = json.dumps(persist.meta_to_json(host_meta))
    cb2 = persist.codebook_from_json(json.loads(cb_json))
    meta2 = persist.meta_from_json(json.loads(meta_json))
    assert bytes(cb2) == bytes(host_cb)
    # stored form: the first comp_bytes bytes of the payload only
    stored = payload[:meta2.comp_bytes].clone()
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(stored, persist.to_device(meta2, DEV), persist.to_device(cb2, DEV), n,
                   status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("make,n,compressed", [
    (W.gaussian_weight, 3 * 8192 + 11, True),
    (W.log_uniform_stress, 50_001, False),
])
def test_pack_unpack(make, n, compressed):
    x = make(n, seed=91).reshape(-1).to(DEV)
    ws = S.Workspace(n, DEV)
    entry, blob = persist.pack("t", x.reshape(1, -1), ws)
    entry = json.loads(json.dumps(entry))
    assert entry["raw"] is (not compressed)
    if compressed:
        assert blob.numel() == entry["meta"]["comp_bytes"] < 2 * n
    back = persist.unpack(entry, blob)
    torch.cuda.synchronize()
    assert back.shape == (1, n)
    assert torch.equal(back.reshape(-1).view(torch.int16), x.view(torch.int16))


def test_unpack_into_out_and_refusals():
    n = 200_003
    x = W.gaussian_weight(n, seed=92).reshape(-1).to(DEV)
    ws = S.Workspace(n, DEV)
    entry, blob = persist.pack("w", x.reshape(1, -1), ws)
    # into a caller buffer: the same buffer comes back, filled
    out = torch.empty(1, n, dtype=torch.bfloat16, device=DEV)
    res = persist.unpack(entry, blob, out=out)
    torch.cuda.synchronize()
    assert res is out and torch.equal(out.reshape(-1).view(torch.int16), x.view(torch.int16))
    # a strided output would be decoded into a copy: refused
    wide = torch.empty(n, 2, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        persist.unpack(entry, blob, out=wide[:, :1].t())
    # a damaged escape stream is reported, not silently decoded
    e = entry["meta"]["n_esc"]
    assert e > 0
    bad = blob.clone()
    off_cid = entry["meta"]["offsets"][2]
    bad[off_cid: off_cid + 4] = torch.tensor([0xFF, 0xFF, 0xFF, 0x7F], dtype=torch.uint8)
    with pytest.raises(ValueError):
        persist.unpack(entry, bad)
