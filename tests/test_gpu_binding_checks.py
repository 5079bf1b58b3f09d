"""The Python binding refuses buffers the kernels would overrun (too small,
non-contiguous, wrong status type) before anything is launched, and sizes
every raw buffer in bytes whatever its dtype."""
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


def _tensor(n=50_001):
    return W.gaussian_weight(n, seed=41).to(DEV)


def test_small_or_strided_buffers_are_refused():
    _say("binding checks")
    x = _tensor()
    ws = S.Workspace(x.numel(), DEV)
    with pytest.raises(ValueError):
        S.calibrate(x, ws, cb=torch.empty(100, dtype=torch.uint8, device=DEV))
    cb = S.calibrate(x, ws)
    with pytest.raises(ValueError):
        S.encode(x, cb[:1000], ws)
    with pytest.raises(ValueError):
        S.encode(x, cb, ws, meta=torch.empty(64, dtype=torch.uint8, device=DEV))
    strided = torch.empty(2 * S.codec.META_BYTES, dtype=torch.uint8, device=DEV)[::2]
    with pytest.raises(ValueError):
        S.encode(x, cb, ws, meta=strided)
    payload, meta = S.encode(x, cb, ws)
    n = x.numel()
    with pytest.raises(ValueError):
        S.decode(payload, meta[:50], cb, n)
    with pytest.raises(ValueError):
        S.decode(payload, meta, cb[:20], n)
    with pytest.raises(ValueError):
        S.decode(payload, meta, cb, n, status=torch.zeros(1, dtype=torch.int64, device=DEV))
    with pytest.raises(ValueError):
        S.decode(payload[::2], meta, cb, n)
    # nothing was launched by the refused calls: the good ones still agree
    out = S.decode(payload, meta, cb, n)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


def test_buffers_of_other_dtypes_are_sized_in_bytes():
    x = _tensor(70_003)
    n = x.numel()
    ws = S.Workspace(n, DEV)
    cb = S.calibrate(x, ws, cb=torch.empty(S.codec.CODEBOOK_BYTES // 8, dtype=torch.int64,
                                           device=DEV))
    cap = S.payload_size(n, n)
    payload = torch.zeros((cap + 3) // 4, dtype=torch.int32, device=DEV)
    meta = torch.zeros(S.codec.META_BYTES // 8, dtype=torch.float64, device=DEV)
    S.encode(x, cb, ws, payload=payload, meta=meta)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=st)
    torch.cuda.synchronize()
    m = S.read_meta(meta.view(torch.uint8))
    assert m.status == 0 and int(st.item()) == 0
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
