"""splitzip_encode_noalloc (no workspace argument: the library's own device
scratch) through the C ABI, byte for byte against splitzip_encode with a
caller workspace and against the oracle, on two calls in a row, the second
with a smaller input; sizes above its limit are refused before anything is
enqueued."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
import oracle
import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _encode_both(x):
    """(no-alloc payload, meta), (workspace payload, meta) for one tensor."""
    n = x.numel()
    xb = x.reshape(-1).view(torch.int16)
    ws = S.Workspace(n, device=DEV)
    cb = S.calibrate(x, ws)
    cap = S.payload_size(n, n) + 64
    outs = []
    for noalloc in (True, False):
        pay = torch.full((cap,), 0xA5, dtype=torch.uint8, device=DEV)
        meta = torch.zeros(S.codec.META_BYTES, dtype=torch.uint8, device=DEV)
        if noalloc:
            rc = _abi.splitzip_encode_noalloc(xb.data_ptr(), n, cb.data_ptr(), pay.data_ptr(), cap,
                                              meta.data_ptr(), _stream())
        else:
            rc = _abi.splitzip_encode(xb.data_ptr(), n, cb.data_ptr(), pay.data_ptr(), cap,
                                      meta.data_ptr(), ws.ptr(), ws.nbytes, _stream())
        assert rc == 0, _abi.status_string(rc)
        outs.append((pay, meta))
    torch.cuda.synchronize()
    return cb, outs


@pytest.mark.parametrize("first,second", [
    (lambda: W.kv_cache_tensor(2, 1).reshape(-1), lambda: W.gaussian_weight(1_000_003, seed=90)),
    (lambda: W.log_uniform_stress(3_000_001, seed=91), lambda: W.log_uniform_stress(8193, seed=92)),
])
def test_noalloc_matches_workspace_encode(first, second):
    for make in (first, second):          # the second call is smaller
        x_cpu = make()
        n = x_cpu.numel()
        print("no-alloc encode n=%d" % n, flush=True)
        cb, ((pa, ma), (pw, mw)) = _encode_both(x_cpu.to(DEV))
        m = S.read_meta(ma)
        assert m.status == 0
        assert torch.equal(ma, mw)
        assert torch.equal(pa, pw)        # payload and the untouched bytes after it
        xs = W.bits(x_cpu).numpy().view(np.uint16)
        opay, om = oracle.encode(xs, oracle.calibrate(xs))
        assert (m.n_esc, m.comp_bytes) == (om.n_esc, om.comp_bytes)
        assert pa[: m.comp_bytes].cpu().numpy().tobytes() == opay
        out = S.decode(pa, ma, cb, n)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), x_cpu.to(DEV).reshape(-1).view(torch.int16))


def test_noalloc_refuses_sizes_above_its_limit():
    x = torch.zeros(16, dtype=torch.int16, device=DEV)
    cb = torch.zeros(S.codec.CODEBOOK_BYTES, dtype=torch.uint8, device=DEV)
    meta = torch.zeros(S.codec.META_BYTES, dtype=torch.uint8, device=DEV)
    pay = torch.zeros(64, dtype=torch.uint8, device=DEV)
    n = _abi.NOALLOC_MAX_N + 1
    # the pointers are never read: the size is refused before any launch
    rc = _abi.splitzip_encode_noalloc(x.data_ptr(), n, cb.data_ptr(), pay.data_ptr(),
                                      S.payload_size(n, n), meta.data_ptr(), _stream())
    assert rc == _abi.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(meta.sum().item()) == 0
