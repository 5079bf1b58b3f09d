"""The workspace carries no state between calls: junk written over it from
the host (standing in for an interrupted call, another process's leftovers
or a stray write) does not change what calibrate and encode produce, which
must equal the oracle byte for byte."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
import oracle
import workloads as W
from test_gpu_parity import DEV, _say, check_codebook, host_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("fill", ["random", "ones", "zeros_then_random"])
def test_junk_workspace(fill):
    xs_cpu = [W.gaussian_weight(1 << 20, seed=71), W.log_uniform_stress(300_001, seed=72),
              W.kv_cache_tensor(1, 0).reshape(-1)]          # 2^20: one counter; 2^25: two levels
    ws = S.Workspace(max(x.numel() for x in xs_cpu), device=DEV)
    g = torch.Generator().manual_seed(len(fill))
    for rep in range(3):
        if fill == "ones" or (fill == "zeros_then_random" and rep == 0):
            ws.buf.fill_(0xFF if fill == "ones" else 0)
        else:
            ws.buf.copy_(torch.randint(0, 256, (ws.nbytes,), dtype=torch.uint8, generator=g))
        for x_cpu in xs_cpu:
            _say("junk workspace %s rep %d n=%d" % (fill, rep, x_cpu.numel()))
            x = x_cpu.to(DEV)
            cb = S.calibrate(x, ws)
            payload, meta = S.encode(x, cb, ws)
            torch.cuda.synchronize()
            xs = host_bits(x_cpu)
            ocb = oracle.calibrate(xs)
            check_codebook(S.read_codebook(cb), ocb)
            opay, om = oracle.encode(xs, ocb)
            m = S.read_meta(meta)
            assert m.status == 0 and m.comp_bytes == om.comp_bytes
            assert payload[: m.comp_bytes].cpu().numpy().tobytes() == opay


def test_batched_calibrate_over_junk():
    xs = [W.gaussian_weight(n, seed=80 + k).to(DEV) for k, n in
          enumerate([1, 4097, 1 << 20, 3 << 20, 33554432 // 4])]
    b = S.Batch(xs)
    ws = S.Workspace(0, device=DEV, batch_ns=b.ns)
    g = torch.Generator().manual_seed(9)
    for rep in range(2):
        ws.buf.copy_(torch.randint(0, 256, (ws.nbytes,), dtype=torch.uint8, generator=g))
        b.calibrate(ws)
        torch.cuda.synchronize()
        for k, x in enumerate(xs):
            check_codebook(S.read_codebook(b.cbs[k]), oracle.calibrate(host_bits(x.cpu())))
