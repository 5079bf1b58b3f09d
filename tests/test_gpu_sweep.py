"""A seeded sweep of sizes, value distributions, chunk sizes and foreign
codebooks: every case byte for byte against the oracle (codebook, metadata,
payload) and decoded back plainly, with validation and in place."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
import oracle
import workloads as W
from test_gpu_parity import DEV, _say, check_codebook, check_meta, host_bits, workspace

pytestmark = pytest.mark.gpu

CASES = 40


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


def make_case(seed):
    """(input, codebook source or None, chunk size) for one seed; all drawn
    from the seeded counter generator, so the case is the same everywhere."""
    key = W.stream_key(900 + seed, 0)
    u = W.uniform(torch.arange(8, dtype=torch.int64), key).tolist()
    n = int(round(10 ** (u[0] * 6.5)))            # 1 .. ~3.2M, log-uniform
    kind = int(u[1] * 5)
    if kind == 0:
        x = W.gaussian_weight(n, seed=seed, sigma=10 ** (-4 + 6 * u[2]))
    elif kind == 1:
        lo = -133 + 100 * u[2]
        x = W.log_uniform_stress(n, seed=seed, lo_exp=lo, hi_exp=lo + 1 + 40 * u[3])
    elif kind == 2:
        x = W.weight_with_outliers(1, n, seed=seed, p_outlier=0.01 * u[2], scale=10 + 1e4 * u[3])
    elif kind == 3:
        x = W.subnormal_gaussian(n, seed=seed)
    else:
        # mostly one value with sparse others (constant runs, extreme codes)
        b = np.full(n, 0x3F80, np.uint16)
        k = np.arange(0, n, max(1, int(1 + 5000 * u[2])))
        b[k] = (k * 2654435761 & 0xFFFF).astype(np.uint16)
        x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    chunk = 1024
    if u[4] < 0.15:
        chunk = 1 << int(u[5] * 17)                 # 1 .. 65536
    elif u[4] < 0.35:
        chunk = 1 + int(u[5] * 65535)
    while (n + chunk - 1) // chunk > (1 << 31):
        chunk *= 2
    src = None
    if u[6] < 0.1:
        src = W.gaussian_weight(max(1, n // 3), seed=seed + 1000)   # foreign codebook
    return x.reshape(-1), src, chunk


@pytest.mark.parametrize("seed", range(CASES))
def test_sweep_case(seed):
    x_cpu, src_cpu, chunk = make_case(seed)
    n = x_cpu.numel()
    _say("sweep seed=%d n=%d chunk=%d foreign=%s" % (seed, n, chunk, src_cpu is not None))
    x = x_cpu.to(DEV)
    src = x if src_cpu is None else src_cpu.to(DEV)
    ws = workspace(max(n, src.numel()))
    cb = S.calibrate(src, ws)
    payload, meta = S.encode(x, cb, ws, chunk_size=chunk)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(payload, meta, cb, n, status=st)
    fast = S.decode(payload, meta, cb, n)
    torch.cuda.synchronize()
    xs = host_bits(x_cpu)
    ocb = oracle.calibrate(host_bits(src_cpu) if src_cpu is not None else xs)
    check_codebook(S.read_codebook(cb), ocb)
    opay, om = oracle.encode(xs, ocb, chunk)
    m = S.read_meta(meta)
    check_meta(m, om, ocb)
    assert payload[: m.comp_bytes].cpu().numpy().tobytes() == opay
    assert int(st.item()) == 0
    assert np.array_equal(host_bits(out.cpu()), xs)
    assert np.array_equal(host_bits(fast.cpu()), xs)
    # in place
    slot = torch.zeros(max(2 * n, m.comp_bytes, S.payload_size(n, 0)), dtype=torch.uint8,
                       device=DEV)
    slot[: m.comp_bytes].copy_(payload[: m.comp_bytes])
    stash = torch.empty(max(m.comp_bytes, 16), dtype=torch.uint8, device=DEV)
    res = S.decode_slot(slot, meta, cb, n, stash)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(res.cpu()), xs)
