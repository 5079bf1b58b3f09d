"""Decoding damaged payloads: random bytes of a valid payload are changed
(dense sections and escape stream alike).  The validating GPU decode must
flag exactly the payloads the oracle rejects, and decode the ones it accepts
to the oracle's output; the plain decode must stay inside its output (the
bytes around it are checked) whatever the stream holds."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
import oracle
import workloads as W
from test_gpu_parity import DEV, _say, host_bits, meta_to_device

pytestmark = pytest.mark.gpu

GUARD = 4096


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.mark.parametrize("seed", range(24))
def test_damaged_payload(seed):
    key = W.stream_key(1700 + seed, 0)
    u = W.uniform(torch.arange(16, dtype=torch.int64), key).numpy()
    n = 20_000 + int(u[0] * 60_000)
    x = W.log_uniform_stress(n, seed=seed, lo_exp=-20.0, hi_exp=-20.0 + 24 * u[1])
    xs = host_bits(x)
    ocb = oracle.calibrate(xs)
    opay, om = oracle.encode(xs, ocb)
    buf = bytearray(opay)
    esc_lo = om.offsets[2]
    k = 1 + int(u[2] * 5)
    for j in range(k):
        # half of the changes land in the escape sections
        if u[3 + j] < 0.5 and om.comp_bytes > esc_lo:
            at = esc_lo + int(u[8 + j] * (om.comp_bytes - esc_lo))
        else:
            at = int(u[8 + j] * om.comp_bytes)
        buf[min(at, om.comp_bytes - 1)] ^= 1 + int(u[13] * 254)
    rc, want = oracle.decode_status(bytes(buf), om, ocb.dec_lut, validate=True)
    _say("damaged seed=%d n=%d changes=%d oracle=%d" % (seed, n, k, rc))

    pay = torch.frombuffer(bytearray(bytes(buf) + b"\0" * 16), dtype=torch.uint8).to(DEV)
    meta = meta_to_device(om)
    lut = torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV)
    # output with guard zones on both sides
    big = torch.full((n + 2 * GUARD,), 0x5A5A, dtype=torch.int16, device=DEV)
    out = big[GUARD: GUARD + n].view(torch.bfloat16)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    S.decode(pay[: len(buf)], meta, lut, n, out=out, status=st)
    torch.cuda.synchronize()
    status = int(st.item())
    assert (status != 0) == (rc != oracle.OK), (status, rc)
    if rc == oracle.OK:
        assert np.array_equal(host_bits(out.cpu()), want)
    # plain decode of the same bytes: never outside out[0, n)
    big.fill_(0x5A5A)
    S.decode(pay[: len(buf)], meta, lut, n, out=out)
    torch.cuda.synchronize()
    g = big.cpu().numpy()
    assert (g[:GUARD] == 0x5A5A).all() and (g[GUARD + n:] == 0x5A5A).all()
