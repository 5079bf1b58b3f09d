"""The C ABI driven from a plain C program (tests/c_smoke): calibrate,
encode with a chunk size, validating decode and in-place decode, run as a
child process; its codebook, metadata and payload must equal the oracle's
byte for byte and both decoded copies must equal the input."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

from lossless_bf16_tensor_splitzip_amd import _abi
import oracle
import workloads as W
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_smoke", "_build",
                   "splitzip_c_smoke")


def setup_module(module):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("make,n,chunk", [
    (W.gaussian_weight, 1_000_003, 1024),
    (W.log_uniform_stress, 300_001, 1000),
    (W.kv_cache_tensor, None, 4096),
])
def test_c_driver(tmp_path, make, n, chunk):
    assert os.path.exists(EXE), "C driver not built (run __graft_entry__.build())"
    x = (make(3, 0) if n is None else make(n, seed=77)).reshape(-1)
    xs = W.bits(x).numpy().view(np.uint16)
    n = xs.size
    inp = tmp_path / "x.bin"
    xs.tofile(inp)
    prefix = str(tmp_path / "res")
    _say("C driver n=%d chunk=%d" % (n, chunk))
    res = subprocess.run([EXE, str(inp), str(n), str(chunk), prefix], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    cb = _abi.Codebook.from_buffer_copy(open(prefix + ".cb", "rb").read())
    meta = _abi.Meta.from_buffer_copy(open(prefix + ".meta", "rb").read())
    payload = open(prefix + ".payload", "rb").read()
    ocb = oracle.calibrate(xs)
    opay, om = oracle.encode(xs, ocb, chunk)
    assert bytes(cb.dec_lut) == ocb.dec_lut.tobytes()
    assert bytes(cb.enc_lut_marked) == ocb.enc_lut_marked.tobytes()
    assert (cb.n_codes, cb.covered, cb.total) == (ocb.n_codes, ocb.covered, ocb.total)
    assert (meta.n, meta.n_esc, meta.comp_bytes, meta.chunk_size) == (n, om.n_esc, om.comp_bytes,
                                                                      chunk)
    assert tuple(meta.offsets) == tuple(om.offsets)
    assert payload == opay
    assert np.array_equal(np.fromfile(prefix + ".out", np.uint16), xs)
    assert np.array_equal(np.fromfile(prefix + ".slot", np.uint16), xs)
