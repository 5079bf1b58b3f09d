"""The seeded input generator: SplitMix64 against its published first outputs
(state 0), determinism, and the shapes/statistics of the workloads."""
import torch

import workloads as W


def test_splitmix64_published_sequence():
    # SplitMix64 from state 0 (Steele, Lea & Flood 2014; the reference
    # generator distributed with xoshiro): first four outputs
    want = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    got = W.splitmix64(torch.arange(0, 4, dtype=torch.int64), 0)
    assert [int(v) & W._M64 for v in got] == want
    state = 0
    for w in want:
        state += W._GOLDEN
        assert W.splitmix64_scalar(state) == w


def test_deterministic_and_seeded():
    a = W.gaussian_weight(10001, seed=0)
    b = W.gaussian_weight(10001, seed=0)
    c = W.gaussian_weight(10001, seed=1)
    assert torch.equal(W.bits(a), W.bits(b)) and not torch.equal(W.bits(a), W.bits(c))
    assert W.checksum(a) == W.checksum(b) != W.checksum(c)


def test_shapes_and_statistics():
    x = W.gaussian_weight(200_003, seed=0)
    assert x.dtype == torch.bfloat16 and x.numel() == 200_003
    assert abs(float(x.float().std()) - 0.02) < 5e-4
    kv = W.kv_layer(seed=2, stream=0, seq=256)
    assert kv.shape == (1, 8, 256, 128)
    per_chan = kv.float().abs().mean(dim=(0, 2))  # [heads, head_dim]
    assert int((per_chan > 10).sum()) == 8 * 4       # 4 outlier channels per head
    s = W.log_uniform_stress(1 << 16, seed=3, stream=0)
    f = s.float()
    assert 0.005 < float((f == 0).float().mean()) < 0.02
    assert 0.0003 < float(torch.isinf(f).float().mean()) < 0.003
    sub = W.subnormal_gaussian(1 << 16, seed=3, stream=1)
    exp = (W.bits(sub).to(torch.int32) >> 7) & 0xFF
    assert int(exp.max()) == 0
    w = W.weight_with_outliers(rows=64, cols=3072, seed=4)
    assert w.shape == (64, 3072)
    t = W.kv_cache_tensor(layer=1, kv=1, seq=64)
    assert t.shape == (1, 8, 64, 128)
