"""Seeded synthetic BF16 inputs shared by the tests, the smoke check and the
benchmark.

This module holds no codec arithmetic: it only draws numbers.  Both the HIP
library and the CPU oracle consume the very bytes it returns (generated once,
then copied to wherever each side needs them).

Generator (counter-based, one value per element index):
  * SplitMix64 (Steele, Lea & Flood, "Fast splittable pseudorandom number
    generators", OOPSLA 2014): output k of a stream keyed by ``key`` is
    mix(key + (k + 1) * 0x9E3779B97F4A7C15) with the published finaliser
    constants.  ``key`` = SplitMix64 output 0 of seed (seed << 32 | stream).
  * uniform in (0, 1): (top 53 bits + 0.5) * 2**-53, in float64.
  * standard normal: Box-Muller, cosine branch, from two counters per index.
  * rounding: float64 -> float32 -> bfloat16, both round-to-nearest-even
    (torch's conversions), so no value passes through fast-math or FTZ.

The workloads stand in for the pages' data (LLM KV activations and diffusers
linear weights, which are not available): a weight-like N(0, 0.02) tensor, a
KV-cache layer with outlier channels, escape-heavy and subnormal-heavy stress
tensors, a large linear weight with rare outliers, and a 32-layer streaming KV
cache.
"""
from __future__ import annotations

import math

import torch

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def _signed(v: int) -> int:
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


def splitmix64_scalar(state: int) -> int:
    """One SplitMix64 step on a Python int (state already advanced)."""
    z = state & _M64
    z = ((z ^ (z >> 30)) * _MIX1) & _M64
    z = ((z ^ (z >> 27)) * _MIX2) & _M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return splitmix64_scalar(((seed << 32) | (stream & 0xFFFFFFFF)) + _GOLDEN)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    # logical right shift of an int64 tensor (torch's >> is arithmetic)
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(counter: torch.Tensor, key: int) -> torch.Tensor:
    """Vectorised SplitMix64 output for int64 counters (wrapping arithmetic)."""
    z = counter * _signed(_GOLDEN) + _signed(key + _GOLDEN)
    z = (z ^ _lsr(z, 30)) * _signed(_MIX1)
    z = (z ^ _lsr(z, 27)) * _signed(_MIX2)
    return z ^ _lsr(z, 31)


def uniform(counter: torch.Tensor, key: int) -> torch.Tensor:
    bits = _lsr(splitmix64(counter, key), 11)
    return (bits.to(torch.float64) + 0.5) * (2.0 ** -53)


def _counters(start: int, count: int, device) -> torch.Tensor:
    return torch.arange(start, start + count, dtype=torch.int64, device=device)


def normal(n: int, seed: int, stream: int, device="cpu", start: int = 0) -> torch.Tensor:
    """float64 standard normals for element indices start .. start+n-1."""
    key = stream_key(seed, stream)
    idx = _counters(start, n, device)
    u1 = uniform(2 * idx, key)
    u2 = uniform(2 * idx + 1, key)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos((2.0 * math.pi) * u2)


def to_bf16(v: torch.Tensor) -> torch.Tensor:
    return v.to(torch.float32).to(torch.bfloat16)


def bits(t: torch.Tensor) -> torch.Tensor:
    """The uint16 view (as int16 storage) of a contiguous BF16 tensor."""
    return t.contiguous().reshape(-1).view(torch.int16)


def checksum(t: torch.Tensor) -> int:
    """64-bit FNV-style checksum of a BF16 tensor's bit patterns (for logs)."""
    b = bits(t).to(torch.int64) & 0xFFFF
    w = _counters(0, b.numel(), b.device) * _signed(_GOLDEN) + b
    w = splitmix64(w, 0)
    return int(torch.bitwise_xor(w[::2].sum(), w[1::2].sum() if w.numel() > 1 else 0)) & _M64


# ---------------------------------------------------------------------------
# The workloads
# ---------------------------------------------------------------------------

def gaussian_weight(n: int, seed: int = 0, stream: int = 0, sigma: float = 0.02,
                    device="cpu") -> torch.Tensor:
    """Weight-like N(0, sigma) values."""
    return to_bf16(sigma * normal(n, seed, stream, device))


def kv_layer(seed: int = 2, stream: int = 0, batch: int = 1, heads: int = 8, seq: int = 4096,
             head_dim: int = 128, outliers: int = 4, scale: float = 30.0,
             device="cpu") -> torch.Tensor:
    """One K or V tensor [batch, heads, seq, head_dim] of N(0, 1) with
    ``outliers`` channels per head scaled by ``scale``; the channels of head h
    are the ``outliers`` smallest hash values among d = 0..head_dim-1."""
    n = batch * heads * seq * head_dim
    v = normal(n, seed, stream, device).reshape(batch, heads, seq, head_dim)
    key = stream_key(seed, 1000 + stream)
    for h in range(heads):
        hsh = splitmix64(_counters(h * head_dim, head_dim, "cpu"), key)
        # order by the unsigned hash value
        chans = torch.argsort(hsh ^ (-(1 << 63)), stable=True)[:outliers]
        v[:, h, :, chans.to(device)] *= scale
    return to_bf16(v)


def log_uniform_stress(n: int, seed: int = 3, stream: int = 0, lo_exp: float = -133.0,
                       hi_exp: float = 20.0, p_zero: float = 0.01, p_inf: float = 0.001,
                       device="cpu") -> torch.Tensor:
    """Magnitudes log-uniform over 2**lo_exp .. 2**hi_exp with random sign; a
    fraction p_zero becomes +-0 and p_inf becomes +-inf (independent draws)."""
    key = stream_key(seed, stream)
    idx = _counters(0, n, device)
    u_mag = uniform(4 * idx, key)
    u_sign = uniform(4 * idx + 1, key)
    u_zero = uniform(4 * idx + 2, key)
    u_inf = uniform(4 * idx + 3, key)
    mag = torch.exp2(lo_exp + (hi_exp - lo_exp) * u_mag)
    sign = torch.where(u_sign < 0.5, -1.0, 1.0).to(torch.float64)
    v = sign * mag
    v = torch.where(u_zero < p_zero, sign * 0.0, v)
    v = torch.where(u_inf < p_inf, sign * math.inf, v)
    return to_bf16(v)


def subnormal_gaussian(n: int, seed: int = 3, stream: int = 1, sigma: float = 1e-39,
                       device="cpu") -> torch.Tensor:
    """N(0, sigma) with sigma in the subnormal range: every value is a BF16
    subnormal or zero."""
    return to_bf16(sigma * normal(n, seed, stream, device))


def weight_with_outliers(rows: int = 12288, cols: int = 3072, seed: int = 4, sigma: float = 0.02,
                         p_outlier: float = 0.001, scale: float = 50.0,
                         device="cpu") -> torch.Tensor:
    """A linear weight [rows, cols] of N(0, sigma); each entry independently
    (probability p_outlier) multiplied by ``scale``."""
    n = rows * cols
    v = sigma * normal(n, seed, 0, device)
    u = uniform(_counters(0, n, device), stream_key(seed, 1))
    v = torch.where(u < p_outlier, v * scale, v)
    return to_bf16(v).reshape(rows, cols)


def kv_cache_tensor(layer: int, kv: int, seed: int = 5, heads: int = 8, seq: int = 32768,
                    head_dim: int = 128, sigma: float = 0.02, device="cpu") -> torch.Tensor:
    """One K (kv=0) or V (kv=1) tensor [1, heads, seq, head_dim] of the
    streaming KV cache, N(0, sigma) like the single weight-like tensor."""
    n = heads * seq * head_dim
    return to_bf16(sigma * normal(n, seed, 2 * layer + kv, device)).reshape(1, heads, seq,
                                                                             head_dim)


# Descriptions of the five workloads (sizes as they run).
WORKLOADS = {
    "weight_1m_odd": "single BF16 tensor, n=1,000,003 (odd), N(0,0.02), seed 0",
    "kv_layer_8x4096x128": "K and V [1,8,4096,128] each, N(0,1), 4 outlier channels/head x30, seed 2",
    "stress_16m": "16M log-uniform 2^-133..2^20 (+-0 1%, +-inf 0.1%) and 16M N(0,1e-39), seed 3",
    "linear_weight_12288x3072": "[12288,3072] N(0,0.02), 0.1% entries x50, seed 4",
    "kv_stream_32x2x8x32768x128": "32 layers x (K,V) x [1,8,32768,128] N(0,0.02) = 4 GiB, seed 5",
}
