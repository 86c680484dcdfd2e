"""Counter-based synthetic value generator, bit-identical on CPU and GPU.

This module holds no arithmetic of the denoising method. It only makes
seeded synthetic inputs (weights, token ids, logits, biases) that both the
HIP path and the CPU oracle consume.

Every value is a pure function of (stream key, element index), computed with
integer operations only, so torch on the CPU and torch on the GPU produce the
same bits:

* ``mix32`` is the 32-bit finaliser of MurmurHash3 (Appleby), applied to
  32-bit words held in int64 tensors. Its 32x32-bit multiplies are split into
  16-bit halves so that no intermediate exceeds 2**49.
* An approximately normal value is the sum of the eight bytes of two hashes
  (an Irwin-Hall sum of 8 uniform bytes, mean 1020, variance 8*(256**2-1)/12),
  centred and scaled by one fp32 multiply (correctly rounded on every device),
  then rounded to the storage dtype by torch's round-to-nearest-even.
"""
from __future__ import annotations

import math

import torch

MASK32 = 0xFFFFFFFF
_IH_MEAN = 1020
_IH_STD = math.sqrt(8.0 * (256.0 ** 2 - 1.0) / 12.0)  # 209.0255...
CHUNK = 1 << 26  # elements per generation chunk (bounds temporaries)


def _mul32(h: torch.Tensor, c: int) -> torch.Tensor:
    """(h * c) mod 2**32 for h in [0, 2**32), c a 32-bit constant."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (h * lo + (((h * hi) & 0xFFFF) << 16)) & MASK32


def mix32(h: torch.Tensor) -> torch.Tensor:
    """MurmurHash3 fmix32 on int64 tensors holding 32-bit words."""
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _mix32_int(h: int) -> int:
    h &= MASK32
    h ^= h >> 16
    h = (h * 0x85EBCA6B) & MASK32
    h ^= h >> 13
    h = (h * 0xC2B2AE35) & MASK32
    h ^= h >> 16
    return h


def stream_key(*ids: int) -> tuple[int, int]:
    """Two 32-bit keys derived from a tuple of non-negative stream ids."""
    a, b = 0x3C6EF372, 0xA54FF53A
    for i in ids:
        i = int(i)
        for w in (i & MASK32, (i >> 32) & MASK32):
            a = _mix32_int(a ^ w ^ 0x9E3779B9)
            b = _mix32_int(b + w + 0x7F4A7C15)
    return a, b


def _hash_pair(key: tuple[int, int], idx: torch.Tensor, lane: int) -> torch.Tensor:
    k0, k1 = key
    h = mix32((idx ^ k0) & MASK32)
    h = mix32(h ^ ((k1 + lane * 0x61C88647) & MASK32))
    return h


def u32(key, n: int, device="cpu", lane: int = 0) -> torch.Tensor:
    """n uniform 32-bit words (int64 tensor) for stream ``key``."""
    if n >= (1 << 32):
        raise ValueError("stream too long")
    idx = torch.arange(n, dtype=torch.int64, device=device)
    return _hash_pair(key, idx, lane)


def uniform(key, n: int, device="cpu", lane: int = 0) -> torch.Tensor:
    """n uniform values in [0, 1), 24-bit resolution, float64 (exact)."""
    return (u32(key, n, device, lane) >> 8).to(torch.float64) * (2.0 ** -24)


def randint(key, n: int, low: int, high: int, device="cpu", lane: int = 0) -> torch.Tensor:
    """n integers uniform in [low, high) (int64), exact integer arithmetic."""
    span = high - low
    if not (0 < span < (1 << 30)):
        raise ValueError("bad range")
    w = u32(key, n, device, lane) >> 8  # 24 bits
    return low + ((w * span) >> 24)


def _irwin_hall(h1: torch.Tensor, h2: torch.Tensor) -> torch.Tensor:
    s = torch.zeros_like(h1)
    for h in (h1, h2):
        s = s + (h & 0xFF) + ((h >> 8) & 0xFF) + ((h >> 16) & 0xFF) + ((h >> 24) & 0xFF)
    return s - _IH_MEAN


def normal_(out: torch.Tensor, key, std: float) -> torch.Tensor:
    """Fill ``out`` (any float dtype, any device, contiguous) with ~N(0, std).

    Generated in chunks so that temporaries stay small; the value at flat
    index i depends only on (key, i).
    """
    flat = out.view(-1)
    n = flat.numel()
    scale = torch.tensor(std / _IH_STD, dtype=torch.float32)
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        idx = torch.arange(s, e, dtype=torch.int64, device=out.device)
        h1 = _hash_pair(key, idx, 0)
        h2 = _hash_pair(key, idx, 1)
        v = _irwin_hall(h1, h2).to(torch.float32) * scale.to(out.device)
        flat[s:e] = v.to(out.dtype)
    return out


def normal(key, shape, std: float, dtype=torch.float32, device="cpu") -> torch.Tensor:
    out = torch.empty(shape, dtype=dtype, device=device)
    return normal_(out, key, std)


def permutation(key, n: int) -> torch.Tensor:
    """A seeded permutation of range(n) (CPU int64): argsort of hash words."""
    w = u32(key, n, "cpu")
    return torch.argsort(w * n + torch.arange(n), stable=True)
