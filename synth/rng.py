"""Counter-based random bits for the seeded synthetic inputs.

Every value is a pure function of (key, index): the SplitMix64 output
function (Steele, Lea & Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014) applied to ``key + (index + 1) * 0x9E3779B97F4A7C15``.
It is evaluated with torch int64 tensor arithmetic (wrapping multiply,
masked shifts), so the same bits come out on the CPU and on the GPU and a
stack of many gigabytes can be filled in place on the device in chunks.

This module holds no arithmetic of the MoE layer itself: it only draws bits.
"""
from __future__ import annotations

import torch

_MASK64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit integer as a signed one (torch int64)."""
    v &= _MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (exact, used for keys and tests)."""
    z &= _MASK64
    z = ((z ^ (z >> 30)) * _M1) & _MASK64
    z = ((z ^ (z >> 27)) * _M2) & _MASK64
    return z ^ (z >> 31)


def derive_key(*ids: int) -> int:
    """Fold a sequence of integers (seed, layer, tensor id, ...) into one 64-bit key."""
    k = 0x243F6A8885A308D3  # arbitrary non-zero start (hex digits of pi)
    for i in ids:
        k = mix64_int(k ^ mix64_int((i & _MASK64) + _GAMMA))
    return k


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor viewed as uint64."""
    return (z >> s) & ((1 << (64 - s)) - 1)


def _mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


_CHUNK = 1 << 24  # words per generation chunk (128 MiB of int64)


def hash_words(key: int, start: int, n: int, device) -> torch.Tensor:
    """int64 tensor of the n words with indices start .. start+n-1 under `key`."""
    idx = torch.arange(start + 1, start + n + 1, dtype=torch.int64, device=device)
    z = idx * _s64(_GAMMA) + _s64(key)
    return _mix64(z)


def fill_bytes(out: torch.Tensor, key: int) -> torch.Tensor:
    """Fill a contiguous uint8 tensor with the byte stream of `key` (little-endian words)."""
    assert out.dtype == torch.uint8 and out.is_contiguous()
    flat = out.view(-1)
    nbytes = flat.numel()
    nwords = (nbytes + 7) // 8
    pos = 0
    while pos < nwords:
        n = min(_CHUNK, nwords - pos)
        w = hash_words(key, pos, n, out.device)
        b = w.view(torch.uint8)
        lo = pos * 8
        hi = min(nbytes, lo + n * 8)
        flat[lo:hi].copy_(b[: hi - lo])
        pos += n
    return out


def uniform01(key: int, n: int, device) -> torch.Tensor:
    """n float64 values uniform on [0, 1): the top 53 bits of each word times 2^-53."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    pos = 0
    while pos < n:
        m = min(_CHUNK, n - pos)
        w = hash_words(key, pos, m, device)
        out[pos:pos + m] = _lsr(w, 11).to(torch.float64) * (2.0 ** -53)
        pos += m
    return out


def normal(key: int, n: int, device) -> torch.Tensor:
    """n float64 standard normals by the Box-Muller transform (cosine branch).

    Value i uses words 2i and 2i+1 of the stream: u1 = (top 53 bits + 0.5) * 2^-53
    lies in (0, 1), so the logarithm is finite."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    pos = 0
    while pos < n:
        m = min(_CHUNK // 2, n - pos)
        w = hash_words(key, 2 * pos, 2 * m, device).view(m, 2)
        u1 = (_lsr(w[:, 0], 11).to(torch.float64) + 0.5) * (2.0 ** -53)
        u2 = _lsr(w[:, 1], 11).to(torch.float64) * (2.0 ** -53)
        out[pos:pos + m] = torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * torch.pi * u2)
        pos += m
    return out


def permutation(key: int, n: int, device) -> torch.Tensor:
    """A seeded permutation of 0..n-1 (argsort of n hash words; ties have probability ~n^2/2^64)."""
    w = hash_words(key, 0, n, device)
    return torch.argsort(w, stable=True)
