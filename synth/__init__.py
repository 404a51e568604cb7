"""Seeded synthetic inputs for the KVarN quantize / decode path.

This module holds none of the method's arithmetic: it only draws K/V values,
queries and page placements.  Both the HIP path and the CPU oracle are fed
the same tensors drawn here.

Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014) keyed by (seed, stream, index),
giving 53-bit uniforms; normals by the Box-Muller transform (cosine branch).
Values depend only on (seed, stream, index), not on the device, chunking or
thread count.  Arithmetic is int64 with two's-complement wrap-around; the
logical right shift is an arithmetic shift followed by a mask.
"""
import math

import torch

_GOLDEN = 0x9E3779B97F4A7C15
_STREAM_MUL = 0xD1B54A32D192ED03
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB

# stream ids
K_STREAM, V_STREAM, Q_STREAM, K_OUT_STREAM, V_OUT_STREAM, PAGE_STREAM = 1, 2, 3, 4, 5, 6
QPAGE_STREAM = 7
ROPE_STREAM, QROPE_STREAM = 8, 9

_CHUNK = 1 << 24


def _s64(x):
    """Reinterpret an unsigned 64-bit constant as a signed int64 value."""
    x &= (1 << 64) - 1
    return x - (1 << 64) if x >= (1 << 63) else x


def _lsr(z, k):
    """Logical right shift of an int64 tensor holding uint64 bits."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix(z):
    z = (z ^ _lsr(z, 30)) * _s64(_M1)
    z = (z ^ _lsr(z, 27)) * _s64(_M2)
    return z ^ _lsr(z, 31)


def _key(seed, stream):
    return _s64(seed * _GOLDEN + stream * _STREAM_MUL)


def raw_u64(seed, stream, idx):
    """SplitMix64 output (as int64 bits) for integer counter tensor idx."""
    return _mix(idx * _s64(_GOLDEN) + _key(seed, stream) + _s64(_GOLDEN))


def uniform(seed, stream, n, offset=0, device="cpu"):
    """n uniforms in [0, 1) (float64) at counters offset .. offset+n-1."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        idx = torch.arange(offset + s, offset + e, dtype=torch.int64, device=device)
        out[s:e] = _lsr(raw_u64(seed, stream, idx), 11).to(torch.float64) * (2.0 ** -53)
    return out


def normal(seed, stream, n, offset=0, device="cpu"):
    """n standard normals (float64); normal i uses uniforms 2i and 2i+1."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        i = torch.arange(offset + s, offset + e, dtype=torch.int64, device=device)
        u1 = _lsr(raw_u64(seed, stream, 2 * i), 11).to(torch.float64) * (2.0 ** -53)
        u2 = _lsr(raw_u64(seed, stream, 2 * i + 1), 11).to(torch.float64) * (2.0 ** -53)
        out[s:e] = torch.sqrt(-2.0 * torch.log1p(-u1)) * torch.cos((2.0 * math.pi) * u2)
    return out


def student_t3(seed, stream, n, offset=0, device="cpu"):
    """n Student-t(3) draws: z0 / sqrt((z1^2 + z2^2 + z3^2) / 3), four normals each."""
    out = torch.empty(n, dtype=torch.float64, device=device)
    for s in range(0, n, _CHUNK // 4):
        e = min(n, s + _CHUNK // 4)
        z = normal(seed, stream, 4 * (e - s), 4 * (offset + s), device).view(-1, 4)
        out[s:e] = z[:, 0] / torch.sqrt((z[:, 1:] ** 2).sum(1) / 3.0)
    return out


def to_f16(x):
    """float64 -> float16 (round to nearest even), clamped to +-65504."""
    return x.clamp(-65504.0, 65504.0).to(torch.float16)


def permutation(seed, stream, n, device="cpu"):
    """A seeded permutation of range(n): the order of n SplitMix64 draws."""
    keys = raw_u64(seed, stream, torch.arange(n, dtype=torch.int64, device=device))
    return torch.argsort(keys, stable=True).to(torch.int32)


def choose(seed, stream, n, k, device="cpu"):
    """k distinct indices out of range(n), sorted."""
    return torch.sort(permutation(seed, stream, n, device)[:k].to(torch.int64)).values
